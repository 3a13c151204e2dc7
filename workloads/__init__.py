"""Seeded synthetic inputs for MLA paged latent decode.

This module only builds inputs: random numbers, their rounding to the storage
formats (bf16 and OCP fp8 e4m3fn, done by torch's CPU casts), page tables and
sequence lengths.  It holds none of the attention arithmetic, so both the
float64 oracle and the GPU path can take their inputs from here without
sharing any part of the computation.

Cache layout (Triton MLA page, "data flow" section): one pool of pages of
shape ``[num_blocks, page_size, head_size]`` where each row is the single
latent vector ``[kv_c (kv_lora_rank) | k_pe (rope 64)]``; ``block_table[b, j]``
names the physical page that holds logical block ``j`` of sequence ``b``
(lshu.cn article, section 11).

The five workloads below are the decode shapes this library is measured and
checked on.  Every array is built from ``numpy.random.default_rng(seed)``
with a fixed draw order (seq_lens, page permutation, q, pool), so a seed
always gives identical bytes.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np

BF16 = "bf16"
FP8_E4M3 = "fp8_e4m3"
# per-token quantised fp8: each row [e4m3fn codes (D) | fp32 scale | 12 zero
# bytes], scale = max|row| / 448 of the token's fp32 row
FP8_PER_TOKEN = "fp8_per_token"
INT8_PER_TOKEN = "int8_per_token"
INT4_PER_TOKEN = "int4_per_token"
PER_TOKEN_PAD = 16

# fp32(192 ** -0.5): the softmax scale of a DeepSeek-V3 style head
# (qk_nope 128 + qk_rope 64).  Kept as the fp32-rounded value.
DSV3_SCALE = float(np.float32(192.0 ** -0.5))


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    batch: int
    num_heads: int
    head_size: int          # D_qk = kv_lora_rank + 64
    kv_lora_rank: int       # D_v
    page_size: int
    num_blocks: int
    kv_dtype: str           # BF16, FP8_E4M3, FP8_PER_TOKEN or INT8_PER_TOKEN
    k_scale: float
    scale: float
    seq_lens_fixed: Optional[Sequence[int]] = None
    seq_len_range: Optional[tuple] = None   # inclusive (lo, hi), uniform draw
    seq_len_head: Optional[Sequence[int]] = None  # fixed leading lengths, rest drawn
    parity_splits: Sequence[int] = (1,)
    description: str = ""
    # query tokens per sequence (multi-token decode: the last q_len positions
    # are verified at once; q is then [B, q_len, H, D])
    q_len: int = 1
    # sparse decode: each sequence attends to min(topk, n) positions drawn at
    # random (distinct, unsorted); 0 = dense
    topk: int = 0

    def draw_seq_lens(self, rng: np.random.Generator) -> np.ndarray:
        if self.seq_lens_fixed is not None:
            return np.asarray(self.seq_lens_fixed, dtype=np.int32)
        head = list(self.seq_len_head or [])
        lo, hi = self.seq_len_range
        rest = rng.integers(lo, hi, size=self.batch - len(head), endpoint=True)
        return np.concatenate([np.asarray(head, np.int64), rest]).astype(np.int32)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in [
        Workload(
            name="tiny", seed=1, batch=2, num_heads=16, head_size=576, kv_lora_rank=512,
            page_size=16, num_blocks=16, kv_dtype=BF16, k_scale=1.0, scale=DSV3_SCALE,
            seq_lens_fixed=(37, 100), parity_splits=(1, 4),
            description="B=2 H=16 D=576 bf16, page 16, 16 pages, seq_lens {37,100}"),
        Workload(
            name="dsv3", seed=2, batch=64, num_heads=128, head_size=576, kv_lora_rank=512,
            page_size=64, num_blocks=8192, kv_dtype=BF16, k_scale=1.0, scale=DSV3_SCALE,
            seq_len_range=(1024, 8192), parity_splits=(16, 1),
            description="B=64 H=128 D=576/512 bf16, page 64, 8192 pages, seq_lens U[1024,8192]"),
        Workload(
            name="skewed", seed=3, batch=8, num_heads=128, head_size=576, kv_lora_rank=512,
            page_size=64, num_blocks=4096, kv_dtype=BF16, k_scale=1.0, scale=DSV3_SCALE,
            seq_len_head=(131072,), seq_len_range=(512, 4096), parity_splits=(256, 1),
            description="B=8 H=128 D=576 bf16, seq_lens {131072, 7 x U[512,4096]}, page 64"),
        Workload(
            name="h320", seed=4, batch=256, num_heads=16, head_size=320, kv_lora_rank=256,
            page_size=16, num_blocks=65536, kv_dtype=BF16, k_scale=1.0, scale=DSV3_SCALE,
            seq_len_range=(256, 4096), parity_splits=(8, 1),
            description="B=256 H=16 D=320/256 bf16, page 16, seq_lens U[256,4096]"),
        Workload(
            name="fp8", seed=5, batch=128, num_heads=128, head_size=576, kv_lora_rank=512,
            page_size=64, num_blocks=16384, kv_dtype=FP8_E4M3, k_scale=float(np.float32(0.05)),
            scale=DSV3_SCALE, seq_len_range=(2048, 8192), parity_splits=(16, 1),
            description="B=128 H=128 D=576 fp8 e4m3 cache (k_scale 0.05), page 64, U[2048,8192]"),
        Workload(
            name="dsv3_mtp2", seed=6, batch=64, num_heads=128, head_size=576, kv_lora_rank=512,
            page_size=64, num_blocks=8192, kv_dtype=BF16, k_scale=1.0, scale=DSV3_SCALE,
            seq_len_range=(1024, 8192), parity_splits=(16, 1), q_len=2,
            description="B=64 q_len=2 H=128 D=576/512 bf16 multi-token decode, page 64, "
                        "8192 pages, seq_lens U[1024,8192]"),
        Workload(
            name="dsv3_sparse", seed=7, batch=64, num_heads=128, head_size=576,
            kv_lora_rank=512, page_size=64, num_blocks=8192, kv_dtype=BF16, k_scale=1.0,
            scale=DSV3_SCALE, seq_len_range=(2048, 8192), parity_splits=(4, 1), topk=2048,
            description="B=64 H=128 D=576/512 bf16 sparse decode over top-2048 positions, "
                        "page 64, 8192 pages, seq_lens U[2048,8192]"),
        Workload(
            name="fp8_pt", seed=8, batch=64, num_heads=128, head_size=576, kv_lora_rank=512,
            page_size=64, num_blocks=8192, kv_dtype=FP8_PER_TOKEN, k_scale=1.0,
            scale=DSV3_SCALE, seq_len_range=(1024, 8192), parity_splits=(16, 1),
            description="B=64 H=128 D=576/512 per-token fp8 cache (inline fp32 scale, rows of "
                        "592 B), page 64, 8192 pages, seq_lens U[1024,8192]"),
        Workload(
            name="int8_pt", seed=9, batch=64, num_heads=128, head_size=576, kv_lora_rank=512,
            page_size=64, num_blocks=8192, kv_dtype=INT8_PER_TOKEN, k_scale=1.0,
            scale=DSV3_SCALE, seq_len_range=(1024, 8192), parity_splits=(16, 1),
            description="B=64 H=128 D=576/512 per-token int8 cache (inline fp32 scale, rows of "
                        "592 B), page 64, 8192 pages, seq_lens U[1024,8192]"),
        Workload(
            name="int4_pt", seed=10, batch=64, num_heads=128, head_size=576, kv_lora_rank=512,
            page_size=64, num_blocks=8192, kv_dtype=INT4_PER_TOKEN, k_scale=1.0,
            scale=DSV3_SCALE, seq_len_range=(1024, 8192), parity_splits=(16, 1),
            description="B=64 H=128 D=576/512 per-token int4 cache (two codes per byte, inline "
                        "fp32 scale, rows of 304 B), page 64, 8192 pages, seq_lens U[1024,8192]"),
    ]
}


@dataclasses.dataclass
class DecodeInputs:
    """One decode batch, every array in its storage format (raw bits)."""
    workload: Workload
    q_bits: np.ndarray          # uint16 [B, H, D] or [B, q_len, H, D] (bf16 bits)
    kv_bits: np.ndarray         # uint16 [NB, P, D] (bf16) or uint8 [NB, P, D] (fp8)
    block_table: np.ndarray     # int32 [B, max_blocks_per_seq]
    seq_lens: np.ndarray        # int32 [B]
    topk_indices: Optional[np.ndarray] = None  # int32 [B, topk] logical positions (sparse)
    topk_lens: Optional[np.ndarray] = None     # int32 [B] entries used per sequence

    @property
    def kv_dtype(self) -> str:
        return self.workload.kv_dtype


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round-to-nearest-even, via torch's CPU cast)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def f32_to_e4m3fn_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to OCP fp8 e4m3fn (RNE), saturating to +-448 first."""
    import torch
    x = np.clip(np.ascontiguousarray(x, dtype=np.float32), -448.0, 448.0)
    t = torch.from_numpy(x).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def per_token_fp8_rows(pool: np.ndarray) -> np.ndarray:
    """fp32 rows [..., D] -> per-token quantised rows [..., D + 16] bytes:
    e4m3fn codes of row / s, then s as fp32, then zeros, with
    s = fp32(max|row| / 448) (1 for an all-zero row)."""
    amax = np.abs(pool).max(axis=-1, keepdims=True).astype(np.float32)
    s = np.where(amax > 0, amax / np.float32(448.0), np.float32(1.0)).astype(np.float32)
    codes = f32_to_e4m3fn_bits(pool / s)
    out = np.zeros(pool.shape[:-1] + (pool.shape[-1] + PER_TOKEN_PAD,), dtype=np.uint8)
    out[..., :pool.shape[-1]] = codes
    out[..., pool.shape[-1]:pool.shape[-1] + 4] = s.view(np.uint8)
    return out


def per_token_int8_rows(pool: np.ndarray) -> np.ndarray:
    """fp32 rows [..., D] -> per-token quantised rows [..., D + 16] bytes:
    int8 codes round(row / s) (symmetric, in [-127, 127]), then s as fp32,
    then zeros, with s = fp32(max|row| / 127) (1 for an all-zero row)."""
    amax = np.abs(pool).max(axis=-1, keepdims=True).astype(np.float32)
    s = np.where(amax > 0, amax / np.float32(127.0), np.float32(1.0)).astype(np.float32)
    codes = np.clip(np.rint(pool / s), -127, 127).astype(np.int8)
    out = np.zeros(pool.shape[:-1] + (pool.shape[-1] + PER_TOKEN_PAD,), dtype=np.uint8)
    out[..., :pool.shape[-1]] = codes.view(np.uint8)
    out[..., pool.shape[-1]:pool.shape[-1] + 4] = s.view(np.uint8)
    return out


def per_token_int4_rows(pool: np.ndarray) -> np.ndarray:
    """fp32 rows [..., D] -> per-token quantised rows [..., D/2 + 16] bytes:
    4-bit codes round(row / s) in [-7, 7], two per byte (element 2i in the low
    nibble), then s as fp32, then zeros, with s = fp32(max|row| / 7) (1 for an
    all-zero row)."""
    amax = np.abs(pool).max(axis=-1, keepdims=True).astype(np.float32)
    s = np.where(amax > 0, amax / np.float32(7.0), np.float32(1.0)).astype(np.float32)
    codes = np.clip(np.rint(pool / s), -7, 7).astype(np.int16) & 0x0F
    D = pool.shape[-1]
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    out = np.zeros(pool.shape[:-1] + (D // 2 + PER_TOKEN_PAD,), dtype=np.uint8)
    out[..., :D // 2] = packed
    out[..., D // 2:D // 2 + 4] = s.view(np.uint8)
    return out


def make_block_table(rng: np.random.Generator, seq_lens: np.ndarray, page_size: int,
                     num_blocks: int) -> np.ndarray:
    """Each sequence takes the next ceil(n/P) pages of one seeded permutation
    of the pool; unused entries are 0."""
    pages_per_seq = [(int(n) + page_size - 1) // page_size for n in seq_lens]
    need = sum(pages_per_seq)
    if need > num_blocks:
        raise ValueError(f"pool of {num_blocks} pages cannot hold {need} pages")
    perm = rng.permutation(num_blocks).astype(np.int32)
    width = max(1, max(pages_per_seq) if pages_per_seq else 1)
    table = np.zeros((len(seq_lens), width), dtype=np.int32)
    at = 0
    for b, k in enumerate(pages_per_seq):
        table[b, :k] = perm[at:at + k]
        at += k
    return table


def _normal_f32(rng: np.random.Generator, shape, chunk: int = 1 << 24) -> np.ndarray:
    out = np.empty(int(np.prod(shape)), dtype=np.float32)
    for s in range(0, out.size, chunk):
        e = min(out.size, s + chunk)
        out[s:e] = rng.standard_normal(e - s, dtype=np.float32)
    return out.reshape(shape)


def generate(workload: Workload | str, *, seq_lens: Optional[Sequence[int]] = None,
             batch: Optional[int] = None, num_blocks: Optional[int] = None) -> DecodeInputs:
    """Build the seeded inputs of a workload.

    ``seq_lens``/``batch``/``num_blocks`` override the workload (used for
    edge cases); the seed and the draw order stay the same.
    """
    w = WORKLOADS[workload] if isinstance(workload, str) else workload
    rng = np.random.default_rng(w.seed)
    if seq_lens is not None:
        sl = np.asarray(seq_lens, dtype=np.int32)
    else:
        sl = w.draw_seq_lens(rng)
    if batch is not None:
        sl = sl[:batch]
    nb = num_blocks if num_blocks is not None else w.num_blocks
    table = make_block_table(rng, sl, w.page_size, nb)
    B = len(sl)
    qshape = (B, w.num_heads, w.head_size) if w.q_len == 1 else (B, w.q_len, w.num_heads,
                                                                  w.head_size)
    q = _normal_f32(rng, qshape)
    q_bits = f32_to_bf16_bits(q)
    pool = _normal_f32(rng, (nb, w.page_size, w.head_size))
    if w.kv_dtype == BF16:
        kv_bits = f32_to_bf16_bits(pool)
    elif w.kv_dtype == FP8_PER_TOKEN:
        kv_bits = per_token_fp8_rows(pool)
    elif w.kv_dtype == INT8_PER_TOKEN:
        kv_bits = per_token_int8_rows(pool)
    elif w.kv_dtype == INT4_PER_TOKEN:
        kv_bits = per_token_int4_rows(pool)
    else:
        kv_bits = f32_to_e4m3fn_bits(pool / np.float32(w.k_scale))
    inp = DecodeInputs(workload=w, q_bits=q_bits, kv_bits=kv_bits, block_table=table,
                       seq_lens=sl)
    if w.topk:
        idx = np.zeros((B, w.topk), dtype=np.int32)
        lens = np.zeros(B, dtype=np.int32)
        for b in range(B):
            k = min(w.topk, int(sl[b]))
            idx[b, :k] = rng.choice(int(sl[b]), size=k, replace=False)
            lens[b] = k
        inp.topk_indices, inp.topk_lens = idx, lens
    return inp


def small_case(*, seed: int, batch: int, num_heads: int, head_size: int, kv_lora_rank: int,
               page_size: int, seq_lens: Sequence[int], kv_dtype: str = BF16,
               k_scale: float = 1.0, extra_pages: int = 3, scale: float = DSV3_SCALE,
               table_pad: int = 0, q_len: int = 1, topk: int = 0) -> DecodeInputs:
    """A custom small batch (edge cases, ragged lengths) with the same recipe."""
    pages = sum((int(n) + page_size - 1) // page_size for n in seq_lens) + extra_pages
    w = Workload(name=f"case{seed}", seed=seed, batch=batch, num_heads=num_heads,
                 head_size=head_size, kv_lora_rank=kv_lora_rank, page_size=page_size,
                 num_blocks=max(1, pages), kv_dtype=kv_dtype, k_scale=k_scale, scale=scale,
                 seq_lens_fixed=tuple(int(n) for n in seq_lens), q_len=q_len, topk=topk)
    inp = generate(w)
    if table_pad:
        inp.block_table = np.pad(inp.block_table, ((0, 0), (0, table_pad)))
    return inp


# ---------------------------------------------------------------- input transforms
# These rearrange or poison inputs without touching values that are read.

def referenced_slots(inp: DecodeInputs) -> np.ndarray:
    """Boolean mask [NB, P]: True where a (page, slot) holds a token some
    sequence reads."""
    P = inp.workload.page_size
    used = np.zeros(inp.kv_bits.shape[:2], dtype=bool)
    for b, n in enumerate(inp.seq_lens):
        n = int(n)
        for j in range((n + P - 1) // P):
            k = min(P, n - j * P)
            used[inp.block_table[b, j], :k] = True
    return used


def poison_unreferenced(inp: DecodeInputs, *, poison_table: bool = True) -> DecodeInputs:
    """Fill every unreferenced page row (including the tail slots of each
    sequence's last page) with NaN, and point unused block_table entries at a
    fully poisoned page when one exists."""
    used = referenced_slots(inp)
    kv = inp.kv_bits.copy()
    nan = np.uint16(0x7FC0) if inp.kv_dtype == BF16 else np.uint8(0x7F)
    # per-token rows get bytes 0x7F: NaN fp8 codes, int8 code 127 or int4 codes (-1, 7), and
    # a scale of about 3.4e38, so that any read of them wrecks the result
    kv[~used] = nan
    table = inp.block_table.copy()
    if poison_table:
        free_pages = np.nonzero(~used.any(axis=1))[0]
        if free_pages.size:
            P = inp.workload.page_size
            for b, n in enumerate(inp.seq_lens):
                k = (int(n) + P - 1) // P
                table[b, k:] = free_pages[0]
    return dataclasses.replace(inp, kv_bits=kv, block_table=table)


def permute_pages(inp: DecodeInputs, seed: int) -> DecodeInputs:
    """Move every physical page to a new seeded position and remap the
    block table so that each sequence still sees the same rows."""
    rng = np.random.default_rng(seed)
    nb = inp.kv_bits.shape[0]
    new_of_old = rng.permutation(nb).astype(np.int32)
    kv = np.empty_like(inp.kv_bits)
    kv[new_of_old] = inp.kv_bits
    table = new_of_old[inp.block_table]
    return dataclasses.replace(inp, kv_bits=kv, block_table=table.astype(np.int32))


def shard_pages(inp: DecodeInputs, shards: int, rank: int) -> DecodeInputs:
    """The same pool as seen by one of ``shards`` context shards: rank r owns
    every sequence's logical pages j with j % shards == r (round robin).  Its
    block table lists those pages in order and its sequence length counts
    their positions (a sequence's last, possibly partial, page stays last).
    The pool itself is shared, so no value moves."""
    P = inp.workload.page_size
    B = len(inp.seq_lens)
    tables, lens = [], []
    for b in range(B):
        n = int(inp.seq_lens[b])
        pages = (n + P - 1) // P
        mine = list(range(rank, pages, shards))
        tables.append([int(inp.block_table[b, j]) for j in mine])
        lens.append(sum(min(P, n - j * P) for j in mine))
    width = max(1, max(len(t) for t in tables))
    table = np.zeros((B, width), dtype=np.int32)
    for b, t in enumerate(tables):
        table[b, :len(t)] = t
    return dataclasses.replace(inp, block_table=table, seq_lens=np.asarray(lens, dtype=np.int32))


def subset(inp: DecodeInputs, batches: Sequence[int]) -> DecodeInputs:
    """The same pool with only the chosen sequences, in the given order."""
    idx = np.asarray(batches, dtype=np.int64)
    return dataclasses.replace(inp, q_bits=inp.q_bits[idx].copy(),
                               block_table=inp.block_table[idx].copy(),
                               seq_lens=inp.seq_lens[idx].copy())


def expected_tokens(w: Workload) -> float:
    """Expected total context tokens of a workload (mean of its length draw)."""
    if w.seq_lens_fixed is not None:
        return float(sum(w.seq_lens_fixed))
    head = list(w.seq_len_head or [])
    lo, hi = w.seq_len_range
    return float(sum(head) + (w.batch - len(head)) * (lo + hi) / 2.0)


__all__ = [
    "BF16", "FP8_E4M3", "DSV3_SCALE", "Workload", "WORKLOADS", "DecodeInputs", "generate",
    "small_case", "f32_to_bf16_bits", "f32_to_e4m3fn_bits", "make_block_table",
    "referenced_slots", "poison_unreferenced", "permute_pages", "subset", "expected_tokens",
    "shard_pages",
]
