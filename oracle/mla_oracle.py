"""Float64 CPU oracle for MLA paged latent decode.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this module.  The library's GPU path
never calls it and shares no code with it: this file reads raw storage bits
and decodes them itself, with plain numpy float64 arithmetic, so that a reader
can check every step against the pages by eye.

What it computes (decode attention of one latent query per head):

* The cache row of a token is the single vector ``[kv_c | k_pe]``; during
  decode all H query heads read it as a one-head K (MQA), and V is its first
  ``kv_lora_rank`` columns  (Triton MLA page, "data flow": the cache is passed
  as a single-head K cache and its ``[..., :kv_lora_rank]`` slice as V).
* A token's row is found through the page table: logical block = pos // P,
  physical block = block_table[req][logical block], physical slot =
  physical block * P + pos % P  (lshu.cn article, section 11).
* A decode query sits at the end of its sequence, so it sees every key: no
  mask  (lshu.cn article, section 9).
* Scores are scaled by the softmax scale, the result is the softmax-weighted
  sum of V, and the log-sum-exp is returned in natural log (Triton MLA page,
  "design motivation": lse is always returned and ``lse_base_on_e`` defaults
  to True; AttentionBackend page, "limits": ln versus log2 matters for the
  cross-shard merge).
* For an fp8 cache one per-layer scale multiplies both K and V
  (Triton MLA page, data flow: ``k_scale = v_scale = layer._k_scale``); for a
  bf16 cache it has no effect (same listing's comment on the fp8 check).
* A per-token-head cache (Triton MLA page, key files: fp8, int8 and int4
  modes whose rows are padded to hold an inline scale) stores each token's
  codes followed by its float32 scale; the token's K and V are code * scale.

The online softmax (lshu.cn article, section 7) and the split-KV merge
(section 12) are exact rewrites of this plain softmax, so ``decode`` is the
plain definition written out, and ``decode_split`` follows section 12 to merge
per-segment partials (used only to pin the merge algebra).
"""
from __future__ import annotations

import math
from typing import Callable, List, Optional, Sequence, Tuple

import numpy as np

ROPE_DIM = 64


# ---------------------------------------------------------------- storage formats

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 is the top half of an IEEE binary32: widen and reinterpret."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def _e4m3fn_table() -> np.ndarray:
    """Value of every OCP fp8 e4m3fn code: 1 sign, 4 exponent (bias 7),
    3 mantissa bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN;
    there is no infinity."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = s * (m / 8.0) * 2.0 ** (-6)
        else:
            vals[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3FN_VALUES = _e4m3fn_table()


def e4m3fn_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return E4M3FN_VALUES[np.asarray(bits, dtype=np.uint8)]


PER_TOKEN_PAD = 16  # bytes after the codes of a per-token row: fp32 scale + 12 unused
PER_TOKEN_DTYPES = ("fp8_per_token", "int8_per_token", "int4_per_token")


def int8_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Two's-complement signed bytes."""
    return np.asarray(bits, dtype=np.uint8).view(np.int8).astype(np.float64)


def int4_bits_to_f64(packed: np.ndarray) -> np.ndarray:
    """Two signed 4-bit codes per byte, element 2i in the low nibble of byte
    i and element 2i+1 in the high nibble (two's complement, -8..7)."""
    b = np.asarray(packed, dtype=np.uint8)
    lo = (b & 0x0F).astype(np.int16)
    hi = (b >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), dtype=np.float64)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def code_bytes(kv_dtype: str, head_size: int) -> int:
    """Bytes of codes in a per-token row (int4 packs two codes per byte)."""
    return head_size // 2 if kv_dtype == "int4_per_token" else head_size


def row_width(kv_dtype: str, head_size: int) -> int:
    """Stored elements (bytes for the 1-byte and packed formats) per cache
    row: the head_size values, and for the per-token layouts the padding that
    holds the inline scale (Triton MLA page, key files: in the per-token-head
    modes, fp8, int8 and int4 among them, the cache shape pads head_dim to
    hold an inline scale)."""
    if kv_dtype in PER_TOKEN_DTYPES:
        return code_bytes(kv_dtype, head_size) + PER_TOKEN_PAD
    return head_size


def decode_kv(kv_bits: np.ndarray, kv_dtype: str, k_scale: float) -> np.ndarray:
    """Cache rows as float64.  fp8 values are multiplied by the fp32-rounded
    k_scale (exact in float64); bf16 rows ignore k_scale.  Per-token rows
    ``[codes (D) | fp32 scale | pad]``, codes e4m3fn or signed int8, decode
    to code * scale of that token (exact in float64); k_scale does not apply
    to them."""
    if kv_dtype == "bf16":
        return bf16_bits_to_f64(kv_bits)
    if kv_dtype == "fp8_e4m3":
        return e4m3fn_bits_to_f64(kv_bits) * float(np.float32(k_scale))
    if kv_dtype in PER_TOKEN_DTYPES:
        rows = np.ascontiguousarray(kv_bits, dtype=np.uint8)
        nb = rows.shape[-1] - PER_TOKEN_PAD  # code bytes
        scale = rows[..., nb:nb + 4].copy().view("<f4")[..., 0].astype(np.float64)
        decode = {"fp8_per_token": e4m3fn_bits_to_f64, "int8_per_token": int8_bits_to_f64,
                  "int4_per_token": int4_bits_to_f64}[kv_dtype]
        return decode(rows[..., :nb]) * scale[..., None]
    raise ValueError(f"unknown kv dtype {kv_dtype!r}")


# ---------------------------------------------------------------- paged addressing

def physical_slot(block_table_row: np.ndarray, pos: int, block_size: int) -> int:
    """lshu.cn article, section 11: logical block, then the table lookup, then
    block * block_size + pos % block_size."""
    logical_block = pos // block_size
    physical_block = int(block_table_row[logical_block])
    return physical_block * block_size + pos % block_size


def gather_rows(kv_rows: np.ndarray, block_table_row: np.ndarray, n: int,
                block_size: int) -> np.ndarray:
    """Rows of positions 0..n-1 of one sequence, read through its table.
    ``kv_rows`` is the pool flattened to [num_blocks * block_size, D] (raw
    bits or decoded values)."""
    slots = [physical_slot(block_table_row, t, block_size) for t in range(n)]
    return kv_rows[np.asarray(slots, dtype=np.int64)] if n else kv_rows[:0]


# ---------------------------------------------------------------- the definition

def attend(q: np.ndarray, K: np.ndarray, d_v: int, scale: float
           ) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of the H query rows q [H, D] over the n keys K [n, D]
    with V = K[:, :d_v].  Returns o [H, d_v] and natural-log lse [H].

    n == 0 gives o = 0 and lse = -inf (the empty sum)."""
    H = q.shape[0]
    n = K.shape[0]
    if n == 0:
        return np.zeros((H, d_v)), np.full(H, -np.inf)
    s = (q @ K.T) * scale                       # [H, n] scores
    m = s.max(axis=1, keepdims=True)            # row max, for a safe exp
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    lse = (m + np.log(z))[:, 0]                 # ln sum_t exp(s_t)
    p = np.exp(s - lse[:, None])                # softmax weights
    o = p @ K[:, :d_v]
    return o, lse


def decode(q_bits: np.ndarray, kv_bits: np.ndarray, block_table: np.ndarray,
           seq_lens: np.ndarray, *, scale: float, k_scale: float, kv_dtype: str,
           kv_lora_rank: int, batches: Optional[Sequence[int]] = None
           ) -> Tuple[np.ndarray, np.ndarray]:
    """MLA latent decode of a batch.

    q_bits [B, H, D] bf16 bits; kv_bits [NB, P, D] (bf16 or fp8 bits);
    block_table [B, W] int32; seq_lens [B].  ``scale`` is used as its fp32
    value.  Returns o [B', H, kv_lora_rank] and lse [B', H] in float64 for
    the chosen ``batches`` (default: all, in order)."""
    B, H, D = q_bits.shape
    NB, P, D2 = kv_bits.shape
    if D2 != row_width(kv_dtype, D):
        raise ValueError("q and cache head sizes differ")
    bits = kv_bits.reshape(NB * P, D2)
    sc = float(np.float32(scale))
    idx = range(B) if batches is None else batches
    outs, lses = [], []
    for b in idx:
        q = bf16_bits_to_f64(q_bits[b])
        # gather the sequence's rows as stored, then decode only those
        K = decode_kv(gather_rows(bits, block_table[b], int(seq_lens[b]), P), kv_dtype, k_scale)
        o, lse = attend(q, K, kv_lora_rank, sc)
        outs.append(o)
        lses.append(lse)
    return np.stack(outs), np.stack(lses)


# ---------------------------------------------------------------- multi-token decode

def visible_keys(n: int, q_len: int, i: int) -> int:
    """lshu.cn article, section 10 (verifying several new positions at once):
    the sequence length n counts every key, the q_len new positions included,
    so the context before them is n - q_len; query token i sits at absolute
    position n - q_len + i and sees the keys at positions up to and including
    it, i.e. the first n - q_len + i + 1 of them (none if that is < 1)."""
    return max(0, min(n, n - q_len + i + 1))


def decode_mtp(q_bits: np.ndarray, kv_bits: np.ndarray, block_table: np.ndarray,
               seq_lens: np.ndarray, *, scale: float, k_scale: float, kv_dtype: str,
               kv_lora_rank: int, batches: Optional[Sequence[int]] = None
               ) -> Tuple[np.ndarray, np.ndarray]:
    """Multi-token MLA decode: q_bits [B, q_len, H, D] bf16 bits.  Query token
    i of sequence b attends to the first visible_keys(n_b, q_len, i) rows of
    its cache (section 10's rectangle plus lower triangle), each exactly as in
    ``decode``.  Returns o [B', q_len, H, kv_lora_rank] and lse [B', q_len, H]."""
    B, q_len, H, D = q_bits.shape
    NB, P, D2 = kv_bits.shape
    if D2 != row_width(kv_dtype, D):
        raise ValueError("q and cache head sizes differ")
    bits = kv_bits.reshape(NB * P, D2)
    sc = float(np.float32(scale))
    idx = range(B) if batches is None else batches
    outs, lses = [], []
    for b in idx:
        n = int(seq_lens[b])
        K = decode_kv(gather_rows(bits, block_table[b], n, P), kv_dtype, k_scale)
        ob, lb = [], []
        for i in range(q_len):
            o, lse = attend(bf16_bits_to_f64(q_bits[b, i]), K[:visible_keys(n, q_len, i)],
                            kv_lora_rank, sc)
            ob.append(o)
            lb.append(lse)
        outs.append(np.stack(ob))
        lses.append(np.stack(lb))
    return np.stack(outs), np.stack(lses)


# ---------------------------------------------------------------- sparse decode

def decode_sparse(q_bits: np.ndarray, kv_bits: np.ndarray, block_table: np.ndarray,
                  topk_indices: np.ndarray, topk_lens: np.ndarray, *, scale: float,
                  k_scale: float, kv_dtype: str, kv_lora_rank: int,
                  batches: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """lshu.cn article, section 13 (dense versus sparse attention): each query
    attends only to a selected list of its positions (e.g. the top 2048), so
    one head's scores are [1, D] x [D, k] instead of a scan of every key; the
    request's isolation is unchanged: its logical positions go through its
    own block table to physical slots.  Sequence b uses the entries
    topk_indices[b, :topk_lens[b]] (a position listed twice counts twice).
    Returns o [B', H, kv_lora_rank] and lse [B', H]."""
    B, H, D = q_bits.shape
    NB, P, D2 = kv_bits.shape
    if D2 != row_width(kv_dtype, D):
        raise ValueError("q and cache head sizes differ")
    bits = kv_bits.reshape(NB * P, D2)
    sc = float(np.float32(scale))
    idx = range(B) if batches is None else batches
    outs, lses = [], []
    for b in idx:
        chosen = [int(t) for t in topk_indices[b, :int(topk_lens[b])]]
        slots = [physical_slot(block_table[b], t, P) for t in chosen]
        K = decode_kv(bits[np.asarray(slots, dtype=np.int64)] if slots else bits[:0], kv_dtype,
                      k_scale)
        o, lse = attend(bf16_bits_to_f64(q_bits[b]), K, kv_lora_rank, sc)
        outs.append(o)
        lses.append(lse)
    return np.stack(outs), np.stack(lses)


# ---------------------------------------------------------------- split-KV merge

def segment_bounds(n: int, chunk: int) -> List[Tuple[int, int]]:
    """lshu.cn article, section 12: consecutive KV segments of ``chunk``
    positions, [s*chunk, min((s+1)*chunk, n)); the last may be short."""
    return [(s, min(s + chunk, n)) for s in range(0, n, chunk)]


def merge_partials(partials: Sequence[Tuple[np.ndarray, np.ndarray, np.ndarray]]
                   ) -> Tuple[np.ndarray, np.ndarray]:
    """lshu.cn article, section 12: each segment brings its local max m_s, its
    local exponent sum l_s and its unnormalised weighted output O_s; then
    m = max_s m_s, l = sum_s e^(m_s - m) l_s, O = sum_s e^(m_s - m) O_s / l.
    Segments with l_s == 0 (empty) carry no weight.  Returns (o, lse)."""
    live = [(m, l, O) for (m, l, O) in partials if np.all(l > 0)]
    if not live:
        m0, l0, O0 = partials[0]
        return np.zeros_like(O0), np.full(m0.shape, -np.inf)
    m = np.max(np.stack([p[0] for p in live]), axis=0)
    l = sum(np.exp(ms - m) * ls for (ms, ls, _) in live)
    O = sum(np.exp(ms - m)[:, None] * Os for (ms, _, Os) in live) / l[:, None]
    return O, m + np.log(l)


def merge_normalised(partials: Sequence[Tuple[np.ndarray, np.ndarray]]
                     ) -> Tuple[np.ndarray, np.ndarray]:
    """The same merge written for partials stored as (o_s, lse_s), the form
    the Triton MLA page keeps (a kv_lora_rank-wide partial plus one LSE slot
    that the second stage uses): lse = ln sum_s e^lse_s,
    o = sum_s e^(lse_s - lse) o_s."""
    live = [(o, l) for (o, l) in partials if np.all(np.isfinite(l))]
    if not live:
        o0, l0 = partials[0]
        return np.zeros_like(o0), np.full(l0.shape, -np.inf)
    M = np.max(np.stack([l for (_, l) in live]), axis=0)
    w = [np.exp(l - M) for (_, l) in live]
    tot = sum(w)
    o = sum(wi[:, None] * oi for wi, (oi, _) in zip(w, live)) / tot[:, None]
    return o, M + np.log(tot)


def segment_partial(q: np.ndarray, K: np.ndarray, d_v: int, scale: float
                    ) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """(m_s, l_s, O_s) of one segment: local max, local exponent sum and the
    unnormalised sum of e^(s - m_s) V (lshu.cn article, section 12)."""
    H = q.shape[0]
    if K.shape[0] == 0:
        return np.full(H, -np.inf), np.zeros(H), np.zeros((H, d_v))
    s = (q @ K.T) * scale
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    return m, e.sum(axis=1), e @ K[:, :d_v]


def decode_split(q_bits: np.ndarray, kv_bits: np.ndarray, block_table: np.ndarray,
                 seq_lens: np.ndarray, *, scale: float, k_scale: float, kv_dtype: str,
                 kv_lora_rank: int,
                 bounds_of: Callable[[int, int], Sequence[Tuple[int, int]]],
                 normalised: bool = False) -> Tuple[np.ndarray, np.ndarray]:
    """Split-KV decode: ``bounds_of(b, n)`` lists the [start, end) segments of
    sequence b; each segment is attended on its own and the partials are merged
    by section 12's formula (or its (o_s, lse_s) form when ``normalised``)."""
    B, H, D = q_bits.shape
    NB, P, D2 = kv_bits.shape
    bits = kv_bits.reshape(NB * P, D2)
    sc = float(np.float32(scale))
    outs, lses = [], []
    for b in range(B):
        n = int(seq_lens[b])
        q = bf16_bits_to_f64(q_bits[b])
        K = decode_kv(gather_rows(bits, block_table[b], n, P), kv_dtype, k_scale)
        segs = list(bounds_of(b, n)) or [(0, 0)]
        if normalised:
            parts = [attend(q, K[s:e], kv_lora_rank, sc) for (s, e) in segs]
            o, lse = merge_normalised(parts)
        else:
            parts = [segment_partial(q, K[s:e], kv_lora_rank, sc) for (s, e) in segs]
            o, lse = merge_partials(parts)
        outs.append(o)
        lses.append(lse)
    return np.stack(outs), np.stack(lses)


# ---------------------------------------------------------------- cross-shard merge

def merge_shards(o_parts: np.ndarray, lse_parts: np.ndarray, lse_base: str = "ln"
                 ) -> Tuple[np.ndarray, np.ndarray]:
    """Merge of the results of G context shards (decode context parallelism:
    Triton MLA page, design motivation, and AttentionBackend page, limits:
    shards are combined through their LSE, which must be read in the base it
    was written in).  o_parts [G, ..., D_v] holds each shard's normalised
    output over its own keys and lse_parts [G, ...] its log-sum-exp, in
    natural log (``lse_base="ln"``) or base 2 (``"log2"``).  Per row:
    lse = ln sum_g e^lse_g and o = sum_g e^(lse_g - lse) o_g; a shard with
    lse_g = -inf (no keys) has weight 0, and a row no shard saw gets o = 0,
    lse = -inf.  Returns (o, lse) with lse in natural log."""
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse = np.asarray(lse_parts, dtype=np.float64)
    if lse_base == "log2":
        lse = lse * math.log(2.0)
    elif lse_base != "ln":
        raise ValueError(f"unknown lse base {lse_base!r}")
    G = lse.shape[0]
    out_o = np.zeros(o_parts.shape[1:])
    out_l = np.full(lse.shape[1:], -np.inf)
    for idx in np.ndindex(*lse.shape[1:]):
        ls = [lse[(g,) + idx] for g in range(G)]
        live = [g for g in range(G) if ls[g] != -np.inf]
        if not live:
            continue
        M = max(ls[g] for g in live)
        w = {g: math.exp(ls[g] - M) for g in live}
        tot = math.fsum(w.values())
        out_o[idx] = sum(w[g] * o_parts[(g,) + idx] for g in live) / tot
        out_l[idx] = M + math.log(tot)
    return out_o, out_l


# ---------------------------------------------------------------- split count rule

def pages_split_count(max_seq_len: int, num_sms: int) -> int:
    """Triton MLA page, key files (``_compute_num_kv_splits``): KV splits from
    max_seq_len / 512, capped at twice the SM count.  Read as a ceiling
    division clamped to [1, 2 * num_sms]."""
    return max(1, min(-(-int(max_seq_len) // 512), 2 * int(num_sms)))


__all__ = [
    "ROPE_DIM", "bf16_bits_to_f64", "e4m3fn_bits_to_f64", "E4M3FN_VALUES", "decode_kv",
    "physical_slot", "gather_rows", "attend", "decode", "segment_bounds", "merge_partials",
    "merge_normalised", "segment_partial", "decode_split", "pages_split_count",
    "visible_keys", "decode_mtp", "decode_sparse", "row_width", "PER_TOKEN_PAD",
    "PER_TOKEN_DTYPES", "int8_bits_to_f64", "int4_bits_to_f64", "code_bytes", "merge_shards",
]
