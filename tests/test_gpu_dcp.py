"""GPU parity of the cross-shard merge of a context-parallel decode (the C
ABI's mla_merge_shards, via the ctypes binding).

Each shard r owns the round-robin pages j % G == r of every sequence
(workloads.shard_pages); the library decodes every shard as an ordinary
batch, and the merge combines the shards through their LSE (Triton MLA page,
design motivation: decode returns lse because the shards are merged with it;
AttentionBackend page, limits: the lse base must be the one it was written
in).  On one GPU the shards run one after the other; across GPUs only the
exchange of (o_g, lse_g) would be added.

Checks: the merge kernel alone against the oracle's merge_shards on random
shard results (dead shards with NaN rows, base-2 lse, bf16 and fp32 in and
out; max-abs 2e-5 of the row scale plus the output's bf16 rounding), and the
whole sharded decode against the oracle's unsharded decode (the decode
tolerances: o 1e-2, lse 1e-3).
"""
import numpy as np
import pytest

import oracle
import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_paged_latent_decode_amd as m
    m.load_library()
    return m


DEV = "cuda:0"


def bf16_round(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def half_ulp_bf16(x):
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(ax)) - 8)


@pytest.mark.parametrize("G", [1, 2, 3, 8, 13])
@pytest.mark.parametrize("d_v", [512, 256])
@pytest.mark.parametrize("parts,out", [("bf16", "bf16"), ("f32", "f32"), ("bf16", "f32")])
@pytest.mark.parametrize("base", ["ln", "log2"])
def test_merge_kernel_matches_oracle(mla, G, d_v, parts, out, base):
    rng = np.random.default_rng(1000 + 7 * G + d_v)
    B, H = 3, 32
    o_p = rng.standard_normal((G, B, H, d_v)).astype(np.float32)
    l_p = (rng.standard_normal((G, B, H)) * 3.0).astype(np.float32)
    dead = rng.random((G, B, H)) < 0.15
    l_p[dead] = -np.inf
    o_p[dead] = np.nan  # a shard without keys may hold anything
    l_p[:, 1, 5] = -np.inf  # a row no shard saw
    o_p[:, 1, 5] = np.nan
    if base == "log2":
        l_in = (l_p / np.float32(np.log(2.0))).astype(np.float32)
    else:
        l_in = l_p
    o_t = bf16_round(o_p) if parts == "bf16" else torch.from_numpy(o_p)
    o_exact = o_t.float().numpy().astype(np.float64)
    ro, rl = oracle.merge_shards(np.where(np.isnan(o_exact), 0.0, o_exact), l_in.astype(np.float64),
                                 lse_base=base)
    print(f"[merge] G={G} d_v={d_v} parts={parts} out={out} base={base}", flush=True)
    o, lse = mla.mla_merge_shards(o_t.to(DEV), torch.from_numpy(l_in).to(DEV), base,
                                  o_dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    empty = np.isneginf(rl)
    assert empty[1, 5]
    assert np.all(o[empty] == 0) and np.all(np.isneginf(lse[empty]))
    live = ~empty
    assert np.all(np.isfinite(o[live])) and np.all(np.isfinite(lse[live]))
    slack = half_ulp_bf16(ro[live]) if out == "bf16" else 0.0
    scale = np.abs(o_exact[np.isfinite(o_exact)]).max()
    assert (np.abs(o[live] - ro[live]) - slack).max() <= 2e-5 * scale
    assert np.abs(lse[live] - rl[live]).max() <= 1e-5 * max(1.0, np.abs(rl[live]).max())


def to_dev(inp):
    q = torch.from_numpy(inp.q_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    kv = torch.from_numpy(inp.kv_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    bt = torch.from_numpy(np.ascontiguousarray(inp.block_table)).to(DEV)
    sl = torch.from_numpy(np.ascontiguousarray(inp.seq_lens)).to(DEV)
    return q, kv, bt, sl


def sharded_decode(mla, inp, G, shard_dtype, out_dtype, kv=None):
    """Decode each page shard with the library, then merge the shards."""
    w = inp.workload
    q = torch.from_numpy(inp.q_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    if kv is None:
        kv = torch.from_numpy(inp.kv_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    os_, ls_ = [], []
    for r in range(G):
        sh = W.shard_pages(inp, G, r)
        bt = torch.from_numpy(np.ascontiguousarray(sh.block_table)).to(DEV)
        sl = torch.from_numpy(np.ascontiguousarray(sh.seq_lens)).to(DEV)
        o, lse = mla.mla_decode(q, kv, bt, sl, w.scale, w.page_size, w.k_scale,
                                o_dtype=shard_dtype, num_cus=256)
        os_.append(o)
        ls_.append(lse)
    o_p = torch.stack(os_).contiguous()
    l_p = torch.stack(ls_).contiguous()
    o, lse = mla.mla_merge_shards(o_p, l_p, "ln", o_dtype=out_dtype)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


CASES = [
    # (H, D, P, seq_lens)
    (128, 576, 64, (1, 63, 64, 65, 700, 1031)),
    (16, 576, 16, (1, 31, 32, 33, 100, 257)),
    (32, 320, 16, (5, 96, 97, 300)),
]


@pytest.mark.parametrize("c", range(len(CASES)))
@pytest.mark.parametrize("G", [2, 4, 8])
def test_sharded_decode_equals_unsharded(mla, c, G):
    H, D, P, sl = CASES[c]
    inp = W.small_case(seed=400 + c, batch=len(sl), num_heads=H, head_size=D,
                       kv_lora_rank=D - 64, page_size=P, seq_lens=sl)
    ro, rl = oracle.decode(inp.q_bits, inp.kv_bits, inp.block_table, inp.seq_lens,
                           scale=inp.workload.scale, k_scale=1.0, kv_dtype="bf16",
                           kv_lora_rank=D - 64)
    print(f"[dcp] case{c} H={H} D={D} P={P} G={G}", flush=True)
    # fp32 shard results and output: the arithmetic alone
    o, lse = sharded_decode(mla, inp, G, torch.float32, torch.float32)
    do, dl = np.abs(o - ro).max(), np.abs(lse - rl).max()
    print(f"  f32: max|do|={do:.3e} max|dlse|={dl:.3e}", flush=True)
    assert do <= 1e-2 and dl <= 1e-3
    # bf16 shard results and output, as a serving stack would exchange them
    o, lse = sharded_decode(mla, inp, G, torch.bfloat16, torch.bfloat16)
    excess = (np.abs(o - ro) - half_ulp_bf16(ro)).max()
    assert excess <= 1e-2 and np.abs(lse - rl).max() <= 1e-3


def test_sharded_decode_full_size_dsv3(mla):
    """The dsv3 batch (B=64, H=128, lengths 1024..8192) over 8 page shards,
    every sequence checked against the unsharded oracle: fp32 shard results and
    output at the plain tolerances, then bf16 shard results and output (as a
    serving stack would exchange them) beyond the final bf16 rounding."""
    inp = W.generate("dsv3")
    w = inp.workload
    ro, rl = oracle.decode(inp.q_bits, inp.kv_bits, inp.block_table, inp.seq_lens,
                           scale=w.scale, k_scale=1.0, kv_dtype="bf16",
                           kv_lora_rank=w.kv_lora_rank)
    print("[dcp] dsv3 G=8, all 64 sequences", flush=True)
    o, lse = sharded_decode(mla, inp, 8, torch.float32, torch.float32)
    do, dl = np.abs(o - ro).max(), np.abs(lse - rl).max()
    print(f"  f32: max|do|={do:.3e} max|dlse|={dl:.3e}", flush=True)
    assert do <= 1e-2 and dl <= 1e-3
    o, lse = sharded_decode(mla, inp, 8, torch.bfloat16, torch.bfloat16)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    excess = (np.abs(o - ro) - half_ulp_bf16(ro)).max()
    assert excess <= 1e-2 and np.abs(lse - rl).max() <= 1e-3
