"""GPU parity of multi-token decode (verification of q_len new positions,
lshu.cn article, section 10) against the float64 oracle, through the C ABI.

Query token i of a sequence with n keys sees positions < n - q_len + 1 + i.
The q_len x H rows run through the same kernels as single-token decode, with
a per-row causal limit on the last tile(s); rows whose limit leaves a split
segment empty must carry no weight in the merge.  Tolerances as for
single-token decode: o 1e-2 / lse 1e-3 (bf16 cache), 3e-2 / 3e-3 (fp8).
"""
import numpy as np
import pytest

import oracle
import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL = {"bf16": (1e-2, 1e-3), "fp8_e4m3": (3e-2, 3e-3)}


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_paged_latent_decode_amd as m
    m.load_library()
    return m


def to_dev(inp):
    dev = torch.device("cuda:0")
    q = torch.from_numpy(inp.q_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    if inp.kv_dtype == "bf16":
        kv = torch.from_numpy(inp.kv_bits.view(np.int16)).view(torch.bfloat16).to(dev)
    else:
        kv = torch.from_numpy(inp.kv_bits).view(torch.float8_e4m3fn).to(dev)
    bt = torch.from_numpy(np.ascontiguousarray(inp.block_table)).to(dev)
    sl = torch.from_numpy(np.ascontiguousarray(inp.seq_lens)).to(dev)
    return q, kv, bt, sl


def run_gpu(mla, inp, splits, mode, o_dtype=None, dev_inputs=None):
    w = inp.workload
    q, kv, bt, sl = dev_inputs or to_dev(inp)
    o, lse = mla.mla_decode(q, kv, bt, sl, w.scale, w.page_size, w.k_scale, splits,
                            split_mode=mode, o_dtype=o_dtype or torch.bfloat16)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def ref(inp, batches=None):
    w = inp.workload
    return oracle.decode_mtp(inp.q_bits, inp.kv_bits, inp.block_table, inp.seq_lens,
                             scale=w.scale, k_scale=w.k_scale, kv_dtype=w.kv_dtype,
                             kv_lora_rank=w.kv_lora_rank, batches=batches)


def bf16_half_ulp(x):
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(ax)) - 8)


def assert_close(inp, o, lse, ro, rl, label, rounding_slack=False, batches=None):
    """Rows that see no key must be exactly o = 0, lse = -inf; the others are
    compared at the stated tolerance (bf16 output: plus the final rounding)."""
    to, tl = TOL[inp.kv_dtype]
    sl = np.asarray(inp.seq_lens if batches is None else inp.seq_lens[batches])
    ql = inp.q_bits.shape[1]
    vis = np.array([[oracle.visible_keys(int(n), ql, i) for i in range(ql)] for n in sl])
    empty = vis == 0                                   # [B, q_len]
    if empty.any():
        assert np.all(o[empty] == 0) and np.all(np.isneginf(lse[empty])), label
    live = ~empty
    do = np.abs(o[live] - ro[live]).max() if live.any() else 0.0
    dl = np.abs(lse[live] - rl[live]).max() if live.any() else 0.0
    print(f"{label}: max|do|={do:.3e} max|dlse|={dl:.3e}", flush=True)
    assert np.all(np.isfinite(o[live])) and np.all(np.isfinite(lse[live])), label
    if rounding_slack:
        excess = (np.abs(o[live] - ro[live]) - bf16_half_ulp(ro[live])).max()
        assert excess <= to and dl <= tl, (label, excess, dl)
    else:
        assert do <= to and dl <= tl, (label, do, dl)


MTP_CASES = [
    # (H, D, P, seq_lens, q_len): short last tiles next to the causal tail, tails
    # that straddle a 32-position tile, and rows that see nothing
    (16, 576, 16, (1, 2, 8, 31, 33, 64, 65, 100), 8),
    (128, 576, 64, (3, 34, 700, 1031), 2),
    (32, 576, 32, (40, 96, 97), 3),
    (128, 576, 64, (65, 66, 129, 2000), 4),
    (16, 320, 16, (5, 33, 250), 5),
    (48, 576, 16, (9, 200), 6),
]


@pytest.mark.parametrize("case", range(len(MTP_CASES)))
@pytest.mark.parametrize("mode,splits", [(0, 1), (0, 3), (1, 1), (1, 4), (1, 37)])
def test_mtp_ragged_cases(mla, case, mode, splits):
    H, D, P, sl, ql = MTP_CASES[case]
    inp = W.small_case(seed=300 + case, batch=len(sl), num_heads=H, head_size=D,
                       kv_lora_rank=D - 64, page_size=P, seq_lens=sl, table_pad=1, q_len=ql)
    ro, rl = ref(inp)
    label = f"mtp case{case} H={H} D={D} q_len={ql} mode={mode} S={splits}"
    o, lse = run_gpu(mla, inp, splits, mode, o_dtype=torch.float32)
    assert_close(inp, o, lse, ro, rl, label + " fp32-o")
    o, lse = run_gpu(mla, inp, splits, mode)
    assert_close(inp, o, lse, ro, rl, label + " bf16-o", rounding_slack=True)


@pytest.mark.parametrize("mode,splits", [(0, 1), (0, 3), (1, 5)])
def test_mtp_fp8_cache(mla, mode, splits):
    sl, ql = (2, 33, 300, 1025), 4
    inp = W.small_case(seed=310, batch=len(sl), num_heads=128, head_size=576, kv_lora_rank=512,
                       page_size=64, seq_lens=sl, kv_dtype=W.FP8_E4M3,
                       k_scale=float(np.float32(0.05)), q_len=ql)
    ro, rl = ref(inp)
    o, lse = run_gpu(mla, inp, splits, mode, o_dtype=torch.float32)
    assert_close(inp, o, lse, ro, rl, f"mtp fp8 mode={mode} S={splits}")


def test_mtp_one_token_equals_plain_decode(mla):
    """A [B, 1, H, D] query through the multi-token path is bitwise the
    [B, H, D] single-token decode."""
    sl = (37, 100, 1, 64)
    inp = W.small_case(seed=311, batch=len(sl), num_heads=128, head_size=576, kv_lora_rank=512,
                       page_size=64, seq_lens=sl)
    q, kv, bt, sl_d = to_dev(inp)
    w = inp.workload
    for mode, splits in ((0, 1), (1, 3)):
        o3, l3 = mla.mla_decode(q, kv, bt, sl_d, w.scale, w.page_size, w.k_scale, splits,
                                split_mode=mode)
        o4, l4 = mla.mla_decode(q[:, None].contiguous(), kv, bt, sl_d, w.scale, w.page_size,
                                w.k_scale, splits, split_mode=mode)
        torch.cuda.synchronize()
        assert torch.equal(o3, o4[:, 0]) and torch.equal(l3, l4[:, 0])


@pytest.mark.parametrize("mode,splits", [(0, 1), (1, 6)])
def test_mtp_page_permutation_is_bitwise_invariant(mla, mode, splits):
    sl, ql = (70, 3, 129), 3
    inp = W.small_case(seed=312, batch=len(sl), num_heads=32, head_size=576, kv_lora_rank=512,
                       page_size=16, seq_lens=sl, q_len=ql, extra_pages=5)
    a = run_gpu(mla, inp, splits, mode)
    b = run_gpu(mla, W.permute_pages(inp, seed=9), splits, mode)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_mtp_full_size(mla):
    """The dsv3_mtp2 workload (B=64, q_len=2, H=128) at the planner's launch
    configuration, at the pages' split count and in the single-split mode, every
    sequence compared with the oracle (fp32 output at the plain tolerances, bf16
    output beyond its final rounding)."""
    inp = W.generate("dsv3_mtp2")
    w = inp.workload
    dev_inputs = to_dev(inp)
    sl = np.asarray(inp.seq_lens)
    ro, rl = ref(inp)
    shape = mla.shape_of(*dev_inputs[:2], dev_inputs[2])
    max_len, tot = int(sl.max()), int(sl.sum())
    mode, units, _ = mla.mla_plan(shape, max_len, tot, 256, q_len=w.q_len)
    print(f"dsv3_mtp2: tokens={tot} plan mode={mode} units={units}", flush=True)
    for mode, splits in [(mode, units)] + [(0, s) for s in w.parity_splits]:
        label = f"dsv3_mtp2 mode={mode} S={splits}"
        o, lse = run_gpu(mla, inp, splits, mode, o_dtype=torch.float32, dev_inputs=dev_inputs)
        assert_close(inp, o, lse, ro, rl, label + " o=f32")
        o, lse = run_gpu(mla, inp, splits, mode, dev_inputs=dev_inputs)
        assert_close(inp, o, lse, ro, rl, label + " o=bf16", rounding_slack=True)
