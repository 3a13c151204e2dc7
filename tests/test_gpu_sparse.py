"""GPU parity of sparse (top-k) decode (lshu.cn article, section 13) against
the float64 oracle, through the C ABI.

Sequence b attends to the cache rows of the logical positions
topk_indices[b, :topk_lens[b]], each reached through its block table.  The
kernels are those of dense decode with an index-driven gather, so beside the
oracle comparison (o 1e-2, lse 1e-3) a list of every position in order must
reproduce dense decode bitwise, and slots no list names may hold NaN.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE = 1e-2, 1e-3


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_paged_latent_decode_amd as m
    m.load_library()
    return m


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.device("cuda:0"))


def kv_dev(inp):
    if inp.kv_dtype == W.BF16:
        return dev(inp.kv_bits.view(np.int16)).view(torch.bfloat16)
    if inp.kv_dtype == W.FP8_E4M3:
        return dev(inp.kv_bits).view(torch.float8_e4m3fn)
    return dev(inp.kv_bits)  # per-token rows: uint8


def run_sparse(mla, inp, splits, mode, idx=None, lens=None, o_dtype=None):
    w = inp.workload
    q = dev(inp.q_bits.view(np.int16)).view(torch.bfloat16)
    print(f"[sparse] {w.kv_dtype} B={len(inp.seq_lens)} H={w.num_heads} D={w.head_size} "
          f"P={w.page_size} mode={mode} S={splits}", flush=True)
    o, lse = mla.mla_decode_sparse(q, kv_dev(inp), dev(inp.block_table),
                                   dev(inp.topk_indices if idx is None else idx),
                                   dev(inp.topk_lens if lens is None else lens), w.scale,
                                   w.page_size, w.k_scale, splits, split_mode=mode,
                                   o_dtype=o_dtype or torch.bfloat16, kv_dtype=w.kv_dtype)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def ref(inp, idx=None, lens=None, batches=None):
    w = inp.workload
    return oracle.decode_sparse(inp.q_bits, inp.kv_bits, inp.block_table,
                                inp.topk_indices if idx is None else idx,
                                inp.topk_lens if lens is None else lens, scale=w.scale,
                                k_scale=w.k_scale, kv_dtype=w.kv_dtype,
                                kv_lora_rank=w.kv_lora_rank, batches=batches)


def check(o, lse, ro, rl, lens, label):
    lens = np.asarray(lens)
    empty = lens == 0
    if empty.any():
        assert np.all(o[empty] == 0) and np.all(np.isneginf(lse[empty])), label
    live = ~empty
    do = np.abs(o[live] - ro[live]).max()
    dl = np.abs(lse[live] - rl[live]).max()
    print(f"{label}: max|do|={do:.3e} max|dlse|={dl:.3e}", flush=True)
    assert np.all(np.isfinite(o[live])) and np.all(np.isfinite(lse[live])), label
    assert do <= TOL_O and dl <= TOL_LSE, (label, do, dl)


SPARSE_CASES = [
    # (H, D, P, seq_lens, topk): every head tiling (16-head waves, 1/2/4 waves
    # of 32 heads, several head chunks) and both head sizes
    (128, 576, 64, (300, 2000, 40, 1031), 256),
    (128, 576, 16, (1, 33, 64, 100), 48),
    (256, 576, 64, (700, 129), 100),
    (16, 576, 16, (1, 33, 64, 100), 48),
    (32, 576, 32, (500, 97), 80),
    (48, 576, 16, (3, 129, 40), 40),
    (64, 576, 64, (300, 2000), 200),
    (16, 320, 16, (1, 31, 33, 250, 513), 64),
    (128, 320, 32, (17, 95, 333), 72),
    # page sizes that are no power of two (the gather divides by P) and large pages
    (128, 576, 48, (1, 47, 48, 49, 500), 64),
    (64, 576, 80, (3, 161, 700), 120),
    (128, 576, 512, (1, 511, 513, 1600), 300),
]


@pytest.mark.parametrize("case", range(len(SPARSE_CASES)))
@pytest.mark.parametrize("mode,splits", [(0, 1), (0, 3), (1, 1), (1, 5), (1, 37)])
def test_sparse_cases(mla, case, mode, splits):
    H, D, P, sl, k = SPARSE_CASES[case]
    inp = W.small_case(seed=400 + case, batch=len(sl), num_heads=H, head_size=D,
                       kv_lora_rank=D - 64, page_size=P, seq_lens=sl, topk=k)
    ro, rl = ref(inp)
    o, lse = run_sparse(mla, inp, splits, mode, o_dtype=torch.float32)
    check(o, lse, ro, rl, inp.topk_lens, f"sparse case{case} mode={mode} S={splits}")


@pytest.mark.parametrize("H,D", [(128, 576), (16, 576), (64, 576), (128, 320), (16, 320)])
@pytest.mark.parametrize("mode,splits", [(0, 1), (0, 4), (1, 7)])
def test_sparse_over_every_position_is_dense_decode_bitwise(mla, mode, splits, H, D):
    sl = (37, 100, 1, 700)
    inp = W.small_case(seed=410, batch=len(sl), num_heads=H, head_size=D, kv_lora_rank=D - 64,
                       page_size=64, seq_lens=sl)
    idx = np.zeros((len(sl), 704), np.int32)
    for b, n in enumerate(sl):
        idx[b, :n] = np.arange(n)
    w = inp.workload
    q = dev(inp.q_bits.view(np.int16)).view(torch.bfloat16)
    kv = dev(inp.kv_bits.view(np.int16)).view(torch.bfloat16)
    bt, lens = dev(inp.block_table), dev(np.asarray(sl, np.int32))
    od, ld = mla.mla_decode(q, kv, bt, lens, w.scale, w.page_size, w.k_scale, splits,
                            split_mode=mode)
    os_, ls_ = mla.mla_decode_sparse(q, kv, bt, dev(idx), lens, w.scale, w.page_size,
                                     w.k_scale, splits, split_mode=mode)
    torch.cuda.synchronize()
    assert torch.equal(od, os_) and torch.equal(ld, ls_)


@pytest.mark.parametrize("mode,splits", [(0, 1), (1, 5)])
def test_sparse_ignores_unlisted_slots(mla, mode, splits):
    """NaN in every cache slot that no list names (including the unused
    entries of each list's row) changes nothing."""
    sl = (300, 900, 64)
    inp = W.small_case(seed=411, batch=len(sl), num_heads=128, head_size=576, kv_lora_rank=512,
                       page_size=16, seq_lens=sl, topk=96)
    a = run_sparse(mla, inp, splits, mode)
    P = inp.workload.page_size
    used = np.zeros(inp.kv_bits.shape[:2], dtype=bool)
    for b in range(len(sl)):
        for t in inp.topk_indices[b, :inp.topk_lens[b]]:
            used[inp.block_table[b, t // P], t % P] = True
    kv = inp.kv_bits.copy()
    kv[~used] = np.uint16(0x7FC0)
    poisoned = dataclasses.replace(inp, kv_bits=kv)
    b_ = run_sparse(mla, poisoned, splits, mode)
    assert np.all(np.isfinite(b_[0])) and np.all(np.isfinite(b_[1]))
    assert np.array_equal(a[0], b_[0]) and np.array_equal(a[1], b_[1])


QUANT_CASES = [
    # (H, D, P, seq_lens, topk): 1-byte and 4-bit caches through the same gather
    (128, 576, 64, (300, 2000, 40, 1031), 256),
    (16, 576, 16, (1, 33, 64, 100), 48),
    (64, 576, 64, (300, 2000), 200),
    (128, 320, 32, (17, 95, 333), 72),
    (128, 576, 48, (47, 49, 500), 64),
    (128, 576, 1024, (1, 1025, 2500), 300),
]
QUANT_DTYPES = [W.FP8_E4M3, W.FP8_PER_TOKEN, W.INT8_PER_TOKEN, W.INT4_PER_TOKEN]


@pytest.mark.parametrize("dt", QUANT_DTYPES)
@pytest.mark.parametrize("case", range(len(QUANT_CASES)))
@pytest.mark.parametrize("mode,splits", [(0, 1), (0, 3), (1, 5), (1, 37)])
def test_sparse_quantised_caches(mla, case, mode, splits, dt):
    """Quantised caches (per-tensor fp8; per-token fp8 / int8 / int4 with
    inline scales) gathered by the index lists; tolerances of the fp8 cache."""
    H, D, P, sl, k = QUANT_CASES[case]
    inp = W.small_case(seed=420 + case, batch=len(sl), num_heads=H, head_size=D,
                       kv_lora_rank=D - 64, page_size=P, seq_lens=sl, topk=k, kv_dtype=dt,
                       k_scale=0.05 if dt == W.FP8_E4M3 else 1.0)
    ro, rl = ref(inp)
    o, lse = run_sparse(mla, inp, splits, mode, o_dtype=torch.float32)
    lens = np.asarray(inp.topk_lens)
    empty = lens == 0
    live = ~empty
    assert np.all(o[empty] == 0) and np.all(np.isneginf(lse[empty]))
    do = np.abs(o[live] - ro[live]).max()
    dl = np.abs(lse[live] - rl[live]).max()
    print(f"sparse {dt} case{case} mode={mode} S={splits}: max|do|={do:.3e} max|dlse|={dl:.3e}",
          flush=True)
    assert np.all(np.isfinite(o[live])) and do <= 3e-2 and dl <= 3e-3


@pytest.mark.parametrize("dt", QUANT_DTYPES)
@pytest.mark.parametrize("mode,splits", [(0, 1), (1, 7)])
def test_sparse_quantised_over_every_position_is_dense_bitwise(mla, mode, splits, dt):
    sl = (37, 100, 1, 700)
    inp = W.small_case(seed=430, batch=len(sl), num_heads=128, head_size=576, kv_lora_rank=512,
                       page_size=64, seq_lens=sl, kv_dtype=dt,
                       k_scale=0.05 if dt == W.FP8_E4M3 else 1.0)
    idx = np.zeros((len(sl), 704), np.int32)
    for b, n in enumerate(sl):
        idx[b, :n] = np.arange(n)
    w = inp.workload
    q = dev(inp.q_bits.view(np.int16)).view(torch.bfloat16)
    kv = kv_dev(inp)
    bt, lens = dev(inp.block_table), dev(np.asarray(sl, np.int32))
    od, ld = mla.mla_decode(q, kv, bt, lens, w.scale, w.page_size, w.k_scale, splits,
                            split_mode=mode, kv_dtype=w.kv_dtype)
    os_, ls_ = mla.mla_decode_sparse(q, kv, bt, dev(idx), lens, w.scale, w.page_size,
                                     w.k_scale, splits, split_mode=mode, kv_dtype=w.kv_dtype)
    torch.cuda.synchronize()
    assert torch.equal(od, os_) and torch.equal(ld, ls_)


def test_sparse_full_size(mla):
    """dsv3_sparse (B=64, H=128, top-2048 of U[2048,8192]) at the planner's
    configuration, at per-sequence split counts and in the single-split mode,
    every sequence compared with the oracle, with fp32 and with bf16 output."""
    inp = W.generate("dsv3_sparse")
    w = inp.workload
    ro, rl = ref(inp)
    q = dev(inp.q_bits.view(np.int16)).view(torch.bfloat16)
    kv = dev(inp.kv_bits.view(np.int16)).view(torch.bfloat16)
    bt, idx, lens = dev(inp.block_table), dev(inp.topk_indices), dev(inp.topk_lens)
    shape = mla.shape_of(q, kv, bt)
    mode, units, _ = mla.mla_plan(shape, w.topk, int(inp.topk_lens.sum()), 256)
    print(f"dsv3_sparse: entries={int(inp.topk_lens.sum())} plan mode={mode} units={units}",
          flush=True)
    runs = [(mode, units)] + [(0, s) for s in w.parity_splits]
    if (0, 1) not in runs:
        runs.append((0, 1))
    for mode, splits in runs:
        for o_dtype in (torch.float32, torch.bfloat16):
            o, lse = mla.mla_decode_sparse(q, kv, bt, idx, lens, w.scale, w.page_size,
                                           w.k_scale, splits, split_mode=mode, o_dtype=o_dtype)
            torch.cuda.synchronize()
            o = o.float().cpu().numpy().astype(np.float64)
            lse = lse.cpu().numpy().astype(np.float64)
            check(o, lse, ro, rl, inp.topk_lens, f"dsv3_sparse mode={mode} S={splits} o={o_dtype}")
