"""GPU parity: libmla's HIP path against the float64 oracle, element by
element, through the C ABI (via the ctypes binding).

Tolerances (max-abs): o 1e-2 and lse 1e-3 for bf16 caches, 3e-2 and 3e-3 for
fp8 e4m3 caches.  Page indexing is checked bit-exactly through invariances:
moving pages, or poisoning every slot no sequence reads, leaves the output
bitwise unchanged.
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
    return oracle.decode(inp.q_bits, inp.kv_bits, inp.block_table, inp.seq_lens, scale=w.scale,
                         k_scale=w.k_scale, kv_dtype=w.kv_dtype, kv_lora_rank=w.kv_lora_rank,
                         batches=batches)


def bf16_half_ulp(x):
    """Half a bf16 ulp of |x| (8 significant bits): the most that rounding
    the exact result to a bf16 output can move it."""
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(ax)) - 8)


def assert_close(inp, o, lse, ro, rl, label="", rounding_slack=False):
    """Max-abs check at the stated tolerances.  With ``rounding_slack`` the
    o bound is widened element-wise by the final bf16 rounding of the exact
    value (used for short sequences, where |o| can exceed 2 and half a bf16
    ulp alone reaches 0.0078 or more)."""
    to, tl = TOL[inp.kv_dtype]
    empty = np.asarray(inp.seq_lens) == 0
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


# ---------------------------------------------------------------- the tiny config

@pytest.mark.parametrize("mode,splits", [(0, 1), (0, 4), (1, 1), (1, 2), (1, 5)])
def test_tiny_config(mla, mode, splits):
    inp = W.generate("tiny")
    o, lse = run_gpu(mla, inp, splits, mode)
    ro, rl = ref(inp)
    assert_close(inp, o, lse, ro, rl, f"tiny mode={mode} S={splits}")


# ---------------------------------------------------------------- ragged small cases

CASES = [
    # (H, D, P, seq_lens)
    (16, 576, 16, (1, 31, 32, 33, 64, 65, 100, 257)),
    (32, 576, 32, (5, 96, 97, 300)),
    (64, 576, 48, (1, 47, 48, 49, 500)),
    (128, 576, 64, (1, 63, 64, 65, 700, 1031)),
    (48, 576, 16, (3, 129, 40)),
    (16, 320, 16, (1, 31, 33, 250, 513)),
    (128, 320, 32, (17, 95, 333)),
    (256, 576, 64, (77, 129)),
    # head counts whose tilings run several head chunks per unit on 1- and 2-wave workgroups
    (96, 576, 32, (5, 97, 300)),
    (80, 576, 16, (1, 33, 129)),
    (192, 576, 64, (64, 65, 400)),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("mode,splits", [(0, 1), (0, 3), (1, 1), (1, 4), (1, 37)])
def test_ragged_cases(mla, case, mode, splits):
    H, D, P, sl = CASES[case]
    inp = W.small_case(seed=100 + case, batch=len(sl), num_heads=H, head_size=D,
                       kv_lora_rank=D - 64, page_size=P, seq_lens=sl, table_pad=2)
    ro, rl = ref(inp)
    label = f"case{case} H={H} D={D} P={P} mode={mode} S={splits}"
    # fp32 output: the kernel's own arithmetic against the stated tolerance
    o, lse = run_gpu(mla, inp, splits, mode, o_dtype=torch.float32)
    assert_close(inp, o, lse, ro, rl, label + " o=f32")
    # bf16 output: the same, plus the final rounding of each value
    o, lse = run_gpu(mla, inp, splits, mode)
    assert_close(inp, o, lse, ro, rl, label + " o=bf16", rounding_slack=True)


FP8_SCALE = float(np.float32(0.05))


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("mode,splits", [(0, 1), (0, 3), (1, 4), (1, 37)])
def test_ragged_cases_fp8(mla, case, mode, splits):
    H, D, P, sl = CASES[case]
    inp = W.small_case(seed=200 + case, batch=len(sl), num_heads=H, head_size=D,
                       kv_lora_rank=D - 64, page_size=P, seq_lens=sl, table_pad=1,
                       kv_dtype=W.FP8_E4M3, k_scale=FP8_SCALE)
    ro, rl = ref(inp)
    label = f"fp8 case{case} H={H} D={D} P={P} mode={mode} S={splits}"
    o, lse = run_gpu(mla, inp, splits, mode, o_dtype=torch.float32)
    assert_close(inp, o, lse, ro, rl, label + " o=f32")
    o, lse = run_gpu(mla, inp, splits, mode)
    assert_close(inp, o, lse, ro, rl, label + " o=bf16", rounding_slack=True)


@pytest.mark.parametrize("P", [512, 1024])
@pytest.mark.parametrize("mode,splits", [(0, 1), (0, 5), (1, 9)])
def test_large_pages_fp8(mla, P, mode, splits):
    """Per-tensor fp8 cache in pages of 512 and 1024 rows (sequences ending
    one row short of, and one row into, a page)."""
    sl = (1, P - 1, P + 1, 3 * P + 5)
    inp = W.small_case(seed=540 + P // 512, batch=len(sl), num_heads=128, head_size=576,
                       kv_lora_rank=512, page_size=P, seq_lens=sl, extra_pages=1,
                       kv_dtype=W.FP8_E4M3, k_scale=FP8_SCALE)
    ro, rl = ref(inp)
    o, lse = run_gpu(mla, inp, splits, mode, o_dtype=torch.float32)
    assert_close(inp, o, lse, ro, rl, f"fp8 P={P} mode={mode} S={splits} o=f32")


FINITE_E4M3 = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


@pytest.mark.parametrize("H,D", [(16, 576), (32, 576), (64, 576), (128, 576), (48, 320),
                                 (128, 320)])
@pytest.mark.parametrize("mode,splits", [(0, 1), (1, 2)])
def test_fp8_one_position_returns_the_widened_row(mla, H, D, mode, splits):
    """With a single position the softmax weight is 1, so o is that row's
    kv_c part times k_scale.  Each sequence's row runs through all 254 finite
    e4m3fn codes (both signs, subnormals, +-448), so every code must come
    back as its exact value: with k_scale = 0.375 the product has at most 6
    significant bits and is exact in bf16 as well as in fp32."""
    Dv, P, B = D - 64, 16, 3
    k_scale = 0.375
    rng = np.random.default_rng(21)
    nb = B + 2
    kv = rng.choice(FINITE_E4M3, size=(nb, P, D)).astype(np.uint8)
    for b in range(B):
        kv[b + 1, 0, :FINITE_E4M3.size] = np.roll(FINITE_E4M3, 37 * b)
    table = np.array([[b + 1, 0] for b in range(B)], dtype=np.int32)
    q = W.f32_to_bf16_bits(rng.standard_normal((B, H, D), dtype=np.float32) * 0.1)
    w = W.Workload(name="fp8-codes", seed=21, batch=B, num_heads=H, head_size=D,
                   kv_lora_rank=Dv, page_size=P, num_blocks=nb, kv_dtype=W.FP8_E4M3,
                   k_scale=k_scale, scale=W.DSV3_SCALE, seq_lens_fixed=(1,) * B)
    inp = W.DecodeInputs(workload=w, q_bits=q, kv_bits=kv, block_table=table,
                         seq_lens=np.ones(B, dtype=np.int32))
    ro, rl = ref(inp)
    o32, l32 = run_gpu(mla, inp, splits, mode, o_dtype=torch.float32)
    o16, _ = run_gpu(mla, inp, splits, mode)
    assert np.array_equal(o32, ro), np.abs(o32 - ro).max()
    assert np.array_equal(o16, ro), np.abs(o16 - ro).max()
    assert np.abs(l32 - rl).max() <= 1e-4 * max(1.0, np.abs(rl).max())


def test_fp32_output(mla):
    inp = W.small_case(seed=7, batch=3, num_heads=128, head_size=576, kv_lora_rank=512,
                       page_size=64, seq_lens=(100, 1000, 5))
    o, lse = run_gpu(mla, inp, 4, 1, o_dtype=torch.float32)
    ro, rl = ref(inp)
    # fp32 output removes the final bf16 rounding
    assert np.abs(o - ro).max() < 1e-2 and np.abs(lse - rl).max() < 1e-3


@pytest.mark.parametrize("mode,splits", [(0, 1), (0, 4), (1, 3)])
def test_empty_sequences(mla, mode, splits):
    inp = W.small_case(seed=9, batch=5, num_heads=16, head_size=576, kv_lora_rank=512,
                       page_size=16, seq_lens=(0, 50, 0, 1, 0))
    ro, rl = ref(inp)
    o, lse = run_gpu(mla, inp, splits, mode, o_dtype=torch.float32)
    assert_close(inp, o, lse, ro, rl, f"empty mode={mode} S={splits} o=f32")
    o, lse = run_gpu(mla, inp, splits, mode)
    assert_close(inp, o, lse, ro, rl, f"empty mode={mode} S={splits} o=bf16", rounding_slack=True)


# ---------------------------------------------------------------- bit-exact indexing

@pytest.mark.parametrize("kv_dtype", [W.BF16, W.FP8_E4M3])
@pytest.mark.parametrize("mode,splits", [(0, 1), (0, 4), (1, 6)])
def test_page_permutation_is_bitwise_invariant(mla, mode, splits, kv_dtype):
    inp = W.small_case(seed=11, batch=4, num_heads=128, head_size=576, kv_lora_rank=512,
                       page_size=16, seq_lens=(37, 100, 64, 257), extra_pages=9,
                       kv_dtype=kv_dtype, k_scale=FP8_SCALE if kv_dtype == W.FP8_E4M3 else 1.0)
    o, lse = run_gpu(mla, inp, splits, mode)
    o2, lse2 = run_gpu(mla, W.permute_pages(inp, seed=5), splits, mode)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


@pytest.mark.parametrize("kv_dtype", [W.BF16, W.FP8_E4M3])
@pytest.mark.parametrize("mode,splits", [(0, 1), (1, 3)])
@pytest.mark.parametrize("H,P", [(128, 64), (16, 16)])
def test_poisoned_unreferenced_slots(mla, mode, splits, H, P, kv_dtype):
    inp = W.small_case(seed=13, batch=3, num_heads=H, head_size=576, kv_lora_rank=512,
                       page_size=P, seq_lens=(37, 100, 5), extra_pages=4, table_pad=3,
                       kv_dtype=kv_dtype, k_scale=FP8_SCALE if kv_dtype == W.FP8_E4M3 else 1.0)
    o, lse = run_gpu(mla, inp, splits, mode)
    o2, lse2 = run_gpu(mla, W.poison_unreferenced(inp), splits, mode)
    assert np.all(np.isfinite(o2)) and np.array_equal(o, o2) and np.array_equal(lse, lse2)


# ---------------------------------------------------------------- determinism

def test_single_split_is_reproducible_and_batch_invariant(mla):
    inp = W.small_case(seed=17, batch=6, num_heads=128, head_size=576, kv_lora_rank=512,
                       page_size=64, seq_lens=(100, 1000, 37, 513, 64, 2000))
    o1, l1 = run_gpu(mla, inp, 1, 0)
    o2, l2 = run_gpu(mla, inp, 1, 0)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    order = [4, 1, 5, 0]
    o3, l3 = run_gpu(mla, W.subset(inp, order), 1, 0)
    assert np.array_equal(o3, o1[order]) and np.array_equal(l3, l1[order])
    o4, l4 = run_gpu(mla, W.subset(inp, [1]), 1, 0)
    assert np.array_equal(o4[0], o1[1]) and np.array_equal(l4[0], l1[1])


@pytest.mark.parametrize("kv_dtype", [W.BF16, W.FP8_E4M3])
@pytest.mark.parametrize("splits", [4, 16])
def test_fixed_split_count_is_reproducible_and_batch_invariant(mla, kv_dtype, splits):
    """The per-sequence split mode with a fixed split count: a sequence's
    segments depend only on its own length and S, each is reduced in a fixed
    tile order and stage 2 merges them in a fixed order, so its result is the
    same bits in any batch (a deterministic mode that still spreads a long
    sequence over S workgroups)."""
    inp = W.small_case(seed=23, batch=6, num_heads=128, head_size=576, kv_lora_rank=512,
                       page_size=64, seq_lens=(100, 1000, 37, 513, 64, 2000), kv_dtype=kv_dtype,
                       k_scale=0.05 if kv_dtype == W.FP8_E4M3 else 1.0)
    o1, l1 = run_gpu(mla, inp, splits, 0)
    o2, l2 = run_gpu(mla, inp, splits, 0)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    order = [4, 1, 5, 0]
    o3, l3 = run_gpu(mla, W.subset(inp, order), splits, 0)
    assert np.array_equal(o3, o1[order]) and np.array_equal(l3, l1[order])
    o4, l4 = run_gpu(mla, W.subset(inp, [5]), splits, 0)
    assert np.array_equal(o4[0], o1[5]) and np.array_equal(l4[0], l1[5])
    ro, rl = ref(inp)
    assert_close(inp, o1, l1, ro, rl, f"{kv_dtype} S={splits}", rounding_slack=True)
    o5, l5 = run_gpu(mla, inp, splits, 0, o_dtype=torch.float32)
    assert_close(inp, o5, l5, ro, rl, f"{kv_dtype} S={splits} fp32 output")


def test_split_results_are_reproducible(mla):
    inp = W.small_case(seed=19, batch=4, num_heads=128, head_size=576, kv_lora_rank=512,
                       page_size=64, seq_lens=(100, 3000, 37, 777))
    a = run_gpu(mla, inp, 7, 1)
    b = run_gpu(mla, inp, 7, 1)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---------------------------------------------------------------- full-size configs

@pytest.mark.parametrize("name", ["dsv3", "skewed", "h320", "fp8"])
def test_full_size_configs(mla, name):
    """Every sequence of each full-size workload against the oracle, in the
    planner's launch configuration, at the pages' split count per sequence and
    in the single-split (deterministic) mode; fp32 output at the stated
    tolerance, bf16 output at the same tolerance (these batches hold only
    sequences of 256 positions or more, where |o| stays far below 1 and the
    final bf16 rounding is below 2^-9)."""
    inp = W.generate(name)
    w = inp.workload
    dev_inputs = to_dev(inp)
    ro, rl = ref(inp)
    max_len, tot = int(inp.seq_lens.max()), int(inp.seq_lens.sum())
    shape = mla.shape_of(*dev_inputs[:2], dev_inputs[2])
    print(f"{name}: B={w.batch} H={w.num_heads} D={w.head_size} {w.kv_dtype} "
          f"tokens={tot}", flush=True)
    mode, units, _ = mla.mla_plan(shape, max_len, tot, 256)
    runs = [(mode, units)] + [(0, s) for s in w.parity_splits]
    if (0, 1) not in runs:
        runs.append((0, 1))
    for mode, splits in runs:
        for o_dtype in (torch.float32, torch.bfloat16):
            o, lse = run_gpu(mla, inp, splits, mode, o_dtype=o_dtype, dev_inputs=dev_inputs)
            assert_close(inp, o, lse, ro, rl, f"{name} mode={mode} S={splits} o={o_dtype}")
