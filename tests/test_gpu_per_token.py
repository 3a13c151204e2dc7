"""GPU parity of decode over per-token quantised caches: each row holds
head_size codes (e4m3fn, signed int8, or signed int4 packed two per byte) and
its own float32 scale inline in a 16-byte pad (Triton MLA page, key files: the
per-token-head modes, fp8, int8 and int4 among them, pad the cache's head_dim
to hold an inline scale).  The HIP path runs through the C ABI (ctypes
binding, kv dtype MLA_FP8_E4M3_PER_TOKEN, MLA_INT8_PER_TOKEN or
MLA_INT4_PER_TOKEN) and is compared with the float64 oracle, which decodes
every row to code * scale of that token.

Tolerances (max-abs) are those of the per-tensor fp8 cache: o 3e-2, lse 3e-3.
Where the scale of each row is exact in bf16 and a sequence has a single
position, o must be that row's values exactly.
"""
import numpy as np
import pytest

import oracle
import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL_O, TOL_LSE = 3e-2, 3e-3
PAD = W.PER_TOKEN_PAD
DTYPES = [W.FP8_PER_TOKEN, W.INT8_PER_TOKEN, W.INT4_PER_TOKEN]


def code_bytes(dt, D):
    return D // 2 if dt == W.INT4_PER_TOKEN else D


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
    kv = torch.from_numpy(np.ascontiguousarray(inp.kv_bits)).to(dev)  # uint8 rows
    bt = torch.from_numpy(np.ascontiguousarray(inp.block_table)).to(dev)
    sl = torch.from_numpy(np.ascontiguousarray(inp.seq_lens)).to(dev)
    return q, kv, bt, sl


def run_gpu(mla, inp, splits, mode, o_dtype=None, dev_inputs=None, k_scale=1.0):
    w = inp.workload
    q, kv, bt, sl = dev_inputs or to_dev(inp)
    print(f"[per-token] {w.kv_dtype} B={w.batch} H={w.num_heads} D={w.head_size} "
          f"P={w.page_size} q_len={w.q_len} mode={mode} S={splits}", flush=True)
    o, lse = mla.mla_decode(q, kv, bt, sl, w.scale, w.page_size, k_scale, splits,
                            split_mode=mode, o_dtype=o_dtype or torch.bfloat16,
                            kv_dtype=w.kv_dtype)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def ref(inp, batches=None):
    w = inp.workload
    fn = oracle.decode_mtp if w.q_len > 1 else oracle.decode
    return fn(inp.q_bits, inp.kv_bits, inp.block_table, inp.seq_lens, scale=w.scale,
              k_scale=w.k_scale, kv_dtype=w.kv_dtype, kv_lora_rank=w.kv_lora_rank,
              batches=batches)


def bf16_half_ulp(x):
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(ax)) - 8)


def assert_close(o, lse, ro, rl, empty, label, rounding_slack=False):
    if empty.any():
        assert np.all(o[empty] == 0) and np.all(np.isneginf(lse[empty])), label
    live = ~empty
    assert np.all(np.isfinite(o[live])) and np.all(np.isfinite(lse[live])), label
    err = np.abs(o[live] - ro[live])
    if rounding_slack:
        err = err - bf16_half_ulp(ro[live])
    do = err.max() if live.any() else 0.0
    dl = np.abs(lse[live] - rl[live]).max() if live.any() else 0.0
    print(f"{label}: max|do|={do:.3e} max|dlse|={dl:.3e}", flush=True)
    assert do <= TOL_O and dl <= TOL_LSE, (label, do, dl)


def case(seed, H, D, P, sl, dt=W.FP8_PER_TOKEN, **kw):
    return W.small_case(seed=seed, batch=len(sl), num_heads=H, head_size=D, kv_lora_rank=D - 64,
                        page_size=P, seq_lens=sl, kv_dtype=dt, **kw)


def set_scales(inp, scales):
    """Replace the inline scale of every row by scales [NB, P] (float32)."""
    kv = inp.kv_bits.copy()
    cb = code_bytes(inp.workload.kv_dtype, inp.workload.head_size)
    kv[..., cb:cb + 4] = np.ascontiguousarray(scales, dtype="<f4").view(np.uint8).reshape(
        scales.shape + (4,))
    inp.kv_bits = kv
    return inp


CASES = [
    # (H, D, P, seq_lens): short and ragged tails, every head tiling, both head sizes
    (16, 576, 16, (1, 31, 32, 33, 64, 65, 100, 257)),
    (32, 576, 32, (5, 96, 97, 300)),
    (64, 576, 48, (1, 47, 48, 49, 500)),
    (128, 576, 64, (1, 63, 64, 65, 700, 1031)),
    (48, 576, 16, (3, 129, 40)),
    (16, 320, 16, (1, 31, 33, 250, 513)),
    (128, 320, 32, (17, 95, 333)),
    (256, 576, 64, (77, 129)),
    (96, 576, 32, (5, 97, 300)),
    (80, 576, 16, (1, 33, 129)),
    (192, 576, 64, (64, 65, 400)),
]


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("c", range(len(CASES)))
@pytest.mark.parametrize("mode,splits", [(0, 1), (0, 3), (1, 4), (1, 37)])
def test_ragged_cases(mla, c, mode, splits, dt):
    H, D, P, sl = CASES[c]
    inp = case(300 + c, H, D, P, sl, dt, table_pad=1)
    ro, rl = ref(inp)
    empty = np.asarray(inp.seq_lens) == 0
    label = f"{dt} case{c} H={H} D={D} P={P} mode={mode} S={splits}"
    o, lse = run_gpu(mla, inp, splits, mode, o_dtype=torch.float32)
    assert_close(o, lse, ro, rl, empty, label + " o=f32")
    o, lse = run_gpu(mla, inp, splits, mode)
    assert_close(o, lse, ro, rl, empty, label + " o=bf16", rounding_slack=True)


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("H,D", [(16, 576), (128, 576), (32, 320), (48, 320)])
@pytest.mark.parametrize("mode,splits", [(0, 1), (1, 5)])
def test_scales_differ_from_token_to_token(mla, H, D, mode, splits, dt):
    """Rows of one page carry scales 2^k apart (k in -2..1, seeded): a scale
    applied to the wrong position, or one scale for a whole tile, moves the
    scores by factors of 2 and fails the tolerance."""
    sl = (45, 200, 33)
    inp = case(41, H, D, 16, sl, dt, extra_pages=2)
    rng = np.random.default_rng(42)
    cb = code_bytes(dt, D)
    D2 = cb + PAD
    base = inp.kv_bits[..., cb:cb + 4].copy().view("<f4")[..., 0]
    mult = np.exp2(rng.integers(-2, 2, size=base.shape)).astype(np.float32)
    set_scales(inp, base * mult)
    assert inp.kv_bits.shape[-1] == D2
    ro, rl = ref(inp)
    o, lse = run_gpu(mla, inp, splits, mode, o_dtype=torch.float32)
    assert_close(o, lse, ro, rl, np.zeros(len(sl), bool), f"{dt} scales H={H} D={D} S={splits}")


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("H,D", [(16, 576), (32, 576), (128, 576), (48, 320), (128, 320)])
@pytest.mark.parametrize("mode,splits", [(0, 1), (1, 2)])
def test_one_position_returns_the_scaled_row(mla, H, D, mode, splits, dt):
    """A single position has softmax weight 1, so o is its kv_c codes times
    its scale.  Each sequence's row runs through the finite code bytes (254
    e4m3fn, 256 int8 or 256 pairs of int4 codes, as far as the row holds
    them) and has its own scale with 2 significant bits (exact in bf16), so
    every product is exact in fp32.  The kernel's weight of the position is
    exp2 of a fused multiply-add residual, 1 to within an ulp, so o must be
    the row to within 2^-22 relative (a wrong code or scale is off by far
    more)."""
    Dv, P, B = D - 64, 16, 3
    rng = np.random.default_rng(51)
    if dt == W.FP8_PER_TOKEN:
        finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    else:
        finite = np.arange(256, dtype=np.uint8)
    nb = B + 2
    cb = code_bytes(dt, D)
    kv = np.zeros((nb, P, cb + PAD), dtype=np.uint8)
    kv[..., :cb] = rng.choice(finite, size=(nb, P, cb))
    scales = np.exp2(rng.integers(-8, 3, size=(nb, P))).astype(np.float32) * np.float32(0.75)
    n = min(finite.size, cb)
    for b in range(B):
        kv[b + 1, 0, :n] = np.roll(finite, 29 * b)[:n]
    kv[..., cb:cb + 4] = scales.astype("<f4").view(np.uint8).reshape(nb, P, 4)
    table = np.array([[b + 1, 0] for b in range(B)], dtype=np.int32)
    q = W.f32_to_bf16_bits(rng.standard_normal((B, H, D), dtype=np.float32) * 0.1)
    w = W.Workload(name="pt-codes", seed=51, batch=B, num_heads=H, head_size=D,
                   kv_lora_rank=Dv, page_size=P, num_blocks=nb, kv_dtype=dt,
                   k_scale=1.0, scale=W.DSV3_SCALE, seq_lens_fixed=(1,) * B)
    inp = W.DecodeInputs(workload=w, q_bits=q, kv_bits=kv, block_table=table,
                         seq_lens=np.ones(B, dtype=np.int32))
    ro, rl = ref(inp)
    o32, l32 = run_gpu(mla, inp, splits, mode, o_dtype=torch.float32)
    assert np.all(np.abs(o32 - ro) <= 2.0 ** -22 * np.abs(ro)), np.abs(o32 - ro).max()
    assert np.abs(l32 - rl).max() <= 1e-4 * max(1.0, np.abs(rl).max())


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("H,D", [(16, 576), (128, 576), (32, 320)])
@pytest.mark.parametrize("mode,splits", [(0, 1), (1, 5)])
def test_zero_and_subnormal_scales(mla, H, D, mode, splits, dt):
    """Rows whose scale is 0 (value 0 whatever their codes, but a full
    softmax weight exp(0 - max)) or subnormal (1e-40) sit among ordinary rows:
    the normaliser must count them with their weight p, which the kernel's
    reciprocal-of-scale correction leaves out for such scales."""
    sl = (70, 200, 33)
    inp = case(71, H, D, 16, sl, dt, extra_pages=2)
    rng = np.random.default_rng(72)
    cb = code_bytes(dt, D)
    base = inp.kv_bits[..., cb:cb + 4].copy().view("<f4")[..., 0]
    pick = rng.random(base.shape)
    scales = np.where(pick < 0.2, np.float32(0.0),
                      np.where(pick < 0.3, np.float32(1e-40), base)).astype(np.float32)
    set_scales(inp, scales)
    ro, rl = ref(inp)
    o, lse = run_gpu(mla, inp, splits, mode, o_dtype=torch.float32)
    assert_close(o, lse, ro, rl, np.zeros(len(sl), bool),
                 f"{dt} zero/subnormal scales H={H} D={D} S={splits}")


@pytest.mark.parametrize("dt", DTYPES)
def test_k_scale_does_not_apply(mla, dt):
    inp = case(61, 128, 576, 64, (100, 513), dt)
    a = run_gpu(mla, inp, 3, 1, k_scale=1.0)
    b = run_gpu(mla, inp, 3, 1, k_scale=7.0)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("mode,splits", [(0, 1), (0, 4), (1, 3)])
def test_empty_sequences(mla, mode, splits, dt):
    inp = case(63, 16, 576, 16, (0, 50, 0, 1, 0), dt)
    ro, rl = ref(inp)
    empty = np.asarray(inp.seq_lens) == 0
    o, lse = run_gpu(mla, inp, splits, mode, o_dtype=torch.float32)
    assert_close(o, lse, ro, rl, empty, f"pt empty S={splits} o=f32")
    o, lse = run_gpu(mla, inp, splits, mode)
    assert_close(o, lse, ro, rl, empty, f"pt empty S={splits} o=bf16", rounding_slack=True)


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("mode,splits", [(0, 1), (0, 4), (1, 6)])
def test_page_permutation_is_bitwise_invariant(mla, mode, splits, dt):
    inp = case(65, 128, 576, 16, (37, 100, 64, 257), dt, extra_pages=9)
    o, lse = run_gpu(mla, inp, splits, mode)
    o2, lse2 = run_gpu(mla, W.permute_pages(inp, seed=5), splits, mode)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("mode,splits", [(0, 1), (1, 3)])
@pytest.mark.parametrize("H,P,D", [(128, 64, 576), (16, 16, 576), (32, 16, 320)])
def test_poisoned_unreferenced_slots(mla, mode, splits, H, P, D, dt):
    """Unreferenced rows get 0x7F bytes: NaN codes (fp8) and a NaN scale; the
    output must not change by a bit."""
    inp = case(67, H, D, P, (37, 100, 5), dt, extra_pages=4, table_pad=3)
    o, lse = run_gpu(mla, inp, splits, mode)
    o2, lse2 = run_gpu(mla, W.poison_unreferenced(inp), splits, mode)
    assert np.all(np.isfinite(o2)) and np.array_equal(o, o2) and np.array_equal(lse, lse2)


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("q_len", [2, 5])
def test_multi_token_decode(mla, q_len, dt):
    sl = (1, 3, 40, 300)
    inp = case(69, 128, 576, 64, sl, dt, q_len=q_len)
    ro, rl = ref(inp)
    o, lse = run_gpu(mla, inp, 4, 1, o_dtype=torch.float32)
    vis = np.array([[oracle.visible_keys(int(n), q_len, i) for i in range(q_len)] for n in sl])
    empty = np.repeat((vis == 0)[:, :, None], 128, axis=2)
    assert_close(o, lse, ro, rl, empty, f"pt mtp q_len={q_len}")


@pytest.mark.parametrize("name", ["fp8_pt", "int8_pt", "int4_pt"])
def test_full_size_per_token(mla, name):
    """The fp8_pt / int8_pt / int4_pt workloads (B=64, H=128, D=576, P=64, lengths
    1024..8192) at the planner's launch configuration, at per-sequence splits
    and in the single-split mode, every sequence compared with the oracle:
    fp32 output at the plain tolerances, bf16 output beyond its final rounding."""
    inp = W.generate(name)
    w = inp.workload
    dev_inputs = to_dev(inp)
    sl = np.asarray(inp.seq_lens)
    ro, rl = ref(inp)
    none_empty = np.zeros(len(sl), bool)
    shape = mla.shape_of(dev_inputs[0], dev_inputs[1], dev_inputs[2], kv_dtype=w.kv_dtype)
    mode, units, _ = mla.mla_plan(shape, int(sl.max()), int(sl.sum()), 256)
    for mode, splits in [(mode, units)] + [(0, s) for s in w.parity_splits]:
        o, lse = run_gpu(mla, inp, splits, mode, o_dtype=torch.float32, dev_inputs=dev_inputs)
        assert_close(o, lse, ro, rl, none_empty, f"{name} mode={mode} S={splits} o=f32")
        o, lse = run_gpu(mla, inp, splits, mode, dev_inputs=dev_inputs)
        assert_close(o, lse, ro, rl, none_empty, f"{name} mode={mode} S={splits} o=bf16",
                     rounding_slack=True)


@pytest.mark.parametrize("dt", DTYPES)
@pytest.mark.parametrize("P", [512, 1024])
@pytest.mark.parametrize("mode,splits", [(0, 1), (0, 5), (1, 9)])
def test_large_pages(mla, P, dt, mode, splits):
    """Pages of 512 and 1024 rows: in-page offsets beyond 64 K rows' bytes of
    a 16-row run, and sequences that end one row into a page."""
    sl = (1, P - 1, P + 1, 3 * P + 5)
    inp = case(530 + P // 512, 128, 576, P, sl, dt, extra_pages=1)
    ro, rl = ref(inp)
    o, lse = run_gpu(mla, inp, splits, mode, o_dtype=torch.float32)
    assert_close(o, lse, ro, rl, np.zeros(len(sl), bool), f"{dt} P={P} mode={mode} S={splits}")
