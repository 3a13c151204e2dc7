"""GPU parity at the edges of the accepted sizes, through the C ABI:
the most query tokens per sequence (MLA_MAX_Q_LEN), large pages, 512 heads
(four head chunks per work unit), a thousand short sequences, the most
split units (MLA_MAX_KV_SPLITS, nearly all of them owning no tile), one very
long sequence, and cache pools past 4 GB (64-bit page addressing, bf16 and
per-token rows, checked bitwise against the same pages in a small pool).  Every case runs twice:
with fp32 output, checked at the plain tolerances (o 1e-2, lse 1e-3), and with bf16 output, checked
at the same tolerances plus the final bf16 rounding of each value (half a bf16 ulp of the exact
result).  Every sequence of every batch is compared.
"""
import numpy as np
import pytest

import oracle
import workloads as W

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import mla_paged_latent_decode_amd as m
    m.load_library()
    return m


def to_dev(inp):
    q = torch.from_numpy(inp.q_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    kv = torch.from_numpy(inp.kv_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    bt = torch.from_numpy(np.ascontiguousarray(inp.block_table)).to(DEV)
    sl = torch.from_numpy(np.ascontiguousarray(inp.seq_lens)).to(DEV)
    return q, kv, bt, sl


def ref(inp, batches=None):
    w = inp.workload
    fn = oracle.decode_mtp if w.q_len > 1 else oracle.decode
    return fn(inp.q_bits, inp.kv_bits, inp.block_table, inp.seq_lens, scale=w.scale,
              k_scale=w.k_scale, kv_dtype=w.kv_dtype, kv_lora_rank=w.kv_lora_rank,
              batches=batches)


def half_ulp_bf16(x):
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(ax)) - 8)


def check(res, ro, rl, label, tol=(1e-2, 1e-3)):
    """res = {"f32": (o, lse), "bf16": (o, lse)} from run(): fp32 output at the
    plain tolerances, bf16 output at the same plus its final rounding."""
    to, tl = tol
    for kind, (o, lse) in res.items():
        empty = np.isneginf(rl)
        assert np.all(o[empty] == 0) and np.all(np.isneginf(lse[empty])), (label, kind)
        live = ~empty
        assert np.all(np.isfinite(o[live])) and np.all(np.isfinite(lse[live])), (label, kind)
        err = np.abs(o[live] - ro[live])
        if kind == "bf16":
            err = err - half_ulp_bf16(ro[live])
        do = err.max()
        dl = np.abs(lse[live] - rl[live]).max()
        print(f"{label} o={kind}: max|do|{' beyond rounding' if kind == 'bf16' else ''}="
              f"{do:.3e} max|dlse|={dl:.3e}", flush=True)
        assert do <= to and dl <= tl, (label, kind, do, dl)


def run(mla, inp, splits=None, mode=None, dev_inputs=None):
    """The decode with fp32 and with bf16 output: {"f32": (o, lse), "bf16": (o, lse)}."""
    w = inp.workload
    q, kv, bt, sl = dev_inputs or to_dev(inp)
    print(f"[limits] {w.name} B={len(inp.seq_lens)} H={w.num_heads} D={w.head_size} "
          f"P={w.page_size} q_len={w.q_len} mode={mode} S={splits}", flush=True)
    res = {}
    for kind, dt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        if splits is None:
            o, lse = mla.mla_decode(q, kv, bt, sl, w.scale, w.page_size, w.k_scale, num_cus=256,
                                    o_dtype=dt)
        else:
            o, lse = mla.mla_decode(q, kv, bt, sl, w.scale, w.page_size, w.k_scale, splits,
                                    split_mode=mode, o_dtype=dt)
        torch.cuda.synchronize()
        res[kind] = (o.float().cpu().numpy().astype(np.float64),
                     lse.cpu().numpy().astype(np.float64))
    return res


@pytest.mark.parametrize("H", [16, 128])
def test_most_query_tokens(mla, H):
    """q_len = MLA_MAX_Q_LEN (16): 16 x H rows per sequence, with sequences
    shorter than q_len (their first rows see nothing)."""
    ql = mla.MLA_MAX_Q_LEN
    sl = (3, 16, 17, 40, 300)
    inp = W.small_case(seed=500 + H, batch=len(sl), num_heads=H, head_size=576, kv_lora_rank=512,
                       page_size=16, seq_lens=sl, q_len=ql)
    ro, rl = ref(inp)
    for mode, splits in ((0, 1), (1, 7), (None, None)):
        check(run(mla, inp, splits, mode), ro, rl, f"q_len {ql} H={H} mode={mode} S={splits}")


@pytest.mark.parametrize("P", [512, 1024])
def test_large_pages(mla, P):
    sl = (1, P - 1, P, P + 1, 3 * P + 5)
    inp = W.small_case(seed=510 + P, batch=len(sl), num_heads=128, head_size=576,
                       kv_lora_rank=512, page_size=P, seq_lens=sl, extra_pages=1)
    ro, rl = ref(inp)
    for mode, splits in ((0, 1), (0, 5), (1, 9), (None, None)):
        check(run(mla, inp, splits, mode), ro, rl, f"P={P} mode={mode} S={splits}")


def test_512_heads(mla):
    sl = (70, 1100, 5)
    inp = W.small_case(seed=520, batch=len(sl), num_heads=512, head_size=576, kv_lora_rank=512,
                       page_size=64, seq_lens=sl)
    ro, rl = ref(inp)
    for mode, splits in ((0, 1), (0, 4), (1, 11), (None, None)):
        check(run(mla, inp, splits, mode), ro, rl, f"H=512 mode={mode} S={splits}")


def test_a_thousand_short_sequences(mla):
    rng = np.random.default_rng(530)
    sl = tuple(int(x) for x in rng.integers(0, 65, size=1024))
    inp = W.small_case(seed=530, batch=len(sl), num_heads=16, head_size=320, kv_lora_rank=256,
                       page_size=16, seq_lens=sl)
    ro, rl = ref(inp)  # every one of the 1024 sequences
    for mode, splits in ((0, 1), (0, 3), (None, None)):
        check(run(mla, inp, splits, mode), ro, rl, f"B=1024 mode={mode} S={splits}")


def test_most_split_units(mla):
    """MLA_MAX_KV_SPLITS balanced units over a few hundred tiles: almost every
    unit owns no tile and writes nothing; stage 2 must skip those slots."""
    sl = (37, 1000, 2)
    inp = W.small_case(seed=540, batch=len(sl), num_heads=16, head_size=576, kv_lora_rank=512,
                       page_size=16, seq_lens=sl)
    ro, rl = ref(inp)
    check(run(mla, inp, mla.MLA_MAX_KV_SPLITS, mla.SPLIT_BALANCED), ro, rl, "U=65536")
    check(run(mla, inp, 4096, mla.SPLIT_PER_SEQUENCE), ro, rl, "per-sequence S=4096")


def test_one_very_long_sequence(mla):
    """262144 positions in one sequence (16 heads) next to a short one."""
    sl = (262144, 77)
    inp = W.small_case(seed=550, batch=len(sl), num_heads=16, head_size=576, kv_lora_rank=512,
                       page_size=64, seq_lens=sl)
    ro, rl = ref(inp)
    for mode, splits in ((0, 1), (0, 64), (None, None)):
        check(run(mla, inp, splits, mode), ro, rl, f"n=262144 mode={mode} S={splits}")


def test_pool_past_4_gb_is_addressed_exactly(mla):
    """The same pages placed at the top of a 5 GB pool (byte offsets past
    2^32) give bitwise the same result as in a small pool."""
    sl = (100, 1031, 37)
    inp = W.small_case(seed=560, batch=len(sl), num_heads=128, head_size=576, kv_lora_rank=512,
                       page_size=16, seq_lens=sl, extra_pages=0)
    q, kv, bt, sl_d = to_dev(inp)
    res = run(mla, inp, 5, mla.SPLIT_BALANCED, dev_inputs=(q, kv, bt, sl_d))
    check(res, *ref(inp), "pool 5 GB (small-pool run)")
    small = res["bf16"]
    nb_small = kv.shape[0]
    page_bytes = 16 * 576 * 2
    nb_big = (5 << 30) // page_bytes + nb_small
    big = torch.empty((nb_big, 16, 576), dtype=torch.bfloat16, device=DEV)
    big[-nb_small:] = kv  # page p of the small pool is page nb_big - nb_small + p
    bt_big = (bt + (nb_big - nb_small)).to(torch.int32)
    assert int(bt_big.max()) * page_bytes > (1 << 32)
    w = inp.workload
    o, lse = mla.mla_decode(q, big, bt_big, sl_d, w.scale, w.page_size, w.k_scale, 5,
                            split_mode=mla.SPLIT_BALANCED)
    torch.cuda.synchronize()
    o = o.float().cpu().numpy().astype(np.float64)
    lse = lse.cpu().numpy().astype(np.float64)
    del big
    assert np.array_equal(o, small[0]) and np.array_equal(lse, small[1])


@pytest.mark.parametrize("dt", [W.FP8_PER_TOKEN, W.INT4_PER_TOKEN])
def test_per_token_pool_past_4_gb_is_addressed_exactly(mla, dt):
    """Per-token rows (592 bytes for fp8 codes, 304 for int4) at the top of
    a 5 GB pool give bitwise the result of the same pages in a small pool."""
    sl = (100, 1031, 37)
    inp = W.small_case(seed=561, batch=len(sl), num_heads=128, head_size=576, kv_lora_rank=512,
                       page_size=16, seq_lens=sl, extra_pages=0, kv_dtype=dt)
    w = inp.workload
    q = torch.from_numpy(inp.q_bits.view(np.int16)).view(torch.bfloat16).to(DEV)
    kv = torch.from_numpy(np.ascontiguousarray(inp.kv_bits)).to(DEV)  # uint8 rows
    bt = torch.from_numpy(np.ascontiguousarray(inp.block_table)).to(DEV)
    sl_d = torch.from_numpy(np.ascontiguousarray(inp.seq_lens)).to(DEV)
    print(f"[limits] per-token {dt} pool past 4 GB", flush=True)
    o_s, l_s = mla.mla_decode(q, kv, bt, sl_d, w.scale, w.page_size, 1.0, 5,
                              split_mode=mla.SPLIT_BALANCED, kv_dtype=dt)
    nb_small, row = kv.shape[0], kv.shape[2]
    page_bytes = 16 * row
    nb_big = (5 << 30) // page_bytes + nb_small
    big = torch.empty((nb_big, 16, row), dtype=torch.uint8, device=DEV)
    big[-nb_small:] = kv
    bt_big = (bt + (nb_big - nb_small)).to(torch.int32)
    assert int(bt_big.max()) * page_bytes > (1 << 32)
    o_b, l_b = mla.mla_decode(q, big, bt_big, sl_d, w.scale, w.page_size, 1.0, 5,
                              split_mode=mla.SPLIT_BALANCED, kv_dtype=dt)
    torch.cuda.synchronize()
    del big
    assert torch.equal(o_s, o_b) and torch.equal(l_s, l_b)
    # quantised-cache tolerances (o 3e-2, lse 3e-3): fp32 output plain, bf16 output
    # beyond its final rounding
    o_f, l_f = mla.mla_decode(q, kv, bt, sl_d, w.scale, w.page_size, 1.0, 5,
                              split_mode=mla.SPLIT_BALANCED, kv_dtype=dt, o_dtype=torch.float32)
    torch.cuda.synchronize()
    res = {"f32": (o_f.cpu().numpy().astype(np.float64), l_f.cpu().numpy().astype(np.float64)),
           "bf16": (o_b.float().cpu().numpy().astype(np.float64),
                    l_b.cpu().numpy().astype(np.float64))}
    check(res, *ref(inp), f"per-token {dt} pool 5 GB", tol=(3e-2, 3e-3))
