"""CPU tests of libmla's host side: the library loads, exports every function
include/mla.h declares, and its planner, workspace sizing and argument checks
behave as documented.  No GPU work is enqueued: every mla_decode call here is
rejected by the host checks before anything reaches HIP."""
import ctypes
import json
import os
import re

import pytest

import mla_paged_latent_decode_amd as mla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mla.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "pages_worked_examples.json")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = mla.load_library()
    names = header_functions()
    assert {"mla_decode", "mla_plan", "mla_workspace_size", "mla_status_string",
            "mla_pages_split_count"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_probe_library_exports_its_probes():
    # the measured-ceiling probes bench.py --peaks calls (mla_peaks.hip)
    from mla_paged_latent_decode_amd import _build
    lib = ctypes.CDLL(_build.PEAKS_LIB_PATH)
    for n in ("mla_peak_stream", "mla_peak_mfma", "mla_peak_mfma_chain", "mla_peak_lds",
              "mla_peak_tileloop"):
        assert hasattr(lib, n), n


def test_status_strings():
    for code in range(12):
        s = mla.mla_status_string(code)
        assert s and "unknown" not in s
    assert "unknown" in mla.mla_status_string(99)


def test_pages_split_count_matches_worked_cases():
    g = json.load(open(GOLDEN))["split_count_rule"]
    for c in g["cases"]:
        assert mla.mla_pages_split_count(c["max_seq_len"], c["sm_count"]) == c["splits"]
    assert mla.mla_pages_split_count(100, 0) == 0


def shape(**kw):
    d = dict(batch=64, num_heads=128, head_size=576, page_size=64, num_blocks=8192,
             max_blocks_per_seq=128)
    d.update(kw)
    return mla.make_shape(**d)


def test_workspace_sizes():
    s = shape()
    assert mla.mla_workspace_size(s, mla.SPLIT_PER_SEQUENCE, 1) == 0
    # fp16 partial rows, an {lse, row scale} float pair per row, then one
    # {first slot, count} int pair per sequence (rounded up to 256 bytes)
    per = 64 * 16 * 128 * 512 * 2
    got = mla.mla_workspace_size(s, mla.SPLIT_PER_SEQUENCE, 16)
    ls_bytes = 64 * 16 * 128 * 8
    seg_bytes = 512  # 64 * 8
    assert got == per + ls_bytes + seg_bytes  # every part a 256-byte multiple here
    bal = mla.mla_workspace_size(s, mla.SPLIT_BALANCED, 256)
    assert bal == (256 + 64) * 128 * (512 * 2 + 8) + seg_bytes
    assert mla.mla_workspace_size(s, 7, 4) == 0
    assert mla.mla_workspace_size(s, mla.SPLIT_BALANCED, 0) == 0
    assert mla.mla_workspace_size(shape(head_size=400), mla.SPLIT_BALANCED, 4) == 0


def test_plan_deterministic_and_balanced():
    s = shape()
    assert mla.mla_plan(s, 8192, 0, 256, deterministic=True) == (mla.SPLIT_PER_SEQUENCE, 1, 0)
    mode, units, ws = mla.mla_plan(s, 8192, 64 * 4608, 256)
    assert mode == mla.SPLIT_BALANCED and units == 256
    assert ws == mla.mla_workspace_size(s, mode, units)
    # tiny batches get few units (at least 4 tiles each)
    t = shape(batch=2, num_heads=16, page_size=16, num_blocks=16, max_blocks_per_seq=7)
    mode, units, ws = mla.mla_plan(t, 100, 137, 256)
    assert mode == mla.SPLIT_BALANCED and 1 <= units <= 2
    # more head chunks -> fewer units per chunk
    big = shape(num_heads=256)
    assert mla.mla_plan(big, 8192, 64 * 4608, 256)[1] == 128


@pytest.mark.parametrize("kw,exc", [
    (dict(head_size=400), ValueError),
    (dict(head_size=576, kv_lora_rank=448), ValueError),
    (dict(page_size=24), ValueError),
    (dict(page_size=0), ValueError),
    (dict(q_dtype=mla.MLA_FP8_E4M3), NotImplementedError),
    (dict(o_dtype=mla.MLA_FP8_E4M3), NotImplementedError),
    (dict(num_heads=24), mla.MlaError),
    (dict(batch=0), mla.MlaError),
    (dict(num_blocks=0), mla.MlaError),
])
def test_plan_rejects_bad_shapes(kw, exc):
    with pytest.raises(exc):
        mla.mla_plan(shape(**kw), 1024, 0, 256)


def _decode_raw(s, *, q=256, kv=256, bt=256, sl=256, scale=0.07, page=None, k_scale=1.0,
                splits=1, mode=0, o=256, lse=256, ws=None, ws_bytes=0):
    lib = mla.load_library()
    return lib.mla_decode(ctypes.byref(s), q, kv, bt, sl, scale,
                          s.page_size if page is None else page, k_scale, splits, mode, o, lse,
                          ws, ws_bytes, None)


def test_decode_argument_checks_fail_before_launch():
    s = shape()
    assert _decode_raw(s, q=None) == mla.MLA_ERR_NULL
    assert _decode_raw(s, lse=None) == mla.MLA_ERR_NULL
    assert _decode_raw(s, page=16) == mla.MLA_ERR_PAGE_SIZE
    assert _decode_raw(shape(head_size=320, kv_lora_rank=512)) == mla.MLA_ERR_HEAD_SIZE
    assert _decode_raw(s, splits=0) == mla.MLA_ERR_SPLITS
    assert _decode_raw(s, mode=5) == mla.MLA_ERR_SPLITS
    assert _decode_raw(s, splits=mla.MLA_MAX_KV_SPLITS + 1) == mla.MLA_ERR_SPLITS
    assert _decode_raw(s, scale=float("nan")) == mla.MLA_ERR_ARGUMENT
    assert _decode_raw(s, scale=-1.0) == mla.MLA_ERR_ARGUMENT
    fp8 = shape(kv_dtype=mla.MLA_FP8_E4M3)
    assert _decode_raw(fp8, k_scale=0.0) == mla.MLA_ERR_ARGUMENT
    assert _decode_raw(fp8, k_scale=float("inf")) == mla.MLA_ERR_ARGUMENT
    assert _decode_raw(s, q=258) == mla.MLA_ERR_ARGUMENT  # misaligned
    # split layouts that need a workspace refuse a missing or short one
    need = mla.mla_workspace_size(s, 0, 16)
    assert _decode_raw(s, splits=16) == mla.MLA_ERR_WORKSPACE
    assert _decode_raw(s, splits=16, ws=256, ws_bytes=need - 1) == mla.MLA_ERR_WORKSPACE
    assert _decode_raw(s, splits=16, mode=1, ws=256, ws_bytes=10) == mla.MLA_ERR_WORKSPACE
    assert _decode_raw(s, splits=16, ws=264, ws_bytes=need) == mla.MLA_ERR_ARGUMENT


def test_size_caps_are_refused_before_launch():
    # heads above MLA_MAX_ROWS, a batch above MLA_MAX_BATCH
    with pytest.raises(mla.MlaError):
        mla.mla_plan(shape(num_heads=mla.MLA_MAX_ROWS + 16), 1024, 0, 256)
    with pytest.raises(mla.MlaError):
        mla.mla_plan(shape(batch=mla.MLA_MAX_BATCH + 1, max_blocks_per_seq=1), 64, 0, 256)
    assert mla.mla_plan(shape(num_heads=mla.MLA_MAX_ROWS), 1024, 0, 256)[0] == mla.SPLIT_BALANCED
    # q_len x heads above MLA_MAX_ROWS (the product would not fit the row count)
    lib = mla.load_library()
    mode, splits, ws = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_size_t()
    s = shape(num_heads=8192)
    assert lib.mla_plan_mtp(ctypes.byref(s), 16, 1024, 0, 256, 0, ctypes.byref(mode),
                            ctypes.byref(splits), ctypes.byref(ws)) == mla.MLA_ERR_ARGUMENT
    assert lib.mla_plan_mtp(ctypes.byref(s), 8, 1024, 0, 256, 0, ctypes.byref(mode),
                            ctypes.byref(splits), ctypes.byref(ws)) == mla.MLA_OK
    # a launch grid beyond what HIP accepts is refused with nothing enqueued:
    # 2^20 sequences x 64 splits x 512 head chunks of stage-1 workgroups
    big = shape(batch=1 << 20, num_heads=mla.MLA_MAX_ROWS, max_blocks_per_seq=1)
    need = mla.mla_workspace_size(big, 0, 64)
    assert need > 0
    assert _decode_raw(big, splits=64, ws=256, ws_bytes=need) == mla.MLA_ERR_SHAPE
    # the shard merge's row cap keeps its grid in range
    assert lib.mla_merge_shards(2, mla.MLA_MAX_MERGE_ROWS + 1, 512, 256, mla.MLA_BF16, 256,
                                0, 256, mla.MLA_BF16, 256, None) == mla.MLA_ERR_SHAPE


def test_fp8_query_is_refused():
    with pytest.raises(NotImplementedError):
        mla.mla_plan(shape(q_dtype=mla.MLA_FP8_E4M3), 100, 0, 256)
    assert _decode_raw(shape(q_dtype=mla.MLA_FP8_E4M3)) == mla.MLA_ERR_DTYPE


# ---------------------------------------------------------------- per-token fp8 cache

@pytest.mark.parametrize("code", [3, 4, 5])
def test_per_token_cache_is_planned_like_the_others(code):
    assert code in (mla.MLA_FP8_E4M3_PER_TOKEN, mla.MLA_INT8_PER_TOKEN, mla.MLA_INT4_PER_TOKEN)
    s, pt = shape(), shape(kv_dtype=code)
    assert mla.mla_plan(pt, 8192, 64 * 4608, 256) == mla.mla_plan(s, 8192, 64 * 4608, 256)
    assert mla.mla_workspace_size(pt, mla.SPLIT_BALANCED, 64) == \
        mla.mla_workspace_size(s, mla.SPLIT_BALANCED, 64)
    with pytest.raises(NotImplementedError):  # MLA_ERR_DTYPE
        mla.mla_plan(shape(kv_dtype=6), 1024, 0, 256)


@pytest.mark.parametrize("code", [3, 4, 5])
def test_per_token_cache_argument_checks(code):
    pt = shape(kv_dtype=code)
    # k_scale is not read for a per-token cache, so 0 passes this check and
    # the call is stopped by the next one (a missing workspace)
    assert _decode_raw(pt, k_scale=0.0, splits=16) == mla.MLA_ERR_WORKSPACE
    assert _decode_raw(pt, q=258) == mla.MLA_ERR_ARGUMENT
    # the sparse gather addresses the pool with 32-bit offsets: pools past
    # 4 GB (here 200000 pages of 64 rows of 592 bytes, or 400000 pages of
    # 304-byte int4 rows) are refused
    lib = mla.load_library()
    big = shape(kv_dtype=code, num_blocks=400000 if code == mla.MLA_INT4_PER_TOKEN else 200000)
    st = lib.mla_decode_sparse(ctypes.byref(big), 2048, 256, 256, 256, 256, 256, 0.07,
                               big.page_size, 1.0, 1, 0, 256, 256, None, 0, None)
    assert st == mla.MLA_ERR_SHAPE
    st = lib.mla_decode_sparse(ctypes.byref(pt), 0, 256, 256, 256, 256, 256, 0.07,
                               pt.page_size, 1.0, 1, 0, 256, 256, None, 0, None)
    assert st == mla.MLA_ERR_ARGUMENT  # topk < 1


def test_shape_of_checks_cache_row_width():
    torch = pytest.importorskip("torch")
    q = torch.zeros(2, 16, 576, dtype=torch.bfloat16)
    bt = torch.zeros(2, 4, dtype=torch.int32)
    pt = torch.zeros(8, 16, 576 + mla.MLA_PER_TOKEN_PAD, dtype=torch.uint8)
    s = mla.shape_of(q, pt, bt, kv_dtype="fp8_per_token")
    assert s.kv_dtype == mla.MLA_FP8_E4M3_PER_TOKEN and s.head_size == 576
    with pytest.raises(ValueError):
        mla.shape_of(q, pt, bt, kv_dtype="fp8_e4m3")  # rows 16 bytes too wide
    with pytest.raises(ValueError):
        mla.shape_of(q, torch.zeros(8, 16, 576, dtype=torch.uint8), bt, kv_dtype="fp8_per_token")
    with pytest.raises(ValueError):
        mla.shape_of(q, torch.zeros(8, 16, 576, dtype=torch.bfloat16), bt, kv_dtype="fp8_e4m3")
    i4 = torch.zeros(8, 16, 288 + mla.MLA_PER_TOKEN_PAD, dtype=torch.uint8)
    s = mla.shape_of(q, i4, bt, kv_dtype="int4_per_token")
    assert s.kv_dtype == mla.MLA_INT4_PER_TOKEN and s.head_size == 576
    with pytest.raises(ValueError):
        mla.shape_of(q, pt, bt, kv_dtype="int4_per_token")  # rows of whole-byte codes


# ---------------------------------------------------------------- cross-shard merge

def _merge_raw(G=2, rows=4, d_v=512, op=256, pd=mla.MLA_BF16, lp=256, base=0, o=256,
               od=mla.MLA_BF16, lse=256):
    return mla.load_library().mla_merge_shards(G, rows, d_v, op, pd, lp, base, o, od, lse, None)


def test_merge_argument_checks_fail_before_launch():
    assert _merge_raw(op=None) == mla.MLA_ERR_NULL
    assert _merge_raw(lse=None) == mla.MLA_ERR_NULL
    assert _merge_raw(G=0) == mla.MLA_ERR_ARGUMENT
    assert _merge_raw(G=mla.MLA_MAX_SHARDS + 1) == mla.MLA_ERR_ARGUMENT
    assert _merge_raw(rows=0) == mla.MLA_ERR_SHAPE
    assert _merge_raw(d_v=320) == mla.MLA_ERR_HEAD_SIZE
    assert _merge_raw(pd=mla.MLA_FP8_E4M3) == mla.MLA_ERR_DTYPE
    assert _merge_raw(od=mla.MLA_FP8_E4M3) == mla.MLA_ERR_DTYPE
    assert _merge_raw(base=2) == mla.MLA_ERR_ARGUMENT
    assert _merge_raw(op=264) == mla.MLA_ERR_ARGUMENT  # misaligned
    assert _merge_raw(lse=258) == mla.MLA_ERR_ARGUMENT


# ---------------------------------------------------------------- host-side table checker

def _tables(B=3, W=4, P=16, num_blocks=20):
    import numpy as np
    s = shape(batch=B, num_heads=16, page_size=P, num_blocks=num_blocks, max_blocks_per_seq=W)
    bt = np.arange(B * W, dtype=np.int32).reshape(B, W) % num_blocks
    sl = np.array([1, P * W, 17], dtype=np.int32)[:B]
    return s, bt, sl


def test_checker_accepts_valid_tables():
    s, bt, sl = _tables()
    mla.mla_check_inputs(s, bt, sl)
    # entries past ceil(n / P) are never read, whatever they hold
    bt2 = bt.copy()
    bt2[0, 1:] = -7
    bt2[2, 2:] = 10 ** 6
    mla.mla_check_inputs(s, bt2, sl)


@pytest.mark.parametrize("what,where", [
    ("len_negative", 0), ("len_past_table", 1), ("page_negative", 2 * 4 + 1),
    ("page_past_pool", 1 * 4 + 3)])
def test_checker_names_the_first_bad_entry(what, where):
    """Request isolation ("vLLM 中 Attention Kernel 如何并行处理多个请求",
    section 十一): a request may reach only pool pages through its own table
    row; a length beyond its row, or a page outside the pool, is refused and
    the flat index of the offending element is reported."""
    s, bt, sl = _tables()
    bt, sl = bt.copy(), sl.copy()
    if what == "len_negative":
        sl[0] = -1
    elif what == "len_past_table":
        sl[1] = 16 * 4 + 1
    elif what == "page_negative":
        bt[2, 1] = -1
    else:
        bt[1, 3] = 20
    with pytest.raises(ValueError, match=rf"flat index {where}\b.*MLA_ERR_TABLE"):
        mla.mla_check_inputs(s, bt, sl)


def test_checker_sparse_lists():
    import numpy as np
    s, bt, sl = _tables()
    ti = np.zeros((3, 5), dtype=np.int32)
    tl = np.array([5, 0, 2], dtype=np.int32)
    ti[0] = [0, 63, 17, 17, 32]
    ti[2, :2] = [5, 40]
    ti[1] = -99  # length 0: never read
    ti[2, 2:] = 10 ** 7  # past topk_lens[2]: never read
    mla.mla_check_inputs(s, bt, None, ti, tl)
    for mutate, where in ((lambda a, l: l.__setitem__(1, 6), 1),
                          (lambda a, l: l.__setitem__(0, -1), 0),
                          (lambda a, l: a.__setitem__((0, 3), 64), 3),
                          (lambda a, l: a.__setitem__((2, 1), -1), 2 * 5 + 1)):
        a, l = ti.copy(), tl.copy()
        mutate(a, l)
        with pytest.raises(ValueError, match=rf"flat index {where}\b"):
            mla.mla_check_inputs(s, bt, None, a, l)
    # a listed position whose page entry is outside the pool: position 63 (entry 1 of
    # sequence 0) is the first to go through table slot 3
    bt2 = bt.copy()
    bt2[0, 3] = 20
    with pytest.raises(ValueError, match=r"flat index 1\b"):
        mla.mla_check_inputs(s, bt2, None, ti, tl)


def test_checker_argument_errors():
    import numpy as np
    lib = mla.load_library()
    s, bt, sl = _tables()
    bad = ctypes.c_int64(5)
    p = lambda a: a.ctypes.data  # noqa: E731
    assert lib.mla_check_inputs(ctypes.byref(s), None, p(sl), 0, None, None,
                                ctypes.byref(bad)) == mla.MLA_ERR_NULL
    assert lib.mla_check_inputs(ctypes.byref(s), p(bt), None, 0, None, None,
                                ctypes.byref(bad)) == mla.MLA_ERR_NULL
    ti = np.zeros((3, 2), dtype=np.int32)
    assert lib.mla_check_inputs(ctypes.byref(s), p(bt), None, 2, p(ti), None,
                                ctypes.byref(bad)) == mla.MLA_ERR_NULL
    assert lib.mla_check_inputs(ctypes.byref(s), p(bt), None, 0, p(ti), p(sl),
                                ctypes.byref(bad)) == mla.MLA_ERR_ARGUMENT
    assert lib.mla_check_inputs(ctypes.byref(shape(head_size=400)), p(bt), p(sl), 0, None,
                                None, ctypes.byref(bad)) == mla.MLA_ERR_HEAD_SIZE
    assert lib.mla_check_inputs(ctypes.byref(s), p(bt), p(sl), 0, None, None, None) == mla.MLA_OK


# ---------------------------------------------------------------- split query (q_nope, q_pe)

def test_split_query_argument_checks():
    """mla_decode_split_q is refused before any launch for a NULL part, a
    misaligned part or a stride that is not a non-negative multiple of 8."""
    lib = mla.load_library()
    s = shape(batch=2, num_heads=16, page_size=16, num_blocks=16, max_blocks_per_seq=8)
    base = 1 << 20  # fake, aligned device addresses: every call here fails its checks first

    def call(q):
        return lib.mla_decode_split_q(ctypes.byref(s), 1, ctypes.byref(q) if q else None,
                                      base, base, base, 0.07, 16, 1.0, 1, 0, base, base,
                                      None, 0, None)
    good = dict(q_nope=base, q_pe=base + 1024, nope_seq_stride=16 * 512, nope_row_stride=512,
                pe_seq_stride=16 * 64, pe_row_stride=64)
    assert call(None) == mla.MLA_ERR_NULL
    assert call(mla.MlaQuery(**dict(good, q_pe=None))) == mla.MLA_ERR_NULL
    assert call(mla.MlaQuery(**dict(good, q_pe=base + 8))) == mla.MLA_ERR_ARGUMENT
    assert call(mla.MlaQuery(**dict(good, nope_row_stride=515))) == mla.MLA_ERR_ARGUMENT
    assert call(mla.MlaQuery(**dict(good, pe_seq_stride=-64))) == mla.MLA_ERR_ARGUMENT
    # a valid query with an invalid shape still fails on the shape
    s.head_size = 400
    assert call(mla.MlaQuery(**good)) == mla.MLA_ERR_HEAD_SIZE


def test_time_next_launch_takes_stage_1_or_2():
    lib = mla.load_library()
    assert lib.mla_time_next_launch(3, None, None) == mla.MLA_ERR_ARGUMENT
    assert lib.mla_time_next_launch(0, None, None) == mla.MLA_ERR_ARGUMENT
    # NULL events: the next launch is a plain one (nothing else changes)
    assert lib.mla_time_next_launch(1, None, None) == mla.MLA_OK
    assert lib.mla_time_next_launch(2, None, None) == mla.MLA_OK
