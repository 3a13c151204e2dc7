"""MLA paged latent decode for MI355X (gfx950): Python binding of libmla.

A thin ctypes layer over the C ABI in ``include/mla.h``.  It only marshals
arguments (shapes, dtypes, raw device pointers, the current HIP stream);
every step of the decode runs in libmla's HIP kernels.  torch provides device
memory and streams.  There is no fallback: if libmla.so is missing or cannot
be loaded, every call raises.

    o, lse = mla_decode(q, kv_cache, block_table, seq_lens, scale, page_size,
                        k_scale, num_kv_splits)

``q`` [B, H, D] bf16 = [q_nope (D_v) | q_pe (64)], or [B, q_len, H, D] for a
multi-token decode (query token i of a sequence with n keys sees positions
< n - q_len + 1 + i), or the tuple ``(q_nope, q_pe)`` of [.., D_v] and [.., 64]
tensors with unit stride on the last axis, read in place (no concatenation);
``kv_cache``
[num_blocks, page_size, D] bf16 or fp8 e4m3fn with rows [kv_c | k_pe];
``block_table`` [B, max_blocks_per_seq] int32; ``seq_lens`` [B] int32.
Returns ``o`` [B, H, D_v] (bf16 by default) and ``lse`` [B, H] float32
(natural log), or [B, q_len, H, D_v] and [B, q_len, H].
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

from . import _build

__all__ = [
    "MlaError", "mla_decode", "mla_decode_sparse", "mla_plan", "mla_check_inputs",
    "mla_decode_noalloc", "mla_noalloc_scratch_bytes", "mla_time_next_launch",
    "mla_workspace_size", "mla_pages_split_count",
    "mla_status_string", "SPLIT_PER_SEQUENCE", "SPLIT_BALANCED", "library_path", "load_library",
    "MLA_BF16", "MLA_FP8_E4M3", "MLA_FP32", "MLA_FP8_E4M3_PER_TOKEN", "MLA_INT8_PER_TOKEN",
    "MLA_INT4_PER_TOKEN",
    "MLA_PER_TOKEN_PAD", "mla_merge_shards", "MLA_LSE_LN", "MLA_LSE_LOG2",
]

MLA_OK, MLA_ERR_NULL, MLA_ERR_HEAD_SIZE, MLA_ERR_PAGE_SIZE, MLA_ERR_DTYPE = 0, 1, 2, 3, 4
MLA_ERR_SHAPE, MLA_ERR_SPLITS, MLA_ERR_WORKSPACE, MLA_ERR_LAUNCH, MLA_ERR_ARGUMENT = 5, 6, 7, 8, 9
MLA_ERR_TABLE, MLA_ERR_SCRATCH = 10, 11
MLA_BF16, MLA_FP8_E4M3, MLA_FP32, MLA_FP8_E4M3_PER_TOKEN, MLA_INT8_PER_TOKEN = 0, 1, 2, 3, 4
MLA_INT4_PER_TOKEN = 5  # two signed 4-bit codes per byte, element 2i in the low nibble
MLA_PER_TOKEN_PAD = 16  # bytes after the codes of a per-token cache row (fp32 scale first)
SPLIT_PER_SEQUENCE, SPLIT_BALANCED = 0, 1
MLA_LSE_LN, MLA_LSE_LOG2 = 0, 1
MLA_MAX_SHARDS = 65536
MLA_MAX_KV_SPLITS = 65536
MLA_MAX_Q_LEN = 16
MLA_MAX_ROWS = 65536  # query rows per sequence: num_heads x q_len
MLA_MAX_BATCH = 1 << 24
MLA_MAX_MERGE_ROWS = 1 << 32


class MlaShape(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "num_heads", "head_size", "kv_lora_rank", "page_size", "num_blocks",
        "max_blocks_per_seq", "q_dtype", "kv_dtype", "o_dtype")]


class MlaQuery(ctypes.Structure):
    _fields_ = [("q_nope", ctypes.c_void_p), ("q_pe", ctypes.c_void_p),
                ("nope_seq_stride", ctypes.c_int64), ("nope_row_stride", ctypes.c_int64),
                ("pe_seq_stride", ctypes.c_int64), ("pe_row_stride", ctypes.c_int64)]


class MlaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


_LIB = None


def library_path() -> str:
    return _build.LIB_PATH


def load_library():
    """Load libmla.so (building it first only if it does not exist)."""
    global _LIB
    if _LIB is None:
        path = _build.ensure_built()
        lib = ctypes.CDLL(path)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        shp = ctypes.POINTER(MlaShape)
        lib.mla_pages_split_count.argtypes = [i32, i32]
        lib.mla_pages_split_count.restype = i32
        lib.mla_plan.argtypes = [shp, i32, i64, i32, i32, ctypes.POINTER(i32),
                                 ctypes.POINTER(i32), ctypes.POINTER(sz)]
        lib.mla_plan.restype = i32
        lib.mla_plan_mtp.argtypes = [shp, i32, i32, i64, i32, i32, ctypes.POINTER(i32),
                                     ctypes.POINTER(i32), ctypes.POINTER(sz)]
        lib.mla_plan_mtp.restype = i32
        lib.mla_workspace_size.argtypes = [shp, i32, i32]
        lib.mla_workspace_size.restype = sz
        lib.mla_workspace_size_mtp.argtypes = [shp, i32, i32, i32]
        lib.mla_workspace_size_mtp.restype = sz
        for fn in (lib.mla_decode, lib.mla_decode_stage1, lib.mla_decode_stage2):
            fn.argtypes = [shp, vp, vp, vp, vp, ctypes.c_float, i32, ctypes.c_float, i32, i32,
                           vp, vp, vp, sz, vp]
            fn.restype = i32
        for fn in (lib.mla_decode_mtp, lib.mla_decode_mtp_stage1, lib.mla_decode_mtp_stage2):
            fn.argtypes = [shp, i32, vp, vp, vp, vp, ctypes.c_float, i32, ctypes.c_float, i32,
                           i32, vp, vp, vp, sz, vp]
            fn.restype = i32
        for fn in (lib.mla_decode_sparse, lib.mla_decode_sparse_stage1,
                   lib.mla_decode_sparse_stage2):
            fn.argtypes = [shp, i32, vp, vp, vp, vp, vp, ctypes.c_float, i32, ctypes.c_float,
                           i32, i32, vp, vp, vp, sz, vp]
            fn.restype = i32
        lib.mla_decode_split_q.argtypes = [shp, i32, ctypes.POINTER(MlaQuery), vp, vp, vp,
                                           ctypes.c_float, i32, ctypes.c_float, i32, i32, vp,
                                           vp, vp, sz, vp]
        lib.mla_decode_split_q.restype = i32
        lib.mla_check_inputs.argtypes = [shp, vp, vp, i32, vp, vp, ctypes.POINTER(i64)]
        lib.mla_decode_noalloc.argtypes = [shp, i32, vp, vp, vp, vp, ctypes.c_float, i32,
                                           ctypes.c_float, i32, i32, vp, vp, vp]
        lib.mla_decode_noalloc.restype = i32
        lib.mla_noalloc_scratch_bytes.argtypes = []
        lib.mla_noalloc_scratch_bytes.restype = sz
        lib.mla_time_next_launch.argtypes = [i32, vp, vp]
        lib.mla_time_next_launch.restype = i32
        lib.mla_check_inputs.restype = i32
        lib.mla_merge_shards.argtypes = [i32, i64, i32, vp, i32, vp, i32, vp, i32, vp, vp]
        lib.mla_merge_shards.restype = i32
        lib.mla_status_string.argtypes = [i32]
        lib.mla_status_string.restype = ctypes.c_char_p
        _LIB = lib
    return _LIB


def mla_status_string(status: int) -> str:
    return load_library().mla_status_string(int(status)).decode()


def _raise(status: int, what: str):
    msg = f"{what}: {mla_status_string(status)}"
    if status in (MLA_ERR_HEAD_SIZE, MLA_ERR_PAGE_SIZE, MLA_ERR_TABLE):
        raise ValueError(msg)
    if status == MLA_ERR_DTYPE:
        raise NotImplementedError(msg)
    raise MlaError(status, msg)


def make_shape(batch, num_heads, head_size, page_size, num_blocks, max_blocks_per_seq,
               kv_dtype=MLA_BF16, o_dtype=MLA_BF16, q_dtype=MLA_BF16,
               kv_lora_rank: Optional[int] = None) -> MlaShape:
    return MlaShape(int(batch), int(num_heads), int(head_size),
                    int(head_size - 64 if kv_lora_rank is None else kv_lora_rank),
                    int(page_size), int(num_blocks), int(max_blocks_per_seq), int(q_dtype),
                    int(kv_dtype), int(o_dtype))


def mla_pages_split_count(max_seq_len: int, num_cus: int) -> int:
    return int(load_library().mla_pages_split_count(int(max_seq_len), int(num_cus)))


def mla_workspace_size(shape: MlaShape, split_mode: int, num_kv_splits: int,
                       q_len: int = 1) -> int:
    return int(load_library().mla_workspace_size_mtp(ctypes.byref(shape), int(q_len),
                                                     int(split_mode), int(num_kv_splits)))


def mla_plan(shape: MlaShape, max_seq_len: int, total_seq_len: int = 0, num_cus: int = 256,
             deterministic: bool = False, q_len: int = 1) -> Tuple[int, int, int]:
    """Returns (split_mode, num_kv_splits, workspace_bytes)."""
    mode, splits, ws = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_size_t()
    st = load_library().mla_plan_mtp(ctypes.byref(shape), int(q_len), int(max_seq_len),
                                     int(total_seq_len), int(num_cus), 1 if deterministic else 0,
                                     ctypes.byref(mode), ctypes.byref(splits), ctypes.byref(ws))
    if st != MLA_OK:
        _raise(st, "mla_plan")
    return mode.value, splits.value, ws.value


def _torch():
    import torch
    return torch


def _kv_code(kv_cache, kv_dtype):
    """Cache dtype code: from ``kv_dtype`` ("bf16", "fp8_e4m3", "fp8_per_token",
    "int8_per_token", "int4_per_token" or an mla_dtype value) or else from the tensor's dtype.
    A per-token cache is a uint8 tensor [num_blocks, page, C + MLA_PER_TOKEN_PAD] (C = head_size
    code bytes, head_size / 2 for int4) and must be named explicitly."""
    torch = _torch()
    if kv_dtype is not None:
        return {"bf16": MLA_BF16, "fp8_e4m3": MLA_FP8_E4M3,
                "fp8_per_token": MLA_FP8_E4M3_PER_TOKEN,
                "int8_per_token": MLA_INT8_PER_TOKEN,
                "int4_per_token": MLA_INT4_PER_TOKEN}.get(kv_dtype, kv_dtype)
    if kv_cache.dtype == torch.bfloat16:
        return MLA_BF16
    if kv_cache.dtype == torch.float8_e4m3fn:
        return MLA_FP8_E4M3
    return -1


def _dtype_code(t):
    torch = _torch()
    return {torch.bfloat16: MLA_BF16, torch.float32: MLA_FP32,
            torch.float8_e4m3fn: MLA_FP8_E4M3}.get(t, -1)


def _check_sizes(shape, rows, block_table, lens, o, lse, topk_indices=None):
    """The buffers the kernels index by sequence and row must hold B of them:
    block_table [B, W], the lengths [B] (seq_lens, or topk_lens with
    topk_indices [B, topk]), o rows + (D_v,) and lse rows float32, contiguous,
    with rows = (B, H), or (B, q_len, H) for a [B, q_len, H, D] query.  The C
    ABI takes raw pointers and cannot check this."""
    torch = _torch()
    B = shape.batch
    if block_table.shape[0] != B:
        raise ValueError(f"block_table has {block_table.shape[0]} rows, expected {B}")
    if lens.dim() != 1 or lens.shape[0] != B:
        raise ValueError(f"sequence lengths must be [{B}]")
    if topk_indices is not None and (topk_indices.dim() != 2 or topk_indices.shape[0] != B):
        raise ValueError(f"topk_indices must be [{B}, topk]")
    if (tuple(o.shape) != rows + (shape.kv_lora_rank,) or tuple(lse.shape) != rows
            or lse.dtype != torch.float32 or not o.is_contiguous() or not lse.is_contiguous()
            or not (o.is_cuda and lse.is_cuda)):
        raise ValueError("o must be [B,(q_len,)H,kv_lora_rank] and lse [B,(q_len,)H] float32, "
                         "contiguous device tensors")


def shape_of(q, kv_cache, block_table, *, kv_dtype=None, o_dtype=None) -> MlaShape:
    """The mla_shape of a call; q is [B, H, D] or [B, q_len, H, D] (H per token)."""
    torch = _torch()
    if q.dim() not in (3, 4) or kv_cache.dim() != 3 or block_table.dim() != 2:
        raise ValueError("expected q [B,H,D] or [B,q_len,H,D], kv_cache [num_blocks,page,D], "
                         "block_table [B,W]")
    B, H, D = q.shape[0], q.shape[-2], q.shape[-1]
    code = _kv_code(kv_cache, kv_dtype)
    per_token = code in (MLA_FP8_E4M3_PER_TOKEN, MLA_INT8_PER_TOKEN, MLA_INT4_PER_TOKEN)
    width = ((D // 2 if code == MLA_INT4_PER_TOKEN else D) + MLA_PER_TOKEN_PAD) if per_token else D
    if kv_cache.shape[-1] != width:
        raise ValueError(f"kv_cache rows hold {kv_cache.shape[-1]} elements, expected {width}")
    if kv_cache.element_size() != (2 if code == MLA_BF16 else 1):
        raise ValueError(f"kv_cache element size {kv_cache.element_size()} does not fit its dtype")
    return make_shape(B, H, D, kv_cache.shape[1], kv_cache.shape[0], block_table.shape[1],
                      kv_dtype=code,
                      o_dtype=_dtype_code(o_dtype or torch.bfloat16),
                      q_dtype=_dtype_code(q.dtype))


def mla_check_inputs(shape: MlaShape, block_table, seq_lens=None, topk_indices=None,
                     topk_lens=None) -> None:
    """Check the tables a decode call will read (host-side, ``mla_check_inputs``
    of the C ABI): lengths within the table width, every page a sequence reads
    inside the pool, and for sparse decode every listed position addressable
    and its page inside the pool.  Device tensors are copied to the host
    first, which synchronises with the device.  Raises ValueError naming the
    first bad entry."""
    import numpy as np
    lib = load_library()

    def host(t):
        if t is None:
            return None
        a = t.detach().cpu().numpy() if hasattr(t, "detach") else np.asarray(t)
        return np.ascontiguousarray(a, dtype=np.int32)
    bt, sl, ti, tl = host(block_table), host(seq_lens), host(topk_indices), host(topk_lens)
    topk = int(ti.shape[1]) if ti is not None else 0
    ptr = lambda a: a.ctypes.data if a is not None else None  # noqa: E731
    bad = ctypes.c_int64(-1)
    st = lib.mla_check_inputs(ctypes.byref(shape), ptr(bt), ptr(sl), topk, ptr(ti), ptr(tl),
                              ctypes.byref(bad))
    if st != MLA_OK:
        _raise(st, f"mla_check_inputs (first bad element: flat index {bad.value})")


def _query_of(q, B, H, D, D_v, q_len):
    """(MlaQuery, device, dtype) of a tuple query (q_nope [.., D_v], q_pe [.., 64]) laid out
    as [B, H, *] or [B, q_len, H, *]; strides in elements, rows merged over (q_len, H)."""
    q_nope, q_pe = q
    q_len_dims = 4 if q_len > 1 else 3
    for name, t, w in (("q_nope", q_nope, D_v), ("q_pe", q_pe, D - D_v)):
        if not t.is_cuda or t.dim() != q_len_dims or t.shape[-1] != w or t.stride(-1) != 1:
            raise ValueError(f"{name} must be a device tensor [B,(q_len,)H,{w}] with unit "
                             "stride on its last axis")
        if tuple(t.shape[:-1]) != tuple(q_nope.shape[:-1]):
            raise ValueError("q_nope and q_pe must have the same leading shape")
        if q_len > 1 and t.stride(1) != H * t.stride(2):
            raise ValueError(f"{name}: the (q_len, H) axes must be mergeable into one row axis")
    row = -2
    return MlaQuery(q_nope.data_ptr(), q_pe.data_ptr(), q_nope.stride(0), q_nope.stride(row),
                    q_pe.stride(0), q_pe.stride(row))


def mla_decode(q, kv_cache, block_table, seq_lens, scale: float, page_size: int,
               k_scale: float = 1.0, num_kv_splits: Optional[int] = None, o=None, lse=None, *,
               split_mode: Optional[int] = None, workspace=None, kv_dtype=None,
               o_dtype=None, max_seq_len: Optional[int] = None,
               total_seq_len: Optional[int] = None, num_cus: Optional[int] = None,
               deterministic: bool = False, stream=None, stages: str = "both",
               check: bool = False):
    """Enqueue one MLA decode step on the current (or given) stream.

    When ``num_kv_splits`` is None the split plan comes from ``mla_plan``
    with the host-side ``max_seq_len`` / ``total_seq_len`` if given (as a
    serving loop keeps them in its metadata); otherwise the table width
    (``block_table.shape[1] * page_size``) bounds every length, so planning
    never reads ``seq_lens`` back from the device.  When ``num_kv_splits`` is
    given without ``split_mode``, the per-sequence split layout is used.
    Missing ``o``/``lse``/``workspace`` are allocated with torch.  ``stages`` =
    "stage1" / "stage2" enqueues only that half (mla_decode_stage1 /
    mla_decode_stage2; not for a tuple q).  ``check=True`` first validates the
    tables on the host (``mla_check_inputs``; a device-to-host copy).  Returns
    (o, lse)."""
    torch = _torch()
    lib = load_library()
    split_q = isinstance(q, (tuple, list))
    if split_q:
        if len(q) != 2:
            raise ValueError("a tuple query is (q_nope, q_pe)")
        q_tuple = (q[0], q[1])
        q = q_tuple[0]  # leading dims, device and dtype come from q_nope
    if not (q.is_cuda and kv_cache.is_cuda and block_table.is_cuda and seq_lens.is_cuda):
        raise ValueError("mla_decode needs device tensors (HIP)")
    for name, t in (("q", q), ("kv_cache", kv_cache), ("block_table", block_table),
                    ("seq_lens", seq_lens)):
        if not t.is_contiguous() and not (split_q and name == "q"):
            raise ValueError(f"{name} must be contiguous")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    if o is not None:
        o_dtype = o.dtype
    if split_q:
        D = q_tuple[0].shape[-1] + q_tuple[1].shape[-1]
        qshape = torch.empty(tuple(q.shape[:-1]) + (D,), dtype=q.dtype, device="meta")
        shape = shape_of(qshape, kv_cache, block_table, kv_dtype=kv_dtype, o_dtype=o_dtype)
    else:
        shape = shape_of(q, kv_cache, block_table, kv_dtype=kv_dtype, o_dtype=o_dtype)
    B, H = shape.batch, shape.num_heads
    q_len = q.shape[1] if q.dim() == 4 else 1
    rows = (B, q_len, H) if q.dim() == 4 else (B, H)
    if check:
        mla_check_inputs(shape, block_table, seq_lens)
    if num_kv_splits is None:
        if max_seq_len is None:
            # no device read-back: the table width bounds every length
            max_seq_len = int(block_table.shape[1]) * int(page_size)
            total_seq_len = total_seq_len or 0
        if num_cus is None:
            num_cus = torch.cuda.get_device_properties(q.device).multi_processor_count
        split_mode, num_kv_splits, _ = mla_plan(shape, max_seq_len, total_seq_len or 0,
                                                num_cus, deterministic, q_len=q_len)
    elif split_mode is None:
        split_mode = SPLIT_PER_SEQUENCE
    ws_need = mla_workspace_size(shape, split_mode, num_kv_splits, q_len)
    if o is None:
        o = torch.empty(rows + (shape.kv_lora_rank,), dtype=o_dtype or torch.bfloat16,
                        device=q.device)
    if lse is None:
        lse = torch.empty(rows, dtype=torch.float32, device=q.device)
    _check_sizes(shape, rows, block_table, seq_lens, o, lse)
    if workspace is None and ws_need > 0:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    if split_q:
        if stages != "both":
            raise ValueError("a tuple query runs both stages (mla_decode_split_q)")
        qd = _query_of(q_tuple, B, H, shape.head_size, shape.kv_lora_rank, q_len)
        st = lib.mla_decode_split_q(ctypes.byref(shape), int(q_len), ctypes.byref(qd),
                                    kv_cache.data_ptr(), block_table.data_ptr(),
                                    seq_lens.data_ptr(), float(scale), int(page_size),
                                    float(k_scale), int(num_kv_splits), int(split_mode),
                                    o.data_ptr(), lse.data_ptr(), ws_ptr, int(ws_bytes), stream)
        if st != MLA_OK:
            _raise(st, "mla_decode_split_q")
        return o, lse
    fn = {"both": lib.mla_decode_mtp, "stage1": lib.mla_decode_mtp_stage1,
          "stage2": lib.mla_decode_mtp_stage2}[stages]
    st = fn(ctypes.byref(shape), int(q_len), q.data_ptr(), kv_cache.data_ptr(),
                        block_table.data_ptr(), seq_lens.data_ptr(), float(scale),
                        int(page_size), float(k_scale), int(num_kv_splits), int(split_mode),
                        o.data_ptr(), lse.data_ptr(), ws_ptr, int(ws_bytes), stream)
    if st != MLA_OK:
        _raise(st, "mla_decode")
    return o, lse


def mla_decode_sparse(q, kv_cache, block_table, topk_indices, topk_lens, scale: float,
                      page_size: int, k_scale: float = 1.0,
                      num_kv_splits: Optional[int] = None, o=None, lse=None, *,
                      split_mode: Optional[int] = None, workspace=None, o_dtype=None,
                      num_cus: Optional[int] = None, stream=None, stages: str = "both",
                      kv_dtype=None, total_topk: Optional[int] = None, check: bool = False):
    """Sparse (top-k) MLA decode: sequence b attends to the cache rows of the
    logical positions ``topk_indices[b, :topk_lens[b]]`` (int32 [B, topk] and
    [B]).  Other arguments as in ``mla_decode``; the split plan counts list
    entries (``total_topk`` = their sum if known on the host, else B * topk is
    assumed; nothing is read back from the device).  ``check=True`` validates
    the lists and tables on the host first.  Returns (o [B, H, D_v], lse [B, H])."""
    torch = _torch()
    lib = load_library()
    for name, t in (("q", q), ("kv_cache", kv_cache), ("block_table", block_table),
                    ("topk_indices", topk_indices), ("topk_lens", topk_lens)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if topk_indices.dtype != torch.int32 or topk_lens.dtype != torch.int32:
        raise ValueError("topk_indices and topk_lens must be int32")
    if o is not None:
        o_dtype = o.dtype
    shape = shape_of(q, kv_cache, block_table, kv_dtype=kv_dtype, o_dtype=o_dtype)
    B, H = shape.batch, shape.num_heads
    topk = int(topk_indices.shape[1])
    if check:
        mla_check_inputs(shape, block_table, None, topk_indices, topk_lens)
    if num_kv_splits is None:
        if num_cus is None:
            num_cus = torch.cuda.get_device_properties(q.device).multi_processor_count
        split_mode, num_kv_splits, _ = mla_plan(shape, topk, int(total_topk or 0), num_cus)
    elif split_mode is None:
        split_mode = SPLIT_PER_SEQUENCE
    ws_need = mla_workspace_size(shape, split_mode, num_kv_splits)
    if o is None:
        o = torch.empty((B, H, shape.kv_lora_rank), dtype=o_dtype or torch.bfloat16,
                        device=q.device)
    if lse is None:
        lse = torch.empty((B, H), dtype=torch.float32, device=q.device)
    _check_sizes(shape, (B, H), block_table, topk_lens, o, lse, topk_indices)
    if workspace is None and ws_need > 0:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    fn = {"both": lib.mla_decode_sparse, "stage1": lib.mla_decode_sparse_stage1,
          "stage2": lib.mla_decode_sparse_stage2}[stages]
    st = fn(ctypes.byref(shape), topk, q.data_ptr(), kv_cache.data_ptr(), block_table.data_ptr(),
            topk_indices.data_ptr(), topk_lens.data_ptr(), float(scale), int(page_size),
            float(k_scale), int(num_kv_splits), int(split_mode), o.data_ptr(), lse.data_ptr(),
            workspace.data_ptr() if workspace is not None else None,
            workspace.numel() * workspace.element_size() if workspace is not None else 0, stream)
    if st != MLA_OK:
        _raise(st, "mla_decode_sparse")
    return o, lse


def mla_noalloc_scratch_bytes() -> int:
    """Bytes of the built-in scratch that mla_decode_noalloc uses per device."""
    return int(load_library().mla_noalloc_scratch_bytes())


def mla_time_next_launch(stage: int, start_event, stop_event) -> None:
    """The next launch of stage 1 or 2 made by this thread records the
    kernel's own start and end into the two torch.cuda.Event objects (created
    with enable_timing=True and recorded once before, so that they exist);
    elapsed_time between them is then the kernel alone."""
    st = load_library().mla_time_next_launch(int(stage), start_event.cuda_event,
                                             stop_event.cuda_event)
    if st != MLA_OK:
        _raise(st, "mla_time_next_launch")


def mla_decode_noalloc(q, kv_cache, block_table, seq_lens, scale: float, page_size: int,
                       k_scale: float, num_kv_splits: int, split_mode: int, o, lse, *,
                       kv_dtype=None, stream=None):
    """Enqueue one decode step through the allocation-free entry point of the C
    ABI (mla_decode_noalloc): no workspace, no allocation by the library or by
    this wrapper, so the caller passes o and lse and the split plan (from
    mla_plan, a host-only call).  Results are bitwise those of mla_decode with
    the same plan.  Calls that overlap in time on one device share its
    built-in scratch and race; calls in order on one stream are safe."""
    torch = _torch()
    lib = load_library()
    for name, t in (("q", q), ("kv_cache", kv_cache), ("block_table", block_table),
                    ("seq_lens", seq_lens)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    shape = shape_of(q, kv_cache, block_table, kv_dtype=kv_dtype, o_dtype=o.dtype)
    q_len = q.shape[1] if q.dim() == 4 else 1
    rows = ((shape.batch, q_len, shape.num_heads) if q.dim() == 4
            else (shape.batch, shape.num_heads))
    _check_sizes(shape, rows, block_table, seq_lens, o, lse)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    st = lib.mla_decode_noalloc(ctypes.byref(shape), int(q_len), q.data_ptr(),
                                kv_cache.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr(),
                                float(scale), int(page_size), float(k_scale), int(num_kv_splits),
                                int(split_mode), o.data_ptr(), lse.data_ptr(), stream)
    if st != MLA_OK:
        _raise(st, "mla_decode_noalloc")
    return o, lse


def mla_merge_shards(o_parts, lse_parts, lse_base: str = "ln", o=None, lse=None, *,
                     o_dtype=None, stream=None):
    """Merge G context shards' decode results through their LSE (the C ABI's
    mla_merge_shards).  o_parts [G, ..., D_v] (bf16 or fp32) and lse_parts
    [G, ...] float32 are device tensors; lse_base is "ln" or "log2".
    Returns (o [..., D_v], lse [...]) with lse in natural log."""
    torch = _torch()
    lib = load_library()
    if not (o_parts.is_cuda and lse_parts.is_cuda):
        raise ValueError("mla_merge_shards needs device tensors (HIP)")
    if o_parts.dim() < 2 or tuple(lse_parts.shape) != tuple(o_parts.shape[:-1]):
        raise ValueError("o_parts must be [G, ..., D_v] and lse_parts [G, ...]")
    if not (o_parts.is_contiguous() and lse_parts.is_contiguous()):
        raise ValueError("o_parts and lse_parts must be contiguous")
    if lse_parts.dtype != torch.float32:
        raise ValueError("lse_parts must be float32")
    G, d_v = o_parts.shape[0], o_parts.shape[-1]
    rows_shape = tuple(o_parts.shape[1:-1])
    rows = 1
    for r in rows_shape:
        rows *= int(r)
    if o is None:
        o = torch.empty(rows_shape + (d_v,), dtype=o_dtype or torch.bfloat16,
                        device=o_parts.device)
    if lse is None:
        lse = torch.empty(rows_shape, dtype=torch.float32, device=o_parts.device)
    if (tuple(o.shape) != rows_shape + (d_v,) or tuple(lse.shape) != rows_shape
            or not o.is_contiguous() or not lse.is_contiguous() or lse.dtype != torch.float32):
        raise ValueError("o must be [..., D_v] and lse [...] float32, contiguous")
    base = {"ln": MLA_LSE_LN, "log2": MLA_LSE_LOG2}[lse_base]
    if stream is None:
        stream = torch.cuda.current_stream(o_parts.device).cuda_stream
    elif hasattr(stream, "cuda_stream"):
        stream = stream.cuda_stream
    st = lib.mla_merge_shards(int(G), int(rows), int(d_v), o_parts.data_ptr(),
                              _dtype_code(o_parts.dtype), lse_parts.data_ptr(), base,
                              o.data_ptr(), _dtype_code(o.dtype), lse.data_ptr(), stream)
    if st != MLA_OK:
        _raise(st, "mla_merge_shards")
    return o, lse


class PreparedDecode:
    """A decode call with every argument marshalled once, for loops that
    launch the same step repeatedly (benchmarks, graph capture).  Calling it
    enqueues the chosen stages through the C ABI; torch tensors are kept
    alive by this object."""

    def __init__(self, q, kv_cache, block_table, seq_lens, scale, page_size, k_scale,
                 num_kv_splits, split_mode, o, lse, workspace=None, kv_dtype=None, stream=None,
                 topk_indices=None):
        """``topk_indices`` [B, topk] selects sparse decode; ``seq_lens`` then
        holds the list lengths."""
        torch = _torch()
        self.lib = load_library()
        self.keep = (q, kv_cache, block_table, seq_lens, o, lse, workspace)
        self.shape = shape_of(q, kv_cache, block_table, kv_dtype=kv_dtype, o_dtype=o.dtype)
        q_len = q.shape[1] if q.dim() == 4 else 1
        rows = ((self.shape.batch, q_len, self.shape.num_heads) if q.dim() == 4
                else (self.shape.batch, self.shape.num_heads))
        _check_sizes(self.shape, rows, block_table, seq_lens, o, lse, topk_indices)
        need = mla_workspace_size(self.shape, split_mode, num_kv_splits, q_len)
        if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
            raise MlaError(MLA_ERR_WORKSPACE, "workspace too small")
        if stream is None:
            stream = torch.cuda.current_stream(q.device).cuda_stream
        elif hasattr(stream, "cuda_stream"):
            stream = stream.cuda_stream
        lead = (ctypes.byref(self.shape), int(q_len), q.data_ptr(), kv_cache.data_ptr(),
                block_table.data_ptr())
        if topk_indices is not None:
            self.keep = self.keep + (topk_indices,)
            lead = (ctypes.byref(self.shape), int(topk_indices.shape[1]), q.data_ptr(),
                    kv_cache.data_ptr(), block_table.data_ptr(), topk_indices.data_ptr())
        self.args = lead + (seq_lens.data_ptr(), float(scale), int(page_size),
                     float(k_scale), int(num_kv_splits), int(split_mode), o.data_ptr(),
                     lse.data_ptr(), workspace.data_ptr() if workspace is not None else None,
                     workspace.numel() * workspace.element_size() if workspace is not None else 0,
                     stream)
        self.fns = {"both": self.lib.mla_decode_mtp, "stage1": self.lib.mla_decode_mtp_stage1,
                    "stage2": self.lib.mla_decode_mtp_stage2}
        if topk_indices is not None:
            self.fns = {"both": self.lib.mla_decode_sparse,
                        "stage1": self.lib.mla_decode_sparse_stage1,
                        "stage2": self.lib.mla_decode_sparse_stage2}

    def __call__(self, stages: str = "both"):
        st = self.fns[stages](*self.args)
        if st != MLA_OK:
            _raise(st, "mla_decode")
