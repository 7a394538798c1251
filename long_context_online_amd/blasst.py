"""ctypes binding of libblasst.so (argument marshalling only).

Every function here only turns torch tensors / Python numbers into the C structs of
include/blasst.h and calls the library; all computation happens in the HIP kernels (or, for the
calibration helpers, in the library's host code).  torch is used for device memory and streams.
The library must have been built (``long_context_online_amd.build``); nothing falls back to
another implementation.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libblasst.so")

OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_HIP, ERR_WORKSPACE = 0, 1, 2, 3, 4
BF16, FP32 = 0, 1
THR_LAMBDA, THR_A_OVER_L, THR_NONE = 0, 1, 2
KEPT, SKIPPED, NOT_LIVE = 0, 1, 2
V_KEPT, V_ALL = 0, 1

EXPORTED = [
    "blasst_prefill", "blasst_prefill_workspace_size", "blasst_decode", "blasst_decode_workspace_size", "blasst_calib_quantile",
    "blasst_calibrate", "blasst_lambda_for", "blasst_status_string", "blasst_last_error",
    "blasst_version", "blasst_prefill_params_size", "blasst_decode_params_size",
    "blasst_prefill_backward", "blasst_prefill_backward_workspace_size", "blasst_prefill_backward_params_size",
    "blasst_prefill_paged", "blasst_prefill_paged_params_size", "blasst_decode_no_alloc",
]


class BlasstError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"blasst status {status}: {message}")
        self.status = status


class Threshold(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("lambda_", ctypes.c_double), ("a", ctypes.c_double)]


class PrefillParams(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("skip_mask", ctypes.c_void_p), ("crit", ctypes.c_void_p), ("counters", ctypes.c_void_p),
        ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
        ("thr", Threshold),
        ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32), ("seqlen_q", ctypes.c_int32), ("seqlen_k", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim_qk", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
        ("causal", ctypes.c_int32), ("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32),
        ("num_splits", ctypes.c_int32), ("stats_only", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("head_counters", ctypes.c_void_p),
        ("v_staging", ctypes.c_int32),
    ]


class DecodeParams(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("skip_mask", ctypes.c_void_p), ("crit", ctypes.c_void_p), ("counters", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("thr", Threshold),
        ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim_qk", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int32),
        ("block_k", ctypes.c_int32), ("num_splits", ctypes.c_int32), ("tile_rows", ctypes.c_int32),
        ("stats_only", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float), ("num_q_tokens", ctypes.c_int32),
    ]


class PagedPrefillParams(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
        ("skip_mask", ctypes.c_void_p), ("crit", ctypes.c_void_p), ("counters", ctypes.c_void_p),
        ("q_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
        ("thr", Threshold),
        ("in_dtype", ctypes.c_int32), ("out_dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32), ("seqlen_q", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim_qk", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32), ("num_pages", ctypes.c_int32),
        ("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32), ("num_splits", ctypes.c_int32),
        ("stats_only", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
    ]


class BackwardParams(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("dout", ctypes.c_void_p),
        ("lse", ctypes.c_void_p), ("skip_mask", ctypes.c_void_p),
        ("dq", ctypes.c_void_p), ("dk", ctypes.c_void_p), ("dv", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t),
        ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
        ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
        ("dout_stride", ctypes.c_int64 * 3), ("dq_stride", ctypes.c_int64 * 3),
        ("dk_stride", ctypes.c_int64 * 3), ("dv_stride", ctypes.c_int64 * 3),
        ("in_dtype", ctypes.c_int32), ("grad_dtype", ctypes.c_int32), ("o_dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32), ("seqlen_q", ctypes.c_int32), ("seqlen_k", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim_qk", ctypes.c_int32), ("head_dim_v", ctypes.c_int32),
        ("causal", ctypes.c_int32), ("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
    ]


_lib = None


def lib():
    """Loads libblasst.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m long_context_online_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.blasst_prefill.argtypes = [ctypes.POINTER(PrefillParams), ctypes.c_void_p]
        L.blasst_prefill.restype = ctypes.c_int
        L.blasst_prefill_workspace_size.argtypes = [ctypes.POINTER(PrefillParams)]
        L.blasst_prefill_workspace_size.restype = ctypes.c_size_t
        L.blasst_decode.argtypes = [ctypes.POINTER(DecodeParams), ctypes.c_void_p]
        L.blasst_decode.restype = ctypes.c_int
        L.blasst_decode_workspace_size.argtypes = [ctypes.POINTER(DecodeParams)]
        L.blasst_decode_workspace_size.restype = ctypes.c_size_t
        L.blasst_decode_no_alloc.argtypes = [ctypes.POINTER(DecodeParams), ctypes.c_void_p]
        L.blasst_decode_no_alloc.restype = ctypes.c_int
        L.blasst_prefill_paged.argtypes = [ctypes.POINTER(PagedPrefillParams), ctypes.c_void_p]
        L.blasst_prefill_paged.restype = ctypes.c_int
        L.blasst_prefill_paged_params_size.restype = ctypes.c_size_t
        L.blasst_prefill_backward.argtypes = [ctypes.POINTER(BackwardParams), ctypes.c_void_p]
        L.blasst_prefill_backward.restype = ctypes.c_int
        L.blasst_prefill_backward_workspace_size.argtypes = [ctypes.POINTER(BackwardParams)]
        L.blasst_prefill_backward_workspace_size.restype = ctypes.c_size_t
        L.blasst_calib_quantile.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_int64, ctypes.c_double,
                                            ctypes.POINTER(ctypes.c_double)]
        L.blasst_calib_quantile.restype = ctypes.c_int
        dp = ctypes.POINTER(ctypes.c_double)
        L.blasst_calibrate.argtypes = [dp, dp, dp, ctypes.c_int32, dp, dp, dp]
        L.blasst_calibrate.restype = ctypes.c_int
        L.blasst_lambda_for.argtypes = [ctypes.c_double] * 4
        L.blasst_lambda_for.restype = ctypes.c_double
        L.blasst_status_string.argtypes = [ctypes.c_int]
        L.blasst_status_string.restype = ctypes.c_char_p
        L.blasst_last_error.argtypes = []
        L.blasst_last_error.restype = ctypes.c_char_p
        L.blasst_version.restype = ctypes.c_int32
        L.blasst_prefill_params_size.restype = ctypes.c_size_t
        L.blasst_decode_params_size.restype = ctypes.c_size_t
        L.blasst_prefill_backward_params_size.restype = ctypes.c_size_t
        if L.blasst_prefill_params_size() != ctypes.sizeof(PrefillParams) or \
                L.blasst_decode_params_size() != ctypes.sizeof(DecodeParams) or \
                L.blasst_prefill_backward_params_size() != ctypes.sizeof(BackwardParams) or \
                L.blasst_prefill_paged_params_size() != ctypes.sizeof(PagedPrefillParams):
            raise ImportError("libblasst.so struct layout does not match this binding")
        _lib = L
    return _lib


def _check(status: int):
    if status != OK:
        raise BlasstError(status, lib().blasst_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _device_of(*ts):
    """The one GPU device that every given tensor lives on (the kernels read and write them all)."""
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("every tensor argument must be a GPU tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensors on {dev} and {t.device}: all must be on one GPU")
    return dev


def _buf(t, name, dtypes, numel, contiguous=True):
    """Pointer to a buffer the kernels index as a flat array of at least `numel` elements."""
    if t is None:
        return None
    if t.dtype not in dtypes:
        raise TypeError(f"{name} must be {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, the call writes {numel}")
    return ctypes.c_void_p(t.data_ptr())


def _shape(t, name, shape):
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _torch_types():
    import torch
    f32, u8, i32 = (torch.float32,), (torch.uint8,), (torch.int32,)
    cnt = (torch.int64,) + ((torch.uint64,) if hasattr(torch, "uint64") else ())
    return f32, u8, i32, cnt


def _cdiv(a, b):
    return -(-a // b)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _threshold(lam, a, no_decision=False):
    if no_decision:
        if lam is not None or a is not None:
            raise ValueError("no_decision takes neither lam nor a")
        return Threshold(THR_NONE, 0, 0.0, 0.0)
    if (lam is None) == (a is None):
        raise ValueError("give exactly one of lam and a")
    if lam is not None:
        return Threshold(THR_LAMBDA, 0, float(lam), 0.0)
    return Threshold(THR_A_OVER_L, 0, 0.0, float(a))


def _stream(stream, device=None):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _call(fn, p, stream, device):
    """Calls the library with the tensors' device current (the library launches on the current
    device) on `stream` (default: that device's current stream)."""
    import torch
    with torch.cuda.device(device):
        _check(fn(ctypes.byref(p), _stream(stream, device)))


def _strides3(t):
    s = t.stride()
    if s[3] != 1:
        raise ValueError("the last dimension must be contiguous")
    return (ctypes.c_int64 * 3)(s[0], s[1], s[2])


def prefill_params(q, k, v, o, *, causal, block_q, block_k, num_splits=1, lam=None, a=None,
                   softmax_scale=0.0, lse=None, skip_mask=None, crit=None, counters=None,
                   stats_only=False, out_dtype=None, no_decision=False, head_counters=None, v_staging=V_KEPT):
    """Fills the C params struct for blasst_prefill from tensors (no call).  Checks what the C side
    cannot: one GPU for every tensor, matching shapes, and diagnostics buffers of the right dtype and
    size."""
    f32, u8, _, cnt = _torch_types()
    _device_of(q, k, v, o, lse, skip_mask, crit, counters, head_counters)
    B, Hq, Lq, _ = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    _shape(k, "k", (B, Hkv, Lk, q.shape[3]))
    _shape(v, "v", (B, Hkv, Lk, v.shape[3]))
    if o is not None:
        _shape(o, "o", (B, Hq, Lq, v.shape[3]))
    nmask = B * Hq * _cdiv(Lq, max(1, block_q)) * _cdiv(Lk, max(1, block_k))
    p = PrefillParams()
    p.struct_size = ctypes.sizeof(PrefillParams)
    p.q, p.k, p.v = _ptr(q), _ptr(k), _ptr(v)
    p.o = _ptr(o)
    p.lse = _buf(lse, "lse", f32, B * Hq * Lq)
    p.skip_mask = _buf(skip_mask, "skip_mask", u8, nmask)
    p.crit = _buf(crit, "crit", f32, nmask)
    p.counters = _buf(counters, "counters", cnt, 2)
    p.q_stride, p.k_stride, p.v_stride = _strides3(q), _strides3(k), _strides3(v)
    p.o_stride = _strides3(o) if o is not None else (ctypes.c_int64 * 3)(0, 0, 0)
    p.thr = _threshold(lam, a, no_decision)
    p.in_dtype = _dtype_code(q)
    p.out_dtype = _dtype_code(o) if o is not None else (p.in_dtype if out_dtype is None else out_dtype)
    p.batch, p.num_q_heads, p.seqlen_q, p.head_dim_qk = q.shape
    p.num_kv_heads, p.seqlen_k = k.shape[1], k.shape[2]
    p.head_dim_v = v.shape[3]
    p.causal, p.block_q, p.block_k = int(bool(causal)), block_q, block_k
    p.num_splits, p.stats_only = num_splits, int(bool(stats_only))
    p.softmax_scale = float(softmax_scale)
    p.head_counters = _buf(head_counters, "head_counters", cnt, B * Hq * 2)
    p.v_staging = int(v_staging)
    return p


def blasst_prefill_workspace_size(q, k, v, o, **kw) -> int:
    """Workspace bytes of blasst_prefill for these arguments (always 0: the prefill keeps every
    partial result on chip); raises on invalid arguments."""
    p = prefill_params(q, k, v, o, **kw)
    n = lib().blasst_prefill_workspace_size(ctypes.byref(p))
    err = lib().blasst_last_error().decode()
    if err:
        raise BlasstError(ERR_INVALID_ARG, err)
    return int(n)


def blasst_prefill(q, k, v, o, *, stream=None, **kw):
    """BLASST prefill forward.  q [B, Hq, Lq, D], k/v [B, Hkv, Lk, D], o [B, Hq, Lq, Dv]
    (last dim contiguous).  Keyword args follow the C params (causal, block_q, block_k,
    num_splits, lam or a, softmax_scale, lse, skip_mask, crit, counters, head_counters,
    stats_only, v_staging)."""
    p = prefill_params(q, k, v, o, **kw)
    _call(lib().blasst_prefill, p, stream, q.device)


def paged_prefill_params(q, k_cache, v_cache, block_table, seq_lens, o, *, num_splits=1, lam=None, a=None,
                         softmax_scale=0.0, lse=None, skip_mask=None, crit=None, counters=None, stats_only=False,
                         out_dtype=None, block_q=128, block_k=128):
    """Fills the C params struct for blasst_prefill_paged from tensors (no call).  q [B, Hq, Lq, D]
    (any strides with a contiguous last dim, e.g. a [B, Lq, Hq, D] tensor viewed with permute)."""
    f32, u8, i32, cnt = _torch_types()
    _device_of(q, k_cache, v_cache, block_table, seq_lens, o, lse, skip_mask, crit, counters)
    B, Hq, Lq, D = q.shape
    P, Hkv, page, _ = k_cache.shape
    _shape(k_cache, "k_cache", (P, Hkv, page, D))
    _shape(v_cache, "v_cache", (P, Hkv, v_cache.shape[2], page))
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table has shape {tuple(block_table.shape)}, expected ({B}, max_pages)")
    _shape(seq_lens, "seq_lens", (B,))
    if o is not None:
        _shape(o, "o", (B, Hq, Lq, v_cache.shape[2]))
    max_pages = block_table.shape[1]
    nmask = B * Hq * _cdiv(Lq, max(1, block_q)) * _cdiv(max_pages * page, max(1, block_k))
    p = PagedPrefillParams()
    p.struct_size = ctypes.sizeof(PagedPrefillParams)
    p.q = _ptr(q)
    p.k_cache = _buf(k_cache, "k_cache", (k_cache.dtype,), 0)
    p.v_cache = _buf(v_cache, "v_cache", (k_cache.dtype,), 0)
    p.block_table = _buf(block_table, "block_table", i32, B * max_pages)
    p.seq_lens = _buf(seq_lens, "seq_lens", i32, B)
    p.o = _ptr(o)
    p.lse = _buf(lse, "lse", f32, B * Hq * Lq)
    p.skip_mask = _buf(skip_mask, "skip_mask", u8, nmask)
    p.crit = _buf(crit, "crit", f32, nmask)
    p.counters = _buf(counters, "counters", cnt, 2)
    p.q_stride = _strides3(q)
    p.o_stride = _strides3(o) if o is not None else (ctypes.c_int64 * 3)(0, 0, 0)
    p.thr = _threshold(lam, a)
    p.in_dtype = _dtype_code(q)
    p.out_dtype = _dtype_code(o) if o is not None else (p.in_dtype if out_dtype is None else out_dtype)
    p.batch, p.num_q_heads, p.seqlen_q, p.head_dim_qk = q.shape
    p.num_pages, p.num_kv_heads, p.page_size, _ = k_cache.shape
    p.head_dim_v = v_cache.shape[2]
    p.max_pages_per_seq = block_table.shape[1]
    p.block_q, p.block_k, p.num_splits, p.stats_only = block_q, block_k, num_splits, int(bool(stats_only))
    p.softmax_scale = float(softmax_scale)
    return p


def blasst_prefill_paged(q, k_cache, v_cache, block_table, seq_lens, o, *, stream=None, **kw):
    """Chunked prefill against a paged cache: q [B, Hq, Lq, D] are the last Lq positions of each
    sequence; k_cache [P, Hkv, 16, D], v_cache [P, Hkv, D, 16] (V transposed per page), block_table
    [B, max_pages] int32, seq_lens [B] int32; o [B, Hq, Lq, D].  Keyword args follow the C params."""
    p = paged_prefill_params(q, k_cache, v_cache, block_table, seq_lens, o, **kw)
    _call(lib().blasst_prefill_paged, p, stream, q.device)


def backward_params(q, k, v, o, dout, lse, dq, dk, dv, *, causal, block_q=128, block_k=128, skip_mask=None,
                    workspace=None, softmax_scale=0.0):
    """Fills the C params struct for blasst_prefill_backward from tensors (no call)."""
    f32, u8, _, _ = _torch_types()
    _device_of(q, k, v, o, dout, lse, dq, dk, dv, skip_mask, workspace)
    B, Hq, Lq, D = q.shape
    Hkv, Lk = k.shape[1], k.shape[2]
    Dv = v.shape[3]
    _shape(k, "k", (B, Hkv, Lk, D))
    _shape(v, "v", (B, Hkv, Lk, Dv))
    for t, name, shp in ((o, "o", (B, Hq, Lq, Dv)), (dout, "dout", (B, Hq, Lq, Dv)), (dq, "dq", (B, Hq, Lq, D)),
                         (dk, "dk", (B, Hkv, Lk, D)), (dv, "dv", (B, Hkv, Lk, Dv))):
        _shape(t, name, shp)
    nmask = B * Hq * _cdiv(Lq, max(1, block_q)) * _cdiv(Lk, max(1, block_k))
    p = BackwardParams()
    p.struct_size = ctypes.sizeof(BackwardParams)
    p.q, p.k, p.v, p.o, p.dout = _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout)
    p.lse = _buf(lse, "lse", f32, B * Hq * Lq)
    p.skip_mask = _buf(skip_mask, "skip_mask", u8, nmask)
    p.dq, p.dk, p.dv = _ptr(dq), _ptr(dk), _ptr(dv)
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    p.workspace = _ptr(workspace)
    p.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    p.q_stride, p.k_stride, p.v_stride = _strides3(q), _strides3(k), _strides3(v)
    p.o_stride, p.dout_stride = _strides3(o), _strides3(dout)
    p.dq_stride, p.dk_stride, p.dv_stride = _strides3(dq), _strides3(dk), _strides3(dv)
    p.in_dtype = _dtype_code(q)
    p.grad_dtype = _dtype_code(dq)
    p.o_dtype = _dtype_code(o)
    p.batch, p.num_q_heads, p.seqlen_q, p.head_dim_qk = q.shape
    p.num_kv_heads, p.seqlen_k = k.shape[1], k.shape[2]
    p.head_dim_v = v.shape[3]
    p.causal, p.block_q, p.block_k = int(bool(causal)), block_q, block_k
    p.softmax_scale = float(softmax_scale)
    return p


def blasst_prefill_backward_workspace_size(*args, **kw) -> int:
    p = backward_params(*args, **kw)
    n = lib().blasst_prefill_backward_workspace_size(ctypes.byref(p))
    if n == 0:
        raise BlasstError(ERR_INVALID_ARG, lib().blasst_last_error().decode())
    return int(n)


def blasst_prefill_backward(q, k, v, o, dout, lse, dq, dk, dv, *, stream=None, **kw):
    """Gradients of the sparse prefill with the forward's decisions fixed.  q [B, Hq, Lq, D], k/v
    [B, Hkv, Lk, D], o/dout [B, Hq, Lq, D] (bf16), lse [B, Hq, Lq] fp32 from the forward; dq/dk/dv
    shaped like q/k/v (bf16 or fp32).  Keyword args follow the C params (causal, skip_mask = the
    forward's mask or None for dense, workspace, softmax_scale)."""
    p = backward_params(q, k, v, o, dout, lse, dq, dk, dv, **kw)
    _call(lib().blasst_prefill_backward, p, stream, q.device)


def decode_params(q, k_cache, v_cache, block_table, seq_lens, o, *, page_size, block_k, num_splits,
                  lam=None, a=None, tile_rows=0, head_dim_v=None, softmax_scale=0.0, lse=None,
                  skip_mask=None, crit=None, counters=None, workspace=None, stats_only=False,
                  out_dtype=None, no_decision=False):
    """Fills the C params struct for blasst_decode from tensors (no call).  The decode takes dense
    layouts (no strides), so q, the caches, o and the index arrays must be contiguous; checks one GPU
    for every tensor, matching shapes, and diagnostics buffers of the right dtype and size."""
    f32, u8, i32, cnt = _torch_types()
    _device_of(q, k_cache, v_cache, block_table, seq_lens, o, lse, skip_mask, crit, counters, workspace)
    if q.dim() == 4:
        B, T, Hq, D = q.shape
    else:
        B, Hq, D = q.shape
        T = 1
    P, Hkv, page, _ = k_cache.shape
    _shape(k_cache, "k_cache", (P, Hkv, page, D))
    dv = head_dim_v if head_dim_v is not None else (v_cache.shape[2] if v_cache is not None else D)
    if v_cache is not None:
        _shape(v_cache, "v_cache", (P, Hkv, dv, page))
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table has shape {tuple(block_table.shape)}, expected ({B}, max_pages)")
    _shape(seq_lens, "seq_lens", (B,))
    max_pages = block_table.shape[1]
    G = Hq // max(1, Hkv)
    tr = tile_rows if tile_rows else G
    nmask = B * Hkv * (G // max(1, tr)) * _cdiv(max_pages * page, max(1, block_k))
    p = DecodeParams()
    p.struct_size = ctypes.sizeof(DecodeParams)
    p.q = _buf(q, "q", (q.dtype,), 0)
    p.k_cache = _buf(k_cache, "k_cache", (q.dtype,), 0)
    p.v_cache = _buf(v_cache, "v_cache", (q.dtype,), 0)
    p.block_table = _buf(block_table, "block_table", i32, B * max_pages)
    p.seq_lens = _buf(seq_lens, "seq_lens", i32, B)
    if o is not None:
        if not o.is_contiguous():
            raise ValueError("o must be contiguous")
        if o.numel() != B * T * Hq * dv:
            raise ValueError(f"o holds {o.numel()} elements, expected {B * T * Hq * dv}")
    p.o = _ptr(o)
    p.lse = _buf(lse, "lse", f32, B * T * Hq)
    p.skip_mask = _buf(skip_mask, "skip_mask", u8, nmask)
    p.crit = _buf(crit, "crit", f32, nmask)
    p.counters = _buf(counters, "counters", cnt, 2)
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    p.workspace = _ptr(workspace)
    p.workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    p.thr = _threshold(lam, a, no_decision)
    p.in_dtype = _dtype_code(q)
    p.out_dtype = _dtype_code(o) if o is not None else (p.in_dtype if out_dtype is None else out_dtype)
    if q.dim() == 4:
        p.batch, p.num_q_tokens, p.num_q_heads, p.head_dim_qk = q.shape
    else:
        p.batch, p.num_q_heads, p.head_dim_qk = q.shape
        p.num_q_tokens = 1
    p.num_pages, p.num_kv_heads, page, _ = k_cache.shape
    if page != page_size:
        raise ValueError("k_cache page dimension does not match page_size")
    if head_dim_v is None:
        head_dim_v = v_cache.shape[2] if v_cache is not None else p.head_dim_qk
    p.head_dim_v = head_dim_v
    p.page_size, p.max_pages_per_seq = page_size, block_table.shape[1]
    p.block_k, p.num_splits, p.tile_rows = block_k, num_splits, tile_rows
    p.stats_only = int(bool(stats_only))
    p.softmax_scale = float(softmax_scale)
    return p


def blasst_decode_workspace_size(*args, **kw) -> int:
    p = decode_params(*args, **kw)
    n = lib().blasst_decode_workspace_size(ctypes.byref(p))
    err = lib().blasst_last_error().decode()
    if n == 0 and err:
        raise BlasstError(ERR_INVALID_ARG, err)
    return int(n)


def blasst_decode(q, k_cache, v_cache, block_table, seq_lens, o, *, stream=None, **kw):
    """BLASST paged split-KV decode.  q [B, Hq, D], or [B, T, Hq, D] for T query tokens per sequence
    (the last T positions, bottom-right causal); k_cache [P, Hkv, page, D]; v_cache
    [P, Hkv, Dv, page] (V transposed per page) or None for latent attention (V = K[..., :Dv]);
    block_table [B, max_pages] int32; seq_lens [B] int32; o [B, Hq, Dv] or [B, T, Hq, Dv]."""
    p = decode_params(q, k_cache, v_cache, block_table, seq_lens, o, **kw)
    _call(lib().blasst_decode, p, stream, q.device)


def blasst_decode_no_alloc(q, k_cache, v_cache, block_table, seq_lens, o, *, stream=None, **kw):
    """blasst_decode with the split partials in the library's own per-GPU scratch array instead of
    a workspace (for callers that cannot allocate); same arguments, no `workspace`."""
    if kw.get("workspace") is not None:
        raise ValueError("blasst_decode_no_alloc takes no workspace")
    p = decode_params(q, k_cache, v_cache, block_table, seq_lens, o, **kw)
    _call(lib().blasst_decode_no_alloc, p, stream, q.device)


def blasst_calib_quantile(crit, target_s: float) -> float:
    """ln(lambda) at which a fraction target_s of the critical values lies below (host array)."""
    c = np.ascontiguousarray(np.asarray(crit, dtype=np.float32).ravel())
    out = ctypes.c_double()
    _check_host(lib().blasst_calib_quantile(c.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), c.size,
                                            float(target_s), ctypes.byref(out)))
    return out.value


def blasst_calibrate(L, s, lam):
    """Least-squares fit of ln(lambda * L) = ln(alpha) + beta * s.  Returns (alpha, beta, rmse)."""
    arrs = [np.ascontiguousarray(np.asarray(x, dtype=np.float64).ravel()) for x in (L, s, lam)]
    n = arrs[0].size
    if any(x.size != n for x in arrs):
        raise ValueError("L, s and lam must have the same length")
    dp = ctypes.POINTER(ctypes.c_double)
    alpha, beta, rmse = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    _check_host(lib().blasst_calibrate(*(x.ctypes.data_as(dp) for x in arrs), n, ctypes.byref(alpha),
                                       ctypes.byref(beta), ctypes.byref(rmse)))
    return alpha.value, beta.value, rmse.value


def blasst_lambda_for(alpha: float, beta: float, s: float, L: float) -> float:
    return float(lib().blasst_lambda_for(alpha, beta, s, L))


def _check_host(status: int):
    _check(status)
