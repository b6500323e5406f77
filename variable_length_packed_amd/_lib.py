"""ctypes view of libva_varlen.so (the C ABI declared in include/va_varlen.h, include/va_kvcache.h
and include/va_pack.h)."""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libva_varlen.so")

VA_OK, VA_ERR_INVALID, VA_ERR_UNSUPPORTED, VA_ERR_WORKSPACE, VA_ERR_HIP = range(5)
VA_F32, VA_BF16, VA_F16 = 0, 1, 2

# Every symbol the headers under include/ declare.
EXPORTS = ("va_varlen_fwd", "va_varlen_bwd", "va_varlen_fwd_workspace_size",
           "va_varlen_bwd_workspace_size", "va_status_string", "va_last_error", "va_version",
           "va_timing_start", "va_timing_stop", "va_pack_metadata", "va_unpad", "va_pad",
           "va_kvcache_fwd", "va_kvcache_fwd_workspace_size", "va_varlen_fwd_noalloc",
           "va_varlen_fwd_bwdplan", "va_varlen_bwd_planned")
VA_PACK_MAX_TENSORS = 4


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("launches", ctypes.c_int), ("total_ms", ctypes.c_double)]


class PackTensor(ctypes.Structure):
    _fields_ = [("padded", ctypes.c_void_p), ("packed", ctypes.c_void_p), ("row_bytes", ctypes.c_int64)]

_lib = None

_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_f = ctypes.c_float
_i64p = ctypes.POINTER(ctypes.c_int64)


def load() -> ctypes.CDLL:
    """Load the library once.  Raises if it has not been built: there is no fallback path."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m variable_length_packed_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    lib.va_varlen_fwd.restype = ctypes.c_int
    # q, k, v, cu_q, cu_k, max_q, max_k, scale, causal, bias, bias_stride, out, lse,
    # qkv_row_stride, workspace, workspace_bytes, batch, total_q, total_k, hq, hkv, d, dtype, stream
    lib.va_varlen_fwd.argtypes = [_p, _p, _p, _p, _p, _i32, _i32, _f, ctypes.c_int, _p, _i64p, _p, _p,
                                  _i64p, _p, ctypes.c_size_t, _i32, _i32, _i32, _i32, _i32, _i32,
                                  ctypes.c_int, _p]
    # the forward's arguments plus the backward's workspace pair after its own
    lib.va_varlen_fwd_bwdplan.restype = ctypes.c_int
    lib.va_varlen_fwd_bwdplan.argtypes = [_p, _p, _p, _p, _p, _i32, _i32, _f, ctypes.c_int, _p, _i64p, _p,
                                          _p, _i64p, _p, ctypes.c_size_t, _p, ctypes.c_size_t, _i32, _i32,
                                          _i32, _i32, _i32, _i32, ctypes.c_int, _p]
    # the forward's arguments without the workspace pair
    lib.va_varlen_fwd_noalloc.restype = ctypes.c_int
    lib.va_varlen_fwd_noalloc.argtypes = [_p, _p, _p, _p, _p, _i32, _i32, _f, ctypes.c_int, _p, _i64p, _p,
                                          _p, _i64p, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_int, _p]
    lib.va_varlen_bwd.restype = ctypes.c_int
    # dout, q, k, v, out, lse, cu_q, cu_k, max_q, max_k, scale, causal, bias, bias_stride,
    # dq, dk, dv, dbias, dbias_stride, qkv_row_stride, workspace, workspace_bytes, batch, total_q,
    # total_k, hq, hkv, d, dtype, grad_dtype, stream
    lib.va_varlen_bwd.argtypes = [_p, _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _f, ctypes.c_int, _p,
                                  _i64p, _p, _p, _p, _p, _i64p, _i64p, _p, ctypes.c_size_t, _i32, _i32,
                                  _i32, _i32, _i32, _i32, ctypes.c_int, ctypes.c_int, _p]
    lib.va_varlen_bwd_planned.restype = ctypes.c_int
    lib.va_varlen_bwd_planned.argtypes = list(lib.va_varlen_bwd.argtypes)
    lib.va_varlen_fwd_workspace_size.restype = ctypes.c_size_t
    lib.va_varlen_fwd_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                 ctypes.c_int]
    lib.va_varlen_bwd_workspace_size.restype = ctypes.c_size_t
    lib.va_varlen_bwd_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                                 ctypes.c_int, ctypes.c_int]
    lib.va_status_string.restype = ctypes.c_char_p
    lib.va_status_string.argtypes = [ctypes.c_int]
    lib.va_last_error.restype = ctypes.c_char_p
    lib.va_last_error.argtypes = []
    lib.va_version.restype = ctypes.c_int
    lib.va_version.argtypes = []
    lib.va_timing_start.restype = ctypes.c_int
    lib.va_timing_start.argtypes = [ctypes.c_int]
    lib.va_timing_stop.restype = ctypes.c_int
    lib.va_timing_stop.argtypes = [ctypes.POINTER(KernelTime), ctypes.c_int]
    lib.va_pack_metadata.restype = ctypes.c_int
    lib.va_pack_metadata.argtypes = [_p, _i32, _i32, _p, _p, _p, _p, _p, _p]
    lib.va_unpad.restype = ctypes.c_int
    lib.va_unpad.argtypes = [ctypes.POINTER(PackTensor), _i32, _p, _p, _i32, _i32, ctypes.c_int64, _p]
    lib.va_kvcache_fwd.restype = ctypes.c_int
    lib.va_kvcache_fwd.argtypes = [_p, _p, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _f, ctypes.c_int,
                                   _p, _p, _p, ctypes.c_size_t, _i32, _i32, _i32, _i32, _i32,
                                   ctypes.c_int, _p]
    lib.va_kvcache_fwd_workspace_size.restype = ctypes.c_size_t
    lib.va_kvcache_fwd_workspace_size.argtypes = [_i32, _i32, _i32, _i32, _i32, _i32, ctypes.c_int]
    lib.va_pad.restype = ctypes.c_int
    lib.va_pad.argtypes = [ctypes.POINTER(PackTensor), _i32, _p, _i32, _i32, ctypes.c_int64, _p]
    _lib = lib
    return lib


def strides_arg(strides):
    """HOST int64[n] for bias_stride (4) or qkv_row_stride (3), or None."""
    if strides is None:
        return None
    arr = (ctypes.c_int64 * len(strides))(*[int(s) for s in strides])
    return arr
