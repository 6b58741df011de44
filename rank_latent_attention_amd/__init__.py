"""Python binding of libqsvd.so, the C ABI of the QSVD latent-attention path on gfx950.

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  PyTorch supplies device memory (tensors) and the current stream.
The functions carry the C names and follow include/qsvd.h; tensors stand in
for device pointers (None for NULL).  A failing call raises QsvdError with
the library's message.  There is no fallback: if the library is not built
the import of a function raises.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "F32", "BF16", "I8", "I4", "QsvdError", "lib", "library_path",
    "qsvd_quantize_latent", "qsvd_project", "qsvd_pack_weight",
    "qsvd_decode_workspace_bytes", "qsvd_decode_default_splits", "qsvd_decode_attn",
    "qsvd_decode_attn_noalloc",
    "qsvd_decode_explicit_workspace_bytes", "qsvd_decode_attn_explicit",
    "qsvd_decode_headwise_workspace_bytes", "qsvd_decode_attn_headwise",
    "qsvd_status_string", "qsvd_last_error", "timing", "EXPORTED",
]

F32, BF16, I8, I4 = 0, 1, 2, 3
_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libqsvd.so")

# every symbol include/qsvd.h declares
EXPORTED = (
    "qsvd_quantize_latent", "qsvd_project", "qsvd_pack_weight", "qsvd_decode_workspace_bytes",
    "qsvd_decode_attn", "qsvd_decode_attn_noalloc", "qsvd_decode_default_splits",
    "qsvd_decode_explicit_workspace_bytes",
    "qsvd_decode_attn_explicit", "qsvd_decode_headwise_workspace_bytes",
    "qsvd_decode_attn_headwise", "qsvd_status_string", "qsvd_last_error",
    "qsvd_timing_begin", "qsvd_timing_end",
)


class QsvdError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status}: {detail}")
        self.status = status


class KernelTime(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 32), ("launches", ctypes.c_int32),
                ("total_ms", ctypes.c_double)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use; raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise ImportError(f"{library_path} is missing: build it with "
                          "`python -m rank_latent_attention_amd.build`")
    L = ctypes.CDLL(library_path)
    vp, i32, i64, f32p, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    L.qsvd_quantize_latent.argtypes = [vp, i32, i64, i32, i32, i32, i32, vp, f32p, vp]
    L.qsvd_project.argtypes = [vp, i32, f32p, i64, i32, vp, i32, f32p, i32, vp, i32, vp]
    L.qsvd_pack_weight.argtypes = [vp, i32, i32, i32, vp, vp]
    L.qsvd_decode_workspace_bytes.argtypes = [i32, i64, i32, i32, i32, i32, i32]
    L.qsvd_decode_workspace_bytes.restype = sz
    L.qsvd_decode_default_splits.argtypes = [i32, i64, i32, i32, i32, i32]
    L.qsvd_decode_attn.argtypes = [vp, i32, vp, i32, f32p, i32, vp, vp, i32, f32p, f32p, i32, i64,
                                   i32, i32, i32, ctypes.c_float, i32, vp, i32, vp, sz, vp]
    L.qsvd_decode_attn_noalloc.argtypes = [vp, i32, vp, i32, f32p, i32, vp, vp, i32, f32p, f32p, i32,
                                           i64, i32, i32, i32, ctypes.c_float, i32, vp, i32, vp]
    L.qsvd_decode_explicit_workspace_bytes.argtypes = [i32, i64, i32, i32, i32]
    L.qsvd_decode_explicit_workspace_bytes.restype = sz
    L.qsvd_decode_attn_explicit.argtypes = [vp, i32, vp, i32, vp, vp, i32, i32, i64, i32, i32, i32,
                                            ctypes.c_float, f32p, f32p, vp, i32, vp, sz, vp]
    L.qsvd_decode_headwise_workspace_bytes.argtypes = [i32, i64, i32, i32, i32, i32, i32]
    L.qsvd_decode_headwise_workspace_bytes.restype = sz
    L.qsvd_decode_attn_headwise.argtypes = [vp, i32, vp, i32, vp, vp, i32, i32, i64, i32, i32, i32,
                                            i32, ctypes.c_float, f32p, f32p, i32, vp, i32, vp, sz, vp]
    L.qsvd_status_string.argtypes = [i32]
    L.qsvd_status_string.restype = ctypes.c_char_p
    L.qsvd_last_error.argtypes = []
    L.qsvd_last_error.restype = ctypes.c_char_p
    L.qsvd_timing_begin.argtypes = [i32]
    L.qsvd_timing_end.argtypes = [ctypes.POINTER(KernelTime), i32, ctypes.POINTER(i32)]
    for name in ("qsvd_quantize_latent", "qsvd_project", "qsvd_pack_weight", "qsvd_decode_attn",
                 "qsvd_decode_attn_noalloc",
                 "qsvd_decode_attn_explicit", "qsvd_decode_attn_headwise", "qsvd_timing_begin", "qsvd_timing_end", "qsvd_decode_default_splits"):
        getattr(L, name).restype = i32
    _lib = L
    return L


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(int(stream))
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check(status: int, where: str):
    if status != 0:
        raise QsvdError(status, where, lib().qsvd_last_error().decode())


def qsvd_status_string(status: int) -> str:
    return lib().qsvd_status_string(status).decode()


def qsvd_last_error() -> str:
    return lib().qsvd_last_error().decode()


def qsvd_quantize_latent(x, in_dtype, M, n, hadamard_block, code_dtype, group, codes, scales,
                         stream=None):
    _check(lib().qsvd_quantize_latent(_ptr(x), in_dtype, M, n, hadamard_block, code_dtype, group,
                                      _ptr(codes), _ptr(scales), _stream(stream)),
           "qsvd_quantize_latent")


def qsvd_project(X, x_dtype, x_scale, M, E, W_packed, w_dtype, col_scale, r, C, c_dtype,
                 stream=None):
    _check(lib().qsvd_project(_ptr(X), x_dtype, _ptr(x_scale), M, E, _ptr(W_packed), w_dtype,
                              _ptr(col_scale), r, _ptr(C), c_dtype, _stream(stream)),
           "qsvd_project")


def qsvd_pack_weight(W, dt, rows, cols, packed, stream=None):
    _check(lib().qsvd_pack_weight(_ptr(W), dt, rows, cols, _ptr(packed), _stream(stream)),
           "qsvd_pack_weight")


def qsvd_decode_workspace_bytes(b, L, r, heads, d, c_dtype, splits=0) -> int:
    return int(lib().qsvd_decode_workspace_bytes(b, L, r, heads, d, c_dtype, splits))


def qsvd_decode_default_splits(b, L, r, heads, d, c_dtype) -> int:
    return int(lib().qsvd_decode_default_splits(b, L, r, heads, d, c_dtype))


def qsvd_decode_attn(q, q_dtype, C, c_dtype, c_scales, c_group, Wu_k, Wu_v, wu_dtype, wu_scale_k,
                     wu_scale_v, b, L, r, heads, d, softmax_scale, splits, O, o_dtype, workspace,
                     workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().qsvd_decode_attn(_ptr(q), q_dtype, _ptr(C), c_dtype, _ptr(c_scales), c_group,
                                  _ptr(Wu_k), _ptr(Wu_v), wu_dtype, _ptr(wu_scale_k),
                                  _ptr(wu_scale_v), b, L, r, heads, d, float(softmax_scale), splits,
                                  _ptr(O), o_dtype, _ptr(workspace), workspace_bytes,
                                  _stream(stream)),
           "qsvd_decode_attn")


def qsvd_decode_attn_noalloc(q, q_dtype, C, c_dtype, c_scales, c_group, Wu_k, Wu_v, wu_dtype,
                             wu_scale_k, wu_scale_v, b, L, r, heads, d, softmax_scale, splits, O,
                             o_dtype, stream=None):
    _check(lib().qsvd_decode_attn_noalloc(_ptr(q), q_dtype, _ptr(C), c_dtype, _ptr(c_scales), c_group,
                                          _ptr(Wu_k), _ptr(Wu_v), wu_dtype, _ptr(wu_scale_k),
                                          _ptr(wu_scale_v), b, L, r, heads, d, float(softmax_scale),
                                          splits, _ptr(O), o_dtype, _stream(stream)),
           "qsvd_decode_attn_noalloc")


def qsvd_decode_explicit_workspace_bytes(b, L, r, heads, d) -> int:
    return int(lib().qsvd_decode_explicit_workspace_bytes(b, L, r, heads, d))


def qsvd_decode_attn_explicit(q, q_dtype, C, c_dtype, Wk_packed, Wv_packed, wu_dtype, b, L, r,
                              heads, d, softmax_scale, rope_cos, rope_sin, O, o_dtype, workspace,
                              workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().qsvd_decode_attn_explicit(_ptr(q), q_dtype, _ptr(C), c_dtype, _ptr(Wk_packed),
                                           _ptr(Wv_packed), wu_dtype, b, L, r, heads, d,
                                           float(softmax_scale), _ptr(rope_cos), _ptr(rope_sin),
                                           _ptr(O), o_dtype, _ptr(workspace), workspace_bytes,
                                           _stream(stream)),
           "qsvd_decode_attn_explicit")


def qsvd_decode_headwise_workspace_bytes(b, L, heads, d, rk, rv, splits=0) -> int:
    return int(lib().qsvd_decode_headwise_workspace_bytes(b, L, heads, d, rk, rv, splits))


def qsvd_decode_attn_headwise(q, q_dtype, C, c_dtype, BK_t, BV, b_dtype, b, L, heads, d, rk, rv,
                              softmax_scale, rope_cos, rope_sin, splits, O, o_dtype, workspace,
                              workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().qsvd_decode_attn_headwise(_ptr(q), q_dtype, _ptr(C), c_dtype, _ptr(BK_t), _ptr(BV),
                                           b_dtype, b, L, heads, d, rk, rv, float(softmax_scale),
                                           _ptr(rope_cos), _ptr(rope_sin), splits, _ptr(O),
                                           o_dtype, _ptr(workspace), workspace_bytes,
                                           _stream(stream)),
           "qsvd_decode_attn_headwise")


class timing:
    """Context manager around qsvd_timing_begin / qsvd_timing_end.

    ``result`` maps kernel name -> (launches, total_ms) after the block exits."""

    def __init__(self, max_launches: int = 4096):
        self.max_launches = max_launches
        self.result = {}

    def __enter__(self):
        _check(lib().qsvd_timing_begin(self.max_launches), "qsvd_timing_begin")
        return self

    def __exit__(self, *exc):
        arr = (KernelTime * 64)()
        n = ctypes.c_int32(0)
        _check(lib().qsvd_timing_end(arr, 64, ctypes.byref(n)), "qsvd_timing_end")
        self.result = {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms)
                       for i in range(min(n.value, 64))}
        return False
