"""ctypes binding of include/fa.h, with the same names and arguments.

Argument marshalling only: every step of the attention forward runs in the
HIP kernels of libfa.so. Importing this module does not load the library;
the first call does, and raises if libfa.so has not been built.
"""
from __future__ import annotations

import ctypes
import os
import threading

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")

FA_DTYPE_F32 = 0
FA_DTYPE_BF16 = 1
FA_DTYPE_F16 = 2

FA_OK = 0
FA_ERR_NULL = -1
FA_ERR_SHAPE = -2
FA_ERR_HEADDIM = -3
FA_ERR_DTYPE = -4
FA_ERR_SCALE = -5
FA_ERR_ALIGN = -6
FA_ERR_TILE = -7
FA_ERR_LAUNCH = -8
FA_ERR_SPLITS = -9
FA_ERR_WORKSPACE = -10
FA_ERR_OFFSET = -11
FA_ERR_SCRATCH = -12

FA_MAX_SPLITS = 64
FA_NOALLOC_SCRATCH_BYTES = 64 << 20

# Every symbol include/fa.h declares.
EXPORTS = ("fa_fwd", "fa_fwd_ex", "fa_default_tile", "fa_tile_supported", "fa_splitkv_workspace_bytes",
           "fa_splitkv_num_splits", "fa_fwd_splitkv", "fa_fwd_splitkv_noalloc", "fa_fwd_fp8", "fa_bwd_workspace_bytes", "fa_bwd", "fa_softmax_fwd",
           "fa_strerror")


class fa_tile(ctypes.Structure):
    _fields_ = [("block_r", ctypes.c_int), ("block_c", ctypes.c_int)]


_lock = threading.Lock()
_lib = None

_P = ctypes.c_void_p
_I = ctypes.c_int
_FWD_ARGS = [_P, _P, _P, _P, _P, _I, _I, _I, _I, ctypes.c_float, _I, _P, _I, _I, _P]


def library():
    """The loaded libfa.so; raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with `python -m online_softmax_03_amd.build` "
                    "(there is no fallback implementation)")
            lib = ctypes.CDLL(LIB_PATH)
            lib.fa_fwd.restype = _I
            lib.fa_fwd.argtypes = _FWD_ARGS
            lib.fa_fwd_ex.restype = _I
            lib.fa_fwd_ex.argtypes = _FWD_ARGS + [ctypes.POINTER(fa_tile)]
            lib.fa_default_tile.restype = _I
            lib.fa_default_tile.argtypes = [_I, _I, _I, _I, _I, _I, _I, _I, ctypes.POINTER(fa_tile)]
            lib.fa_tile_supported.restype = _I
            lib.fa_tile_supported.argtypes = [_I, _I, _I, ctypes.POINTER(fa_tile)]
            lib.fa_splitkv_workspace_bytes.restype = ctypes.c_size_t
            lib.fa_splitkv_workspace_bytes.argtypes = [_I, _I, _I, _I, _I]
            lib.fa_splitkv_num_splits.restype = _I
            lib.fa_splitkv_num_splits.argtypes = [_I, _I, _I, _I, _I, _I]
            lib.fa_fwd_splitkv.restype = _I
            lib.fa_fwd_splitkv.argtypes = _FWD_ARGS[:-1] + [_I, _P, ctypes.c_size_t, _P]
            lib.fa_fwd_splitkv_noalloc.restype = _I
            lib.fa_fwd_splitkv_noalloc.argtypes = _FWD_ARGS[:-1] + [_I, _P]
            lib.fa_fwd_fp8.restype = _I
            lib.fa_fwd_fp8.argtypes = ([_P] * 5 + [_I, _I, _I, _I] + [ctypes.c_float] * 4 +
                                       [_I, _P, _I, _I, _P])
            lib.fa_bwd_workspace_bytes.restype = ctypes.c_size_t
            lib.fa_bwd_workspace_bytes.argtypes = [_I, _I, _I]
            lib.fa_bwd.restype = _I
            lib.fa_bwd.argtypes = ([_P] * 9 + [_I, _I, _I, _I, ctypes.c_float, _I, _P, _I, _I, _P,
                                                ctypes.c_size_t, _P])
            lib.fa_softmax_fwd.restype = _I
            lib.fa_softmax_fwd.argtypes = [_P, _P, _P, ctypes.c_longlong, _I, _I, _I, _P]
            lib.fa_strerror.restype = ctypes.c_char_p
            lib.fa_strerror.argtypes = [_I]
            _lib = lib
        return _lib


def fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, key_padding_mask, in_dtype, out_dtype,
           stream) -> int:
    """Pointers are integers (device addresses) or None; returns the status."""
    return library().fa_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, key_padding_mask,
                            in_dtype, out_dtype, stream)


def fa_fwd_ex(q, k, v, o, lse, B, H, N, d, scale, causal, key_padding_mask, in_dtype, out_dtype,
              stream, tile=None) -> int:
    t = None
    if tile is not None:
        t = ctypes.byref(fa_tile(int(tile[0]), int(tile[1])))
    return library().fa_fwd_ex(q, k, v, o, lse, B, H, N, d, scale, causal, key_padding_mask,
                               in_dtype, out_dtype, stream, t)


def fa_default_tile(B, H, N, d, in_dtype, out_dtype, causal, has_mask):
    """Returns (status, (block_r, block_c))."""
    t = fa_tile()
    st = library().fa_default_tile(B, H, N, d, in_dtype, out_dtype, causal, has_mask, ctypes.byref(t))
    return st, (t.block_r, t.block_c)


def fa_tile_supported(d, in_dtype, out_dtype, tile) -> int:
    return library().fa_tile_supported(d, in_dtype, out_dtype, ctypes.byref(fa_tile(*tile)))


def fa_splitkv_workspace_bytes(B, H, N, d, num_splits) -> int:
    return int(library().fa_splitkv_workspace_bytes(B, H, N, d, num_splits))


def fa_splitkv_num_splits(B, H, N, d, in_dtype, causal) -> int:
    return library().fa_splitkv_num_splits(B, H, N, d, in_dtype, int(causal))


def fa_fwd_splitkv(q, k, v, o, lse, B, H, N, d, scale, causal, key_padding_mask, in_dtype, out_dtype,
                   num_splits, workspace, workspace_bytes, stream) -> int:
    return library().fa_fwd_splitkv(q, k, v, o, lse, B, H, N, d, scale, causal, key_padding_mask,
                                    in_dtype, out_dtype, num_splits, workspace, workspace_bytes, stream)


def fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, N, d, scale, causal, key_padding_mask, in_dtype, out_dtype,
                           num_splits, stream) -> int:
    return library().fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, N, d, scale, causal, key_padding_mask,
                                            in_dtype, out_dtype, num_splits, stream)


def fa_fwd_fp8(q, k, v, o, lse, B, H, N, d, scale, descale_q, descale_k, descale_v, causal, key_padding_mask,
               out_dtype, max_offset, stream) -> int:
    return library().fa_fwd_fp8(q, k, v, o, lse, B, H, N, d, scale, descale_q, descale_k, descale_v, causal,
                                key_padding_mask, out_dtype, max_offset, stream)


def fa_bwd_workspace_bytes(B, H, N) -> int:
    return int(library().fa_bwd_workspace_bytes(B, H, N))


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, key_padding_mask, in_dtype, grad_dtype,
           workspace, workspace_bytes, stream) -> int:
    return library().fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, key_padding_mask,
                            in_dtype, grad_dtype, workspace, workspace_bytes, stream)


def fa_softmax_fwd(x, y, lse, rows, cols, in_dtype, out_dtype, stream) -> int:
    return library().fa_softmax_fwd(x, y, lse, rows, cols, in_dtype, out_dtype, stream)


def fa_strerror(status) -> str:
    return library().fa_strerror(int(status)).decode()
