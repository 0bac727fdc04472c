"""Python front end of the float64 attention oracle (attention_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline use it; the product path never imports it.

The C file is compiled with the system C compiler into oracle/liboracle.so
(no GPU toolchain involved). `build()` always recompiles; `load()` compiles
only when the library is missing or older than its source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attention_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None


def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile the oracle (plain C, float64, OpenMP). Returns the .so path."""
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = open_library(_LIB)
        return _lib


def open_library(path):
    """Open an oracle shared library at `path` and declare its signatures."""
    lib = ctypes.CDLL(path)
    lib.oracle_attention_rows.restype = ctypes.c_int
    lib.oracle_attention_rows.argtypes = [
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_double, ctypes.c_int, ctypes.c_void_p, ctypes.c_longlong,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    return lib


def _as_f32(x) -> np.ndarray:
    """Exact float32 container of the input values (bf16/fp16/fp32 all embed)."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().to(torch.float32).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def attention(q, k, v, scale, causal=False, mask=None, rows=None, nthreads=0, lib=None):
    """Exact (float64) attention forward for all rows, or for selected rows.

    q, k, v: [B][H][N][d] (torch CPU tensors or numpy arrays, any of
    fp32/bf16/fp16). scale: the float32 scale value the GPU receives (used
    as its exact float64 upcast). mask: None or [B][N], nonzero = key valid.
    rows: None for every row, else flat indices (b*H + h)*N + i.

    Returns (O float64, lse float64, fully_masked bool): shaped [B][H][N][d],
    [B][H][N] for all rows, or [len(rows)][d], [len(rows)] for a selection.
    `lib` overrides the shared library (a handle from `open_library`).
    """
    lib = load() if lib is None else lib
    qf, kf, vf = _as_f32(q), _as_f32(k), _as_f32(v)
    B, H, N, d = qf.shape
    if kf.shape != qf.shape or vf.shape != qf.shape:
        raise ValueError("q, k, v must share the shape [B][H][N][d]")
    mk = None
    if mask is not None:
        mk = np.ascontiguousarray(_as_u8(mask))
        if mk.shape != (B, N):
            raise ValueError("mask must be [B][N]")
    if rows is None:
        nrows = B * H * N
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        nrows = rows_arr.size
    o = np.zeros((nrows, d), dtype=np.float64)
    lse = np.zeros(nrows, dtype=np.float64)
    fm = np.zeros(nrows, dtype=np.uint8)
    rc = lib.oracle_attention_rows(
        qf.ctypes.data, kf.ctypes.data, vf.ctypes.data,
        None if mk is None else mk.ctypes.data,
        B, H, N, d, float(scale), int(bool(causal)),
        None if rows_arr is None else rows_arr.ctypes.data, nrows,
        o.ctypes.data, lse.ctypes.data, fm.ctypes.data, int(nthreads))
    if rc != 0:
        raise RuntimeError(f"oracle_attention_rows failed with {rc}")
    if rows is None:
        return o.reshape(B, H, N, d), lse.reshape(B, H, N), fm.reshape(B, H, N).astype(bool)
    return o, lse, fm.astype(bool)


def _as_u8(x) -> np.ndarray:
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach().cpu().to(torch.uint8).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.uint8)


def max_threads() -> int:
    return int(load().oracle_max_threads())


def fully_masked_rows(B, H, N, causal=False, mask=None):
    """The rows with no allowed key, [B][H][N] bool, from the definition of
    the allowed set alone (no scores): row (b, h, i) attends key j when
    (not causal or j <= i) and (mask is None or mask[b][j] != 0), and is fully
    masked when no j qualifies ("Online Softmax 算法详解" sections 7.2-7.3
    give such rows O = 0 and LSE = -inf)."""
    if mask is None:
        valid = np.ones((B, N), dtype=bool)
    else:
        valid = _as_u8(mask).reshape(B, N) != 0
    # number of allowed keys of row i: valid keys among j <= i (causal) or all
    seen = np.cumsum(valid, axis=1)
    count = seen if causal else np.repeat(seen[:, -1:], N, axis=1)
    return np.broadcast_to((count == 0)[:, None, :], (B, H, N)).copy()
