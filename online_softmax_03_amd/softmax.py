"""Torch-tensor front end of `fa_softmax_fwd` (row softmax with the online
normaliser). Checks devices, dtypes and shapes, allocates the outputs with
torch, and calls the C ABI on the current HIP stream; the arithmetic runs in
libfa.so.
"""
from __future__ import annotations

import torch

from . import capi
from .attention import _DT, FaError


def softmax_rows(x: torch.Tensor, out_dtype: torch.dtype | None = None, out: torch.Tensor | None = None,
                 lse: torch.Tensor | None = None, want_lse: bool = True):
    """Softmax over the last dimension of a contiguous GPU tensor.

    Returns (y, lse): y has x's shape and `out_dtype` (default x.dtype); lse
    is float32 with shape x.shape[:-1] (natural log; -inf on rows with no
    finite entry), or None when want_lse is False and no lse is given.
    """
    if x.dim() < 1 or x.numel() == 0:
        raise ValueError("x must have at least one element")
    if not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous GPU tensor")
    if x.dtype not in _DT:
        raise ValueError("x must be float32, bfloat16 or float16")
    out_dtype = x.dtype if out_dtype is None else out_dtype
    if out_dtype not in _DT:
        raise ValueError("unsupported out_dtype")
    cols = x.shape[-1]
    rows = x.numel() // cols
    if out is None:
        out = torch.empty(x.shape, dtype=out_dtype, device=x.device)
    if out.shape != x.shape or out.dtype != out_dtype or not out.is_contiguous() or out.device != x.device:
        raise ValueError("out must be a contiguous tensor of x's shape and out_dtype on x's device")
    if lse is None and want_lse:
        lse = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    if lse is not None and (lse.shape != x.shape[:-1] or lse.dtype != torch.float32 or not lse.is_contiguous()
                            or lse.device != x.device):
        raise ValueError("lse must be a contiguous float32 tensor of shape x.shape[:-1]")
    stream = torch.cuda.current_stream(x.device).cuda_stream
    st = capi.fa_softmax_fwd(x.data_ptr(), out.data_ptr(), None if lse is None else lse.data_ptr(), rows, cols,
                             _DT[x.dtype], _DT[out_dtype], stream)
    if st != capi.FA_OK:
        raise FaError(st)
    return out, lse
