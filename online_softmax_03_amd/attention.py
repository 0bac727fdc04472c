"""Torch-tensor front end of the C ABI.

`attention_fwd` checks devices, dtypes, shapes and contiguity, allocates O
and LSE with torch (device memory is all torch provides here), and calls
`fa_fwd_ex` on the current HIP stream. All arithmetic happens in libfa.so.
"""
from __future__ import annotations

import math

import torch

from . import capi

_DT = {torch.float32: capi.FA_DTYPE_F32, torch.bfloat16: capi.FA_DTYPE_BF16,
       torch.float16: capi.FA_DTYPE_F16}


class FaError(RuntimeError):
    def __init__(self, status: int):
        super().__init__(f"fa_fwd failed: {capi.fa_strerror(status)} (status {status})")
        self.status = status


def attention_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float | None = None,
                  causal: bool = False, key_padding_mask: torch.Tensor | None = None,
                  out_dtype: torch.dtype | None = None, tile=None, out: torch.Tensor | None = None,
                  lse: torch.Tensor | None = None, num_splits: int | None = None,
                  workspace: torch.Tensor | None = None):
    """O = softmax(scale * Q K^T, masked) V and LSE for [B, H, N, d] tensors.

    scale defaults to 1/sqrt(d). key_padding_mask: [B, N] bool/uint8 on the
    same device, True/nonzero = key valid. out_dtype defaults to q.dtype.
    tile (block_r, block_c) forces a tile shape; None takes the library's
    choice for the shape (`fa_default_tile`). num_splits selects the
    split-KV path (`fa_fwd_splitkv`): an int >= 1, or 0 for the library's
    choice (`fa_splitkv_num_splits`); it runs the base tile (128 x 32 at
    d = 128, 256 x 64 at d = 64), so `tile` must then be None. `workspace` is an optional device
    buffer of at least `fa_splitkv_workspace_bytes` bytes (else one is
    allocated). Returns (o [B, H, N, d], lse [B, H, N] float32).
    """
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must all be [B, H, N, d] with the same shape")
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on the same GPU")
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share a dtype among float32, bfloat16, float16")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out_dtype = q.dtype if out_dtype is None else out_dtype
    if out_dtype not in _DT:
        raise ValueError("unsupported out_dtype")
    mask_ptr = None
    if key_padding_mask is not None:
        if key_padding_mask.shape != (B, N) or key_padding_mask.device != q.device:
            raise ValueError("key_padding_mask must be [B, N] on the same device")
        key_padding_mask = key_padding_mask.to(torch.uint8).contiguous()
        mask_ptr = key_padding_mask.data_ptr()
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != out_dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous [B, H, N, d] tensor of out_dtype on q's device")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous [B, H, N] float32 tensor on q's device")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    if num_splits is not None:
        if tile is not None:
            raise ValueError("the split-KV path runs the base tile; tile must be None")
        if num_splits == 0:
            num_splits = capi.fa_splitkv_num_splits(B, H, N, d, _DT[q.dtype], causal)
            if num_splits < 0:
                raise FaError(num_splits)
        need = capi.fa_splitkv_workspace_bytes(B, H, N, d, num_splits)
        if workspace is None:
            workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
        elif workspace.device != q.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous buffer on the same device")
        ws_bytes = workspace.numel() * workspace.element_size()
        st = capi.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                 B, H, N, d, float(scale), int(bool(causal)), mask_ptr, _DT[q.dtype],
                                 _DT[out_dtype], int(num_splits), workspace.data_ptr(), ws_bytes, stream)
        if st != capi.FA_OK:
            raise FaError(st)
        return out, lse
    st = capi.fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                        B, H, N, d, float(scale), int(bool(causal)), mask_ptr, _DT[q.dtype],
                        _DT[out_dtype], stream, tile)
    if st != capi.FA_OK:
        raise FaError(st)
    return out, lse


def attention_fwd_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, scale: float | None = None,
                      descale_q: float = 1.0, descale_k: float = 1.0, descale_v: float = 1.0,
                      causal: bool = False, key_padding_mask: torch.Tensor | None = None,
                      out_dtype: torch.dtype = torch.bfloat16, max_offset: int = 8,
                      out: torch.Tensor | None = None, lse: torch.Tensor | None = None):
    """Attention forward of FP8 E4M3 inputs (`fa_fwd_fp8`): q, k, v are
    [B, H, N, 128] float8_e4m3fn (or uint8 holding E4M3 codes) whose real
    values are value * descale. O = softmax(scale * (dq Q)(dk K)^T) (dv V) in
    out_dtype (bfloat16, float16 or float32) and LSE [B, H, N] float32.
    max_offset = 8 is the FP8 setting (P formed as 256 P before its E4M3
    rounding); 0 rounds P in [0, 1]. Returns (o, lse)."""
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must all be [B, H, N, d] with the same shape")
    if not (q.is_cuda and k.device == q.device and v.device == q.device):
        raise ValueError("q, k, v must be on the same GPU")
    if any(t.dtype not in (torch.float8_e4m3fn, torch.uint8) for t in (q, k, v)):
        raise ValueError("q, k, v must be float8_e4m3fn (or uint8 E4M3 codes)")
    if any(not t.is_contiguous() for t in (q, k, v)):
        raise ValueError("q, k, v must be contiguous")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out_dtype not in _DT:
        raise ValueError("unsupported out_dtype")
    mask_ptr = None
    if key_padding_mask is not None:
        if key_padding_mask.shape != (B, N) or key_padding_mask.device != q.device:
            raise ValueError("key_padding_mask must be [B, N] on the same device")
        key_padding_mask = key_padding_mask.to(torch.uint8).contiguous()
        mask_ptr = key_padding_mask.data_ptr()
    if out is None:
        out = torch.empty((B, H, N, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if out.shape != q.shape or out.dtype != out_dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous [B, H, N, d] tensor of out_dtype on q's device")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous [B, H, N] float32 tensor on q's device")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = capi.fa_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N, d,
                         float(scale), float(descale_q), float(descale_k), float(descale_v), int(bool(causal)),
                         mask_ptr, _DT[out_dtype], int(max_offset), stream)
    if st != capi.FA_OK:
        raise FaError(st)
    return out, lse


def attention_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor, dout: torch.Tensor,
                  lse: torch.Tensor, scale: float | None = None, causal: bool = False,
                  key_padding_mask: torch.Tensor | None = None, grad_dtype: torch.dtype | None = None,
                  workspace: torch.Tensor | None = None, out=None):
    """dQ, dK, dV of `attention_fwd` from its output `o` and `lse` and the
    output gradient `dout` (all [B, H, N, d] in q's dtype, bf16 or fp16; lse
    [B, H, N] float32). grad_dtype defaults to q.dtype (float32 allowed).
    `out` may give preallocated (dq, dk, dv). Returns (dq, dk, dv)."""
    if q.dim() != 4 or any(t.shape != q.shape for t in (k, v, o, dout)):
        raise ValueError("q, k, v, o, dout must all be [B, H, N, d] with the same shape")
    if any(not t.is_cuda or t.device != q.device for t in (q, k, v, o, dout, lse)):
        raise ValueError("all tensors must be on the same GPU")
    if q.dtype not in (torch.bfloat16, torch.float16) or any(t.dtype != q.dtype for t in (k, v, o, dout)):
        raise ValueError("q, k, v, o, dout must share a dtype among bfloat16, float16")
    if any(not t.is_contiguous() for t in (q, k, v, o, dout, lse)):
        raise ValueError("inputs must be contiguous")
    B, H, N, d = q.shape
    if lse.shape != (B, H, N) or lse.dtype != torch.float32:
        raise ValueError("lse must be a [B, H, N] float32 tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    grad_dtype = q.dtype if grad_dtype is None else grad_dtype
    if grad_dtype not in (q.dtype, torch.float32):
        raise ValueError("grad_dtype must be q.dtype or float32")
    mask_ptr = None
    if key_padding_mask is not None:
        if key_padding_mask.shape != (B, N) or key_padding_mask.device != q.device:
            raise ValueError("key_padding_mask must be [B, N] on the same device")
        key_padding_mask = key_padding_mask.to(torch.uint8).contiguous()
        mask_ptr = key_padding_mask.data_ptr()
    need = capi.fa_bwd_workspace_bytes(B, H, N)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    elif workspace.device != q.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous buffer on the same device")
    if out is None:
        dq, dk, dv = (torch.empty(q.shape, dtype=grad_dtype, device=q.device) for _ in range(3))
    else:
        dq, dk, dv = out
        if any(t.shape != q.shape or t.dtype != grad_dtype or not t.is_contiguous() or t.device != q.device
               for t in out):
            raise ValueError("out must be three contiguous [B, H, N, d] tensors of grad_dtype")
    stream = torch.cuda.current_stream(q.device).cuda_stream
    st = capi.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                     dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, float(scale), int(bool(causal)),
                     mask_ptr, _DT[q.dtype], _DT[grad_dtype], workspace.data_ptr(),
                     workspace.numel() * workspace.element_size(), stream)
    if st != capi.FA_OK:
        raise FaError(st)
    return dq, dk, dv
