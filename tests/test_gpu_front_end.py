"""The torch front ends refuse tensors the kernels cannot use (needs a GPU for
the inputs): outputs, statistics and workspaces on the host or a different
layout are rejected before anything is launched, so a host pointer never
reaches a kernel."""
import pytest
import torch

from online_softmax_03_amd import attention as A
from online_softmax_03_amd import softmax as S
from online_softmax_03_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def _qkv(dtype=torch.bfloat16, shape=(1, 2, 64, 128)):
    g = torch.Generator().manual_seed(3)
    return [torch.randn(shape, generator=g).to(dtype).to(DEV) for _ in range(3)]


def test_forward_rejects_host_or_misshapen_outputs():
    q, k, v = _qkv()
    cases = [
        dict(out=torch.empty(q.shape, dtype=q.dtype)),                               # host O
        dict(lse=torch.empty(q.shape[:3], dtype=torch.float32)),                     # host LSE
        dict(out=torch.empty(q.shape, dtype=torch.float16, device=DEV)),             # wrong dtype
        dict(out=torch.empty((1, 2, 128, 64), dtype=q.dtype, device=DEV).transpose(2, 3)),  # not contiguous
        dict(lse=torch.empty((1, 2, 63), dtype=torch.float32, device=DEV)),          # wrong shape
        dict(num_splits=2, workspace=torch.empty(1 << 20, dtype=torch.uint8)),       # host workspace
    ]
    for kw in cases:
        with pytest.raises(ValueError):
            A.attention_fwd(q, k, v, **kw)
    with pytest.raises(ValueError):
        A.attention_fwd(q, k.cpu(), v)                                                # host input
    with pytest.raises(ValueError):
        A.attention_fwd(q, k, v, key_padding_mask=torch.ones((1, 64), dtype=torch.bool))  # host mask
    torch.cuda.synchronize()


def test_fp8_forward_rejects_host_outputs():
    w = W.FP8_BY_NAME["fp8_causal_n8192_d128"].with_shape(B=1, H=2, N=64)
    x = W.generate(w)
    q, k, v = (x[n].to(DEV) for n in ("q", "k", "v"))
    for kw in (dict(out=torch.empty(q.shape, dtype=torch.bfloat16)),
               dict(lse=torch.empty(q.shape[:3], dtype=torch.float32))):
        with pytest.raises(ValueError):
            A.attention_fwd_fp8(q, k, v, **kw)
    torch.cuda.synchronize()


def test_backward_rejects_host_workspace_and_gradients():
    q, k, v = _qkv()
    o, lse = A.attention_fwd(q, k, v, causal=True)
    dout = torch.randn(q.shape, generator=torch.Generator().manual_seed(4)).to(q.dtype).to(DEV)
    with pytest.raises(ValueError):
        A.attention_bwd(q, k, v, o, dout, lse, causal=True, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    with pytest.raises(ValueError):
        A.attention_bwd(q, k, v, o, dout, lse, causal=True,
                        out=tuple(torch.empty(q.shape, dtype=q.dtype) for _ in range(3)))
    with pytest.raises(ValueError):
        A.attention_bwd(q, k, v, o, dout, lse.cpu(), causal=True)
    torch.cuda.synchronize()


def test_softmax_rejects_host_outputs():
    x = torch.randn((8, 100), generator=torch.Generator().manual_seed(5)).to(DEV)
    with pytest.raises(ValueError):
        S.softmax_rows(x, out=torch.empty(x.shape))
    with pytest.raises(ValueError):
        S.softmax_rows(x, lse=torch.empty(8, dtype=torch.float32))
    torch.cuda.synchronize()
