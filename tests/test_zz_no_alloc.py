"""fa_fwd_splitkv_noalloc (the split-KV forward on the library's fixed device
scratch) against fa_fwd_splitkv with a caller workspace, through the C ABI.

Both entry points launch the same kernels on the same split, so the outputs
must agree bit for bit; each is also held to the float64 oracle's parity
bar. Two calls in a row, the second on a smaller input with another dtype,
head dim and key mask: the scratch keeps the first call's partials, which
the second must not read.
"""
import numpy as np
import pytest
import torch

import oracle
from online_softmax_03_amd import attention as A
from online_softmax_03_amd import capi
from online_softmax_03_amd import workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

CASES = [
    # (base workload, shape overrides, key lengths, parts)
    ("bf16_causal_n8192_d128", dict(B=1, H=4, N=2048), None, 4),
    ("f16_keypad_n4096_d64", dict(B=3, H=2, N=700), [0, 333, 700], 3),
]


def _run(x, num_splits, noalloc):
    dev = torch.device("cuda:0")
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    B, H, N, d = q.shape
    mask = None if x["mask"] is None else x["mask"].to(dev).contiguous()
    out_dt = W.DTYPES[x["out_dtype"]]
    o = torch.full(q.shape, float("nan"), dtype=out_dt, device=dev)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, N, d,
            float(x["scale"]), int(x["causal"]), None if mask is None else mask.data_ptr(), A._DT[q.dtype],
            A._DT[out_dt], num_splits)
    if noalloc:
        st = capi.fa_fwd_splitkv_noalloc(*args, stream)
    else:
        nbytes = capi.fa_splitkv_workspace_bytes(B, H, N, d, num_splits)
        ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=dev)
        st = capi.fa_fwd_splitkv(*args, ws.data_ptr(), nbytes, stream)
    assert st == capi.FA_OK, capi.fa_strerror(st)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def test_noalloc_matches_workspace_entry_point_twice():
    for base, over, lens, parts in CASES:
        w = W.BY_NAME[base].with_shape(**over)
        x = W.generate(w, lens=None if lens is None else torch.tensor(lens, dtype=torch.int64))
        U.log(f"case noalloc {base} B,H,N,d={w.B},{w.H},{w.N},{w.d} parts={parts}")
        need = capi.fa_splitkv_workspace_bytes(w.B, w.H, w.N, w.d, parts)
        assert 0 < need <= capi.FA_NOALLOC_SCRATCH_BYTES
        O1, L1 = _run(x, parts, noalloc=True)
        O0, L0 = _run(x, parts, noalloc=False)
        assert np.array_equal(O1, O0), "O differs from fa_fwd_splitkv"
        assert np.array_equal(L1, L0), "LSE differs from fa_fwd_splitkv"
        Oref, Lref, fm = oracle.attention(x["q"], x["k"], x["v"], x["scale"], x["causal"], x["mask"])
        eo, el = U.compare(O1, L1, Oref, Lref, fm, x["in_dtype"], f"noalloc {base}")
        U.log(f"  noalloc {base}: identical to the workspace call; max|dO|={eo:.2e} max|dLSE|={el:.2e}")
