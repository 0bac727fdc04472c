"""The backward tests' reference with D taken from the rounded O (d_shift in
test_gpu_bwd.py), checked on the CPU against a direct evaluation: dS =
P (dP - rowsum(dO * O_rounded)), dQ = scale dS K, dK = scale dS^T Q."""
import numpy as np
import pytest
import torch

import oracle
from online_softmax_03_amd import workloads as W
from tests.test_gpu_bwd import C, C3, C5, _oracle_inputs, d_shift


@pytest.mark.parametrize("over,mask", [
    (dict(B=3, H=1, N=2, d=128, in_dtype="f16", out_dtype="f16", causal=False, q_dist=("normal", 2.0),
          k_dist=("normal", 2.0), key_padding=False, seed=151003), "general"),
    (dict(B=2, H=2, N=37, d=64, in_dtype="bf16", out_dtype="bf16", causal=True, key_padding=False, seed=7), None),
    (dict(B=2, H=1, N=50, d=64, in_dtype="f16", out_dtype="f16", causal=False, seed=8), "padding"),
])
def test_shifted_reference_is_the_gradient_with_d_from_the_rounded_o(over, mask):
    w = C[C3 if mask != "padding" else C5].with_shape(**over)
    g = torch.Generator().manual_seed(over["seed"] + 1)
    lens = torch.tensor([0, over["N"] // 2]) if mask == "padding" else None
    x = W.generate(w, lens=lens)
    if mask == "general":
        x["mask"] = (torch.rand((w.B, w.N), generator=g) < 0.6).to(torch.uint8)
    do = W.generate_dout(w)
    ref, o, lse = _oracle_inputs(x, do)
    sh = d_shift(x, do, o, ref)
    q, k, v = (x[n].double().numpy() for n in ("q", "k", "v"))
    dO, od = do.double().numpy(), o.double().numpy()
    s = np.einsum("bhid,bhjd->bhij", q, k) * x["scale"]
    N = w.N
    allow = np.ones(s.shape, dtype=bool)
    if x["causal"]:
        allow &= np.tril(np.ones((N, N), dtype=bool))
    if x["mask"] is not None:
        allow &= (x["mask"].numpy() != 0)[:, None, None, :]
    L = ref["lse"][..., None]
    p = np.where(allow & np.isfinite(L), np.exp(np.where(allow, s, 0.0) - np.where(np.isfinite(L), L, 0.0)), 0.0)
    ds = p * (np.einsum("bhid,bhjd->bhij", dO, v) - (dO * od).sum(-1)[..., None])
    assert np.abs(sh["dq"] - x["scale"] * np.einsum("bhij,bhjd->bhid", ds, k)).max() <= 1e-12
    assert np.abs(sh["dk"] - x["scale"] * np.einsum("bhij,bhid->bhjd", ds, q)).max() <= 1e-12
    assert np.array_equal(sh["dv"], ref["dv"])
    # and with the exact O the shift is zero
    sh0 = d_shift(x, do, torch.from_numpy(ref["o"]), ref)
    assert np.abs(sh0["dq"] - ref["dq"]).max() <= 1e-12 and np.abs(sh0["dk"] - ref["dk"]).max() <= 1e-12
