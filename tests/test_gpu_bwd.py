"""Parity of the HIP attention backward (fa_bwd) with the float64 oracle
(needs a GPU).

The backward takes the forward's O and LSE as inputs. The small cases give
it the oracle's own O (rounded to the input dtype) and LSE (rounded to
float32), so nothing the oracle computes depends on the HIP path; the
full-size case feeds it the HIP forward's O and LSE, as a training step
would, and the oracle recomputes everything from Q, K, V, dO alone.

Bar: for each of dQ, dK, dV, max |HIP - oracle| <= tol * max |oracle| of
that tensor, tol = 2e-2 for bf16 inputs and 5e-3 for fp16 (P and dS are
rounded to the input dtype as MFMA operands, O enters D = rowsum(dO * O)
rounded, and bf16 output adds 2^-9 relative), with max |oracle| floored at
1e-2 for a gradient that is exactly zero (one key: dS = 0, and the GPU's
D - dP cancellation leaves rounding noise); gradients of masked keys and
of queries with no allowed key are exactly 0. Where the backward is given
the oracle's O rounded to the input dtype, the reference takes D from that
same O (d_shift: an exact, linear correction of dQ and dK computed from the
oracle's P); under a peaked softmax dP - D is small and the rounding of O
alone can move dQ by its own size. Outputs are pre-filled with NaN so an
unwritten element fails.
"""
import numpy as np
import pytest
import torch

import oracle
from online_softmax_03_amd import attention as A
from online_softmax_03_amd import workloads as W
from tests.gpu_util import log

pytestmark = pytest.mark.gpu

TOL = {"bf16": 2e-2, "f16": 5e-3}
C = {w.name: w for w in W.WORKLOADS}
TINY, C2, C3, C4, C5 = (w.name for w in W.WORKLOADS)


def run_bwd(x, do, o, lse, grad_dtype=None):
    dev = torch.device("cuda:0")
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    mask = None if x["mask"] is None else x["mask"].to(dev)
    gd = None if grad_dtype is None else W.DTYPES[grad_dtype]
    dq, dk, dv = A.attention_bwd(q, k, v, o.to(dev), do.to(dev), lse.to(dev), scale=x["scale"], causal=x["causal"],
                                 key_padding_mask=mask, grad_dtype=gd)
    torch.cuda.synchronize()
    return [t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv)]


def d_shift(x, do, o, ref):
    """The oracle's gradients with D = rowsum(dO * O) taken from the O the
    backward is given (`o`, the oracle's O rounded to the input dtype)
    instead of the exact O. dS_ij = P_ij (dP_ij - D_i) is linear in D, so a
    change dD_i = rowsum(dO * (o - O))_i changes dS_ij by -P_ij dD_i, dQ_i by
    -scale dD_i sum_j P_ij K_j and dK_j by -scale sum_i P_ij dD_i Q_i (dV =
    P^T dO has no D), exactly, with P from the oracle's LSE. Under a peaked
    softmax dP - D is small and this term can reach the size of dQ itself
    (seen on random draws at N = 2 and 4 with logits of standard deviation
    4), while every operation of the kernel is as accurate as its dtype."""
    q, k = (x[n].double().numpy() for n in ("q", "k"))
    dd = (do.double().numpy() * (o.double().numpy() - ref["o"])).sum(-1)  # [B, H, N]
    s = np.einsum("bhid,bhjd->bhij", q, k) * x["scale"]
    N = q.shape[2]
    allow = np.ones(s.shape, dtype=bool)
    if x["causal"]:
        allow &= np.tril(np.ones((N, N), dtype=bool))
    if x["mask"] is not None:
        allow &= (x["mask"].numpy() != 0)[:, None, None, :]
    lse = ref["lse"][..., None]
    p = np.where(allow & np.isfinite(lse), np.exp(np.where(allow, s, 0.0) - np.where(np.isfinite(lse), lse, 0.0)), 0.0)
    out = dict(ref)
    out["dq"] = ref["dq"] - x["scale"] * dd[..., None] * np.einsum("bhij,bhjd->bhid", p, k)
    out["dk"] = ref["dk"] - x["scale"] * np.einsum("bhij,bhid->bhjd", p, dd[..., None] * q)
    return out


def check(got, ref, in_dtype, what, dead_q=None, dead_k=None):
    errs = []
    for name, g, r in zip(("dq", "dk", "dv"), got, (ref["dq"], ref["dk"], ref["dv"])):
        assert not np.isnan(g).any(), f"{what}: NaN in {name}"
        scale = max(float(np.abs(r).max()), 1e-2)
        e = float(np.abs(g - r).max()) / scale
        assert e <= TOL[in_dtype], f"{what}: {name} max|d|/max|ref| = {e:.3e} > {TOL[in_dtype]}"
        errs.append(e)
    if dead_q is not None:
        assert np.all(got[0][dead_q] == 0.0), f"{what}: dq of queries with no allowed key not 0"
    if dead_k is not None:
        assert np.all(got[1][dead_k] == 0.0) and np.all(got[2][dead_k] == 0.0), f"{what}: masked keys not 0"
    return errs


SMALL = [
    ("bf16_causal_d128_n333", C3, dict(B=1, H=3, N=333), None),
    ("bf16_noncausal_d128_n190", C3, dict(B=2, H=1, N=190, causal=False), None),
    ("bf16_d64_n300", C2, dict(B=2, H=2, N=300, out_dtype="bf16"), None),
    ("bf16_causal_d64_n100", C2, dict(B=1, H=2, N=100, causal=True, out_dtype="bf16"), None),
    ("bf16_causal_long_logits_n500", C4, dict(B=1, H=2, N=500), None),
    ("f16_keypad_d64_n257", C5, dict(B=6, H=2, N=257), [0, 1, 63, 64, 256, 257]),
    ("f16_keypad_causal_d128_n130", C5, dict(B=3, H=2, N=130, d=128, causal=True), [0, 5, 130]),
    ("f16_d64_n1", C5, dict(B=1, H=1, N=1, key_padding=False), None),
    ("bf16_d128_n31", C3, dict(B=1, H=1, N=31), None),
    ("bf16_d128_n64_causal", C3, dict(B=2, H=1, N=64), None),
    # causal launches over 32 and 16 heads deal their tiles over groups of 4
    # and 2 heads
    ("bf16_causal_d128_h32_n300", C3, dict(B=2, H=16, N=300), None),
    ("f16_keypad_causal_d64_h16_n600", C5, dict(B=2, H=8, N=600, causal=True), [600, 417]),
]


def _oracle_inputs(x, do):
    ref = oracle.attention_bwd(x["q"].double().numpy(), x["k"].double().numpy(), x["v"].double().numpy(),
                               do.double().numpy(), x["scale"], x["causal"],
                               None if x["mask"] is None else x["mask"].numpy())
    o = torch.from_numpy(ref["o"]).to(W.DTYPES[x["in_dtype"]])
    lse = torch.from_numpy(ref["lse"]).float()
    return ref, o, lse


@pytest.mark.parametrize("grad", ["same", "f32"])
@pytest.mark.parametrize("ident,base,over,lens", SMALL, ids=[s[0] for s in SMALL])
def test_small_shapes_every_element(ident, base, over, lens, grad):
    w = C[base].with_shape(**over)
    x = W.generate(w, lens=None if lens is None else torch.tensor(lens, dtype=torch.int64))
    do = W.generate_dout(w)
    log(f"case bwd {ident} grad={grad}: B,H,N,d={w.B},{w.H},{w.N},{w.d} {w.in_dtype} causal={w.causal}")
    ref, o, lse = _oracle_inputs(x, do)
    got = run_bwd(x, do, o, lse, None if grad == "same" else "f32")
    dead_q = np.isneginf(ref["lse"])
    dead_k = None
    if x["mask"] is not None:
        dead_k = np.broadcast_to((x["mask"].numpy() == 0)[:, None, :], dead_q.shape)
    e = check(got, d_shift(x, do, o, ref), w.in_dtype, ident, dead_q, dead_k)
    log(f"  rel errors dq={e[0]:.2e} dk={e[1]:.2e} dv={e[2]:.2e}")


@pytest.mark.parametrize("d,dtype,causal", [(64, "f16", False), (128, "bf16", True)])
def test_general_key_mask(d, dtype, causal):
    N, B, H = 211, 4, 2
    w = C[C5].with_shape(B=B, H=H, N=N, d=d, in_dtype=dtype, out_dtype=dtype, causal=causal, key_padding=False)
    x = W.generate(w)
    g = torch.Generator().manual_seed(123 + d)
    mask = (torch.rand((B, N), generator=g) > 0.5).to(torch.uint8)
    mask[1] = 0
    mask[2] = 0
    mask[2, 150] = 1
    mask[3, ::7] = 1
    x["mask"] = mask
    do = W.generate_dout(w)
    ref, o, lse = _oracle_inputs(x, do)
    got = run_bwd(x, do, o, lse)
    dead_k = np.broadcast_to((mask.numpy() == 0)[:, None, :], ref["lse"].shape)
    check(got, d_shift(x, do, o, ref), dtype, f"general mask d={d} {dtype} causal={causal}",
          np.isneginf(ref["lse"]), dead_k)


def test_full_size_headline_heads():
    """B=2, H=32, N=8192, d=128, bf16, causal: the HIP forward's O and LSE go
    into the HIP backward; two whole heads are checked against the oracle."""
    w = C[C3]
    log(f"case bwd {C3}: full size")
    x = W.generate(w)
    do = W.generate_dout(w)
    dev = torch.device("cuda:0")
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    o, lse = A.attention_fwd(q, k, v, scale=x["scale"], causal=True)
    dq, dk, dv = A.attention_bwd(q, k, v, o, do.to(dev), lse, scale=x["scale"], causal=True)
    torch.cuda.synchronize()
    for (b, h) in ((0, 0), (w.B - 1, w.H - 1)):
        sl = lambda t: t[b:b + 1, h:h + 1].double().numpy()  # noqa: E731
        ref = oracle.attention_bwd(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(do), x["scale"], True)
        got = [t[b:b + 1, h:h + 1].float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv)]
        e = check(got, ref, "bf16", f"{C3} head ({b},{h})")
        log(f"  head ({b},{h}): rel errors dq={e[0]:.2e} dk={e[1]:.2e} dv={e[2]:.2e}")


def _draw(i):
    r = np.random.default_rng(50000 + i)
    d = int(r.choice([64, 128]))
    dtype = ["bf16", "f16"][int(r.integers(2))]
    return dict(d=d, dtype=dtype, grad=["same", "f32"][int(r.integers(2))], causal=bool(r.integers(2)),
                B=int(r.integers(1, 4)), H=int(r.integers(1, 5)), N=max(1, int(np.exp(r.uniform(0.0, np.log(500.0))))),
                qk=float(r.choice([0.5, 1.0, 2.0])), mask=["none", "padding", "general"][int(r.integers(3))],
                seed=51000 + i)


RANDOM = [_draw(i) for i in range(100)]


@pytest.mark.parametrize("i", range(len(RANDOM)))
def test_random_shapes_every_element(i):
    """Seeded random draws: head dim, dtype, gradient dtype, causal, 1-3
    batches of 1-4 heads, length log-uniform in 1 ... 500, logit spread, and
    no key mask, a padding mask (random lengths, 0 and N included) or a
    random non-contiguous one; every element against the oracle."""
    c = RANDOM[i]
    w = C[C3].with_shape(B=c["B"], H=c["H"], N=c["N"], d=c["d"], in_dtype=c["dtype"], out_dtype=c["dtype"],
                         causal=c["causal"], q_dist=("normal", c["qk"]), k_dist=("normal", c["qk"]),
                         key_padding=False, seed=c["seed"])
    g = torch.Generator().manual_seed(c["seed"] + 1)
    lens = None
    if c["mask"] == "padding":
        lens = torch.randint(0, c["N"] + 1, (c["B"],), generator=g, dtype=torch.int64)
    x = W.generate(w, lens=lens)
    if c["mask"] == "general":
        x["mask"] = (torch.rand((c["B"], c["N"]), generator=g) < 0.6).to(torch.uint8)
    do = W.generate_dout(w)
    log(f"case bwd random {i}: {c}")
    ref, o, lse = _oracle_inputs(x, do)
    got = run_bwd(x, do, o, lse, None if c["grad"] == "same" else "f32")
    dead_k = None
    if x["mask"] is not None:
        dead_k = np.broadcast_to((x["mask"].numpy() == 0)[:, None, :], ref["lse"].shape)
    e = check(got, d_shift(x, do, o, ref), c["dtype"], f"bwd random {i}", np.isneginf(ref["lse"]), dead_k)
    log(f"  rel errors dq={e[0]:.2e} dk={e[1]:.2e} dv={e[2]:.2e}")
