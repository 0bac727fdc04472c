"""Shared helpers of the GPU parity tests: run the HIP path through the C ABI
and compare it with the float64 oracle on the same seeded inputs."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from online_softmax_03_amd import attention as A
from online_softmax_03_amd import workloads as W

# Tolerances of the attention forward against the float64 oracle: max abs
# error on O by input dtype, and on LSE; the fully masked row set must match
# exactly, with O exactly 0 and LSE exactly -inf there.
O_TOL = {"bf16": 2e-2, "f16": 5e-3, "f32": 1e-4}
LSE_TOL = 1e-3


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def run_gpu(x: dict, tile=None, canary=True, num_splits=None):
    """Runs the HIP path on inputs `x` (from workloads.generate); with
    `num_splits` the split-KV entry point, on a workspace pre-filled with NaN
    bytes. Returns (O float64 numpy, LSE float64 numpy) on the CPU."""
    dev = torch.device("cuda:0")
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    mask = None if x["mask"] is None else x["mask"].to(dev)
    out_dt = W.DTYPES[x["out_dtype"]]
    o = torch.empty(q.shape, dtype=out_dt, device=dev)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    if canary:
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
    ws = None
    if num_splits is not None:
        B, H, N, d = q.shape
        s = num_splits or A.capi.fa_splitkv_num_splits(B, H, N, d, A._DT[q.dtype], x["causal"])
        ws = torch.full((A.capi.fa_splitkv_workspace_bytes(B, H, N, d, s),), 0xFF, dtype=torch.uint8, device=dev)
        num_splits = s
    A.attention_fwd(q, k, v, scale=x["scale"], causal=x["causal"], key_padding_mask=mask,
                    out_dtype=out_dt, tile=tile, out=o, lse=lse, num_splits=num_splits, workspace=ws)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def compare(O, L, Oref, Lref, fm, in_dtype, what=""):
    """Asserts the parity bar; returns (max |dO|, max |dLSE|)."""
    assert not np.isnan(O).any(), f"{what}: NaN in O"
    assert not np.isnan(L).any(), f"{what}: NaN in LSE"
    dead = np.isneginf(L)
    assert np.array_equal(dead, fm), f"{what}: fully masked rows differ ({dead.sum()} vs {fm.sum()})"
    assert np.all(O[fm] == 0.0), f"{what}: O not exactly 0 on fully masked rows"
    errO = float(np.abs(O - Oref).max()) if O.size else 0.0
    live = ~fm
    errL = float(np.abs(L[live] - Lref[live]).max()) if live.any() else 0.0
    assert errO <= O_TOL[in_dtype], f"{what}: max |dO| = {errO:.3e} > {O_TOL[in_dtype]}"
    assert errL <= LSE_TOL, f"{what}: max |dLSE| = {errL:.3e} > {LSE_TOL}"
    return errO, errL


def check_full(x: dict, tile=None, what="", num_splits=None):
    O, L = run_gpu(x, tile, num_splits=num_splits)
    Oref, Lref, fm = oracle.attention(x["q"], x["k"], x["v"], x["scale"], x["causal"], x["mask"])
    e = compare(O, L, Oref, Lref, fm, x["in_dtype"], what)
    log(f"  {what}: max|dO|={e[0]:.2e} max|dLSE|={e[1]:.2e} masked_rows={int(fm.sum())}")
    return e


def sample_rows(B, H, N, n, seed, causal):
    """Flat row ids: random rows plus the first/last rows of a few heads."""
    g = np.random.default_rng(seed)
    rows = set(g.integers(0, B * H * N, size=n).tolist())
    for bh in {0, B * H - 1, (B * H) // 2}:
        for i in (0, 1, 31, 32, 127, 128, N // 2, N - 2, N - 1):
            if 0 <= i < N:
                rows.add(bh * N + i)
    return np.array(sorted(rows), dtype=np.int64)


def check_sampled(x: dict, rows, tile=None, what="", num_splits=None):
    """Full-size run on the GPU; the oracle computes only `rows`, one head at a
    time (the oracle reads just that head's Q, K, V)."""
    O, L = run_gpu(x, tile, num_splits=num_splits)
    B, H, N, d = x["q"].shape
    Of, Lf = O.reshape(-1, d), L.reshape(-1)
    errs = []
    for bh in sorted(set((rows // N).tolist())):
        b, h = divmod(bh, H)
        rr = rows[(rows // N) == bh]
        sl = lambda t: t[b:b + 1, h:h + 1]  # noqa: E731
        mask = None if x["mask"] is None else x["mask"][b:b + 1]
        Oref, Lref, fm = oracle.attention(sl(x["q"]), sl(x["k"]), sl(x["v"]), x["scale"], x["causal"],
                                          mask, rows=rr - bh * N)
        errs.append(compare(Of[rr], Lf[rr], Oref, Lref, fm, x["in_dtype"], f"{what} head {bh}"))
    e = (max(a for a, _ in errs), max(b for _, b in errs))
    log(f"  {what}: {len(rows)} sampled rows, max|dO|={e[0]:.2e} max|dLSE|={e[1]:.2e}")
    return O, L, e
