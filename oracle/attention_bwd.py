"""Attention backward oracle: float64 gradients of the attention forward.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline use it; the product path never imports it, and it shares no code
with the HIP library.

The pages describe the backward only by its inputs and outputs ("Online
Softmax 算法详解" section 8.3; the online-softmax interview card, section 四,
point ③): it keeps no N x N matrix, recomputes S = scale * Q K^T, recovers
P = exp(S - LSE) from the LSE saved by the forward, and produces dQ, dK, dV.
The gradient itself is the derivative of the forward's plain definition
(O = softmax(S) V over the allowed keys); written out with the chain rule
through V, through the softmax and through S:

    dV = P^T dO
    dP = dO V^T
    D_i = sum_j P_ij dP_ij  (= sum_t dO_it O_it)
    dS = P * (dP - D)        (elementwise; the softmax Jacobian applied to dP)
    dQ = scale * dS K
    dK = scale * dS^T Q

Masked entries have P = 0 and so dS = 0; a row with no allowed key has
P = 0, O = 0 and contributes nothing. Everything is float64 numpy, one
(batch, head) at a time, with the full N x N matrices of that head.
"""
from __future__ import annotations

import numpy as np


def _allowed(N, causal, mask_row):
    a = np.ones((N, N), dtype=bool)
    if causal:
        a &= np.tril(np.ones((N, N), dtype=bool))
    if mask_row is not None:
        a &= (np.asarray(mask_row) != 0)[None, :]
    return a


def attention_bwd(q, k, v, do, scale, causal=False, mask=None):
    """q, k, v, do: [B][H][N][d] arrays (any float dtype, upcast exactly);
    mask: [B][N] (nonzero = valid key) or None.

    Returns dict(dq, dk, dv, o, lse, D) as float64 arrays ([B][H][N][d] for
    the gradients and o, [B][H][N] for lse and D).
    """
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    B, H, N, d = q.shape
    out = {n: np.zeros((B, H, N, d)) for n in ("dq", "dk", "dv", "o")}
    out["lse"] = np.full((B, H, N), -np.inf)
    out["D"] = np.zeros((B, H, N))
    for b in range(B):
        allowed = _allowed(N, causal, None if mask is None else mask[b])
        live = allowed.any(axis=1)
        for h in range(H):
            Q, K, V, dO = q[b, h], k[b, h], v[b, h], do[b, h]
            S = np.where(allowed, scale * (Q @ K.T), -np.inf)
            m = np.where(live, S.max(axis=1, initial=-np.inf), 0.0)
            E = np.exp(S - m[:, None])                 # masked -> 0
            l = E.sum(axis=1)
            P = np.where(live[:, None], E / np.where(live, l, 1.0)[:, None], 0.0)
            O = P @ V
            dV = P.T @ dO
            dP = dO @ V.T
            D = (P * dP).sum(axis=1)
            dS = P * (dP - D[:, None])
            out["dq"][b, h] = scale * (dS @ K)
            out["dk"][b, h] = scale * (dS.T @ Q)
            out["dv"][b, h] = dV
            out["o"][b, h] = O
            out["lse"][b, h] = np.where(live, m + np.log(np.where(live, l, 1.0)), -np.inf)
            out["D"][b, h] = D
    return out
