"""Score-level reference routines: safe softmax and the online (m, l, O) recurrence.

TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
benchmark's CPU baseline, never by the product path.

All arithmetic is numpy float64 unless a float32 run is requested explicitly
(to show what the recurrence does in the GPU's accumulator precision).
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def safe_softmax(s):
    """Three-pass safe softmax of a 1-D score vector.

    Follows "在线Softmax算法解析" section 1.1 and "Online Softmax 算法详解"
    section 2.1: pass 1 takes the maximum m, pass 2 the normaliser
    l = sum exp(s_i - m), pass 3 divides. Entries equal to -inf are excluded
    (masked); if every entry is -inf the row is fully masked and the result is
    p = 0, l = 0, lse = -inf (the all-masked convention of "Online Softmax
    算法详解" sections 7.2-7.3).

    Returns (p, m, l, lse) with lse = m + ln(l) (section 8.1 of the same page).
    """
    s = np.asarray(s, dtype=np.float64)
    if s.size == 0 or not np.any(np.isfinite(s)):
        return np.zeros_like(s), NEG_INF, 0.0, NEG_INF
    m = np.max(s)                       # pass 1
    e = np.exp(s - m)                   # exp(-inf) = 0 removes masked entries
    l = float(np.sum(e))                # pass 2
    p = e / l                           # pass 3
    return p, float(m), l, float(m + np.log(l))


def online_two_pass(x):
    """The online softmax in two passes over a 1-D vector, element by element.

    Follows "Online Softmax 算法详解" section 2.2: pass 1 fuses the maximum
    and the normaliser (for each element, m_new = max(m, x_i), then
    l = exp(m - m_new) * l + exp(x_i - m_new), m = m_new), pass 2 writes
    exp(x_i - m) / l. The -inf guard of section 7.1 of that page replaces the
    reference point by 0 while everything seen is -inf. Pure Python over
    float64 scalars, for small inputs only.

    Returns (y list, m, l, lse).
    """
    import math

    m, l = -math.inf, 0.0
    for xi in x:                                   # pass 1
        xi = float(xi)
        m_new = max(m, xi)
        ref = 0.0 if m_new == -math.inf else m_new
        l = (math.exp(m - ref) if m != -math.inf else 0.0) * l + math.exp(xi - ref)
        m = m_new
    if m == -math.inf:
        return [0.0] * len(x), m, 0.0, -math.inf
    y = [math.exp(float(xi) - m) / l for xi in x]  # pass 2
    return y, m, l, m + math.log(l)


def online_softmax(blocks, v_blocks=None, dtype=np.float64):
    """The online recurrence over a sequence of score blocks.

    State (m, l, O) starts at (-inf, 0, 0) ("在线Softmax算法解析" section 3.2).
    For each block, in the pages' order:
      1. m_block = max of the block
      2. m_cand  = max(m, m_block)
      3. alpha   = exp(m - m_cand)  (the rescale factor of section 2.2 there)
      4. l <- l * alpha,  O <- O * alpha
      5. P = exp(S_block - m_cand)
      6. l <- l + sum(P),  O <- O + P @ V_block
      7. m <- m_cand
    and the result is O / l. When m_cand is still -inf (everything seen so
    far masked) the reference point used in the exponents is 0 instead, which
    is the -inf guard described in "Online Softmax 算法详解" section 7.1; it
    keeps exp(-inf - (-inf)) from producing NaN.

    blocks: list of 1-D score arrays (may contain -inf for masked scores).
    v_blocks: list of [len(block), dv] arrays, or None (then O is not kept).
    dtype: arithmetic precision (float64 by default; float32 to mimic an
    fp32 accumulator).

    Returns dict(m, l, O, out, lse, trace) where trace holds per block
    (m_block, m_cand, alpha, l_scaled, l_after, P, O).
    """
    dt = np.dtype(dtype)
    m = dt.type(NEG_INF)
    l = dt.type(0.0)
    O = None
    trace = []
    for bi, sb in enumerate(blocks):
        sb = np.asarray(sb, dtype=dt)
        m_block = np.max(sb) if sb.size else dt.type(NEG_INF)
        m_cand = max(m, m_block)
        ref = dt.type(0.0) if m_cand == NEG_INF else m_cand
        alpha = np.exp(dt.type(m - ref)) if m != NEG_INF else dt.type(0.0)
        l = dt.type(l * alpha)
        l_scaled = l
        if v_blocks is not None:
            vb = np.asarray(v_blocks[bi], dtype=dt)
            if O is None:
                O = np.zeros(vb.shape[1], dtype=dt)
            O = (O * alpha).astype(dt)
        P = np.exp((sb - ref).astype(dt)).astype(dt)
        l = dt.type(l + np.sum(P, dtype=dt))
        if v_blocks is not None:
            O = (O + (P[:, None] * vb).sum(axis=0, dtype=dt)).astype(dt)
        m = m_cand
        trace.append(dict(m_block=float(m_block), m_cand=float(m_cand), alpha=float(alpha),
                          l_scaled=float(l_scaled), l_after=float(l), P=P.astype(np.float64),
                          O=None if O is None else O.astype(np.float64)))
    if l == 0 or np.isnan(l):
        out = None if O is None else np.zeros_like(O)
        lse = NEG_INF
    else:
        out = None if O is None else (O / l).astype(dt)
        lse = float(m) + float(np.log(np.float64(l)))
    return dict(m=float(m), l=float(l), O=O, out=out, lse=lse, trace=trace)


def merge_states(m1, l1, O1, m2, l2, O2):
    """Combine two partial states computed over disjoint key sets.

    m = max(m1, m2); l = l1 exp(m1 - m) + l2 exp(m2 - m); O likewise, as in
    the block-combination equations of "Online Softmax (interview card)" (the
    airsota page, section 三). A side whose m is -inf contributes nothing.
    """
    m = max(m1, m2)
    if m == NEG_INF:
        return NEG_INF, 0.0, np.zeros_like(np.asarray(O1, dtype=np.float64))
    a1 = 0.0 if m1 == NEG_INF else np.exp(m1 - m)
    a2 = 0.0 if m2 == NEG_INF else np.exp(m2 - m)
    O = np.asarray(O1, dtype=np.float64) * a1 + np.asarray(O2, dtype=np.float64) * a2
    return m, l1 * a1 + l2 * a2, O


def online_attention(q, k, v, scale, causal=False, mask=None, block_c=64, dtype=np.float64):
    """Blocked attention forward by the online recurrence, rows vectorised.

    q, k, v: [B][H][N][d] arrays (any float dtype; upcast to `dtype`).
    The score matrix S = scale * Q K^T is formed with a library matmul, then
    the keys are walked in blocks of `block_c` with the seven steps of
    `online_softmax` applied to every query row at once (each row keeps its
    own (m, l, O), "在线Softmax算法解析" section 3.3). Masked scores are -inf.

    Returns (O [B][H][N][d], lse [B][H][N], fully_masked [B][H][N] bool).
    """
    dt = np.dtype(dtype)
    q = np.asarray(q, dtype=dt)
    k = np.asarray(k, dtype=dt)
    v = np.asarray(v, dtype=dt)
    B, H, N, d = q.shape
    S = (np.matmul(q, np.swapaxes(k, -1, -2)) * dt.type(scale)).astype(dt)
    allow = np.ones((B, 1, N, N), dtype=bool)
    if causal:
        allow = allow & np.tril(np.ones((N, N), dtype=bool))[None, None]
    if mask is not None:
        allow = allow & (np.asarray(mask) != 0)[:, None, None, :]
    S = np.where(allow, S, dt.type(NEG_INF))
    m = np.full((B, H, N), NEG_INF, dtype=dt)
    l = np.zeros((B, H, N), dtype=dt)
    O = np.zeros((B, H, N, d), dtype=dt)
    with np.errstate(invalid="ignore"):
        for j0 in range(0, N, block_c):
            Sb = S[..., j0:j0 + block_c]
            m_cand = np.maximum(m, Sb.max(axis=-1))
            ref = np.where(m_cand == NEG_INF, dt.type(0.0), m_cand)
            alpha = np.where(m == NEG_INF, dt.type(0.0), np.exp(m - ref)).astype(dt)
            l = l * alpha
            O = O * alpha[..., None]
            P = np.exp(Sb - ref[..., None]).astype(dt)
            l = (l + P.sum(axis=-1, dtype=dt)).astype(dt)
            O = (O + np.matmul(P, v[..., j0:j0 + block_c, :])).astype(dt)
            m = m_cand
    dead = (l == 0) | np.isnan(l)
    with np.errstate(divide="ignore", invalid="ignore"):
        out = np.where(dead[..., None], dt.type(0.0), O / l[..., None]).astype(dt)
        lse = np.where(dead, NEG_INF, m.astype(np.float64) + np.log(l.astype(np.float64)))
    return out, lse, dead
