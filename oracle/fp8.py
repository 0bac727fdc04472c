"""E4M3 (OCP FP8) values and the FP8 attention forward, in float64.

TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
benchmark's CPU baseline, never by the product path; it shares no code with
the HIP library.

"Online Softmax 算法详解" section 6 runs the attention forward with FP8 E4M3
operands and scales the unnormalised probabilities by 2^Max_offset before they
are rounded to E4M3 (section 6.2), compensating the row sum afterwards
(section 6.3). The result is still the plain attention of the inputs; only the
rounding of P differs. So:

- `e4m3_decode(b)`: the value of each E4M3 byte, by the format's definition
  (OCP 8-bit floating point, E4M3): bit 7 sign, bits 6..3 exponent with bias
  7, bits 2..0 mantissa; exponent field 0 encodes subnormals m/8 * 2^-6; the
  pattern S.1111.111 is NaN; there are no infinities. Largest finite value
  1.75 * 2^8 = 448 (the range the page quotes in section 6.1).
- `e4m3_round(x)`: the nearest E4M3 value, ties to the even mantissa; a
  magnitude of 464 or more (halfway from 448 to 480, the step the format
  gives to NaN) becomes NaN, i.e. the conversion does not saturate.
- `attention_fp8(...)`: the plain definition over dequantized inputs,
  O = softmax(scale * (dq Q)(dk K)^T, masked) (dv V), LSE = ln sum exp(...),
  through the float64 three-pass oracle.
- `online_attention_e4m3(...)`: the blocked recurrence of one row with the
  probabilities formed as P' = 2^((s - m) log2(e) + Max_offset), rounded to
  E4M3 for the P V product, the row sum taken from the unrounded P' and
  divided by 2^Max_offset at the end (section 6.3). It models the rounding
  that section 6.1 warns about, to pin that the offset reduces it.
"""
from __future__ import annotations

import math

import numpy as np

from .attention import attention as _attention_oracle

E4M3_MAX = 448.0
# Halfway between 448 and 480: from here on the nearest step is the NaN code.
E4M3_OVERFLOW = 464.0


def e4m3_decode(b) -> np.ndarray:
    """float64 values of E4M3 bytes (any integer array, or a torch uint8 /
    float8_e4m3fn tensor)."""
    b = _as_bytes(b).astype(np.int64)
    sign = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    val = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    val = sign * val
    return np.where((b & 0x7F) == 0x7F, np.nan, val)


def _all_values() -> np.ndarray:
    """The 127 non-negative finite E4M3 values in increasing order (codes 0..126)."""
    return e4m3_decode(np.arange(0, 127))


def e4m3_round(x) -> np.ndarray:
    """Round float64 values to the nearest E4M3 value (ties to even mantissa).

    The candidates are the format's finite values themselves (from
    `e4m3_decode`); between two neighbours the nearer wins and a tie goes to
    the one with an even code (even mantissa). |x| >= 464 and NaN give NaN.
    """
    x = np.asarray(x, dtype=np.float64)
    vals = _all_values()
    a = np.abs(x)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, vals.size - 1)  # first value >= a
    lo = np.clip(hi - 1, 0, vals.size - 1)
    dlo = a - vals[lo]
    dhi = vals[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    pick_hi |= a <= vals[0]
    r = np.where(pick_hi, vals[hi], vals[lo])
    r = np.where(a >= E4M3_OVERFLOW, np.nan, r)
    r = np.where(np.isnan(x), np.nan, r)
    return np.copysign(r, x)


def e4m3_encode(x) -> np.ndarray:
    """E4M3 byte codes of `e4m3_round(x)` (NaN -> 0x7F with the sign of x)."""
    r = e4m3_round(x)
    vals = _all_values()
    code = np.searchsorted(vals, np.where(np.isnan(r), 0.0, np.abs(r)))
    code = np.where(np.isnan(r), 0x7F, code)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def attention_fp8(q, k, v, scale, descale_q=1.0, descale_k=1.0, descale_v=1.0, causal=False, mask=None,
                  rows=None, nthreads=0):
    """Exact (float64) attention forward of FP8 inputs.

    q, k, v: [B][H][N][d] E4M3 bytes (numpy uint8, or torch uint8 /
    float8_e4m3fn). The real inputs are descale * value. Since the scores are
    bilinear in Q and K and the output linear in V,
        softmax(scale * (dq Q)(dk K)^T) (dv V) = dv * softmax((scale dq dk) Q K^T) V,
    so the decoded values (exact in float32: 4 significant bits) go to the
    three-pass oracle with the float64 scale scale*dq*dk, and O is multiplied
    by dv. Returns (O, LSE, fully_masked) like `oracle.attention`.
    """
    qf, kf, vf = (e4m3_decode(t) for t in (q, k, v))
    if np.isnan(qf).any() or np.isnan(kf).any() or np.isnan(vf).any():
        raise ValueError("NaN codes in the FP8 inputs")
    s = float(scale) * float(descale_q) * float(descale_k)
    o, lse, fm = _attention_oracle(qf.astype(np.float32), kf.astype(np.float32), vf.astype(np.float32), s,
                                   causal=causal, mask=mask, rows=rows, nthreads=nthreads)
    return o * float(descale_v), lse, fm


def online_attention_e4m3(s, v, block: int, max_offset: int):
    """One query row by the blocked recurrence with E4M3-rounded probabilities.

    s: 1-D float64 scores (already scaled, -inf = masked); v: [len(s)][dv].
    Per block, in the order of "在线Softmax算法解析" section 3.2: m_new =
    max(m, max s_block), alpha = exp(m - m_new), l and O scaled by alpha,
    P' = exp(s - m_new) * 2^max_offset (the + Max_offset inside exp2 of
    "Online Softmax 算法详解" section 6.2), l += sum P' (unrounded), O +=
    e4m3_round(P') @ v. At the end l is divided by 2^max_offset (section 6.3)
    and O / l carries the factor 2^max_offset of both, so out = O / l_raw.
    Returns (out, lse).
    """
    s = np.asarray(s, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    m, l = -math.inf, 0.0
    O = np.zeros(v.shape[1])
    off = float(2 ** max_offset)
    for j0 in range(0, s.size, block):
        sb, vb = s[j0:j0 + block], v[j0:j0 + block]
        m_new = max(m, float(np.max(sb)))
        if m_new == -math.inf:
            continue
        alpha = 0.0 if m == -math.inf else math.exp(m - m_new)
        l *= alpha
        O *= alpha
        p = np.exp(sb - m_new) * off
        l += float(np.sum(p))
        O += e4m3_round(p) @ vb
        m = m_new
    if not l > 0:
        return np.zeros(v.shape[1]), -math.inf
    return O / l, m + math.log(l / off)


def _as_bytes(b) -> np.ndarray:
    try:
        import torch
        if isinstance(b, torch.Tensor):
            t = b.detach().cpu()
            if t.dtype != torch.uint8:
                t = t.contiguous().view(torch.uint8)
            return t.numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(b)
