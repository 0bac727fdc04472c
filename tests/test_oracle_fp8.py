"""Pins of the FP8 (E4M3) oracle: the byte decoder and rounding against the
format's definition and torch's float8_e4m3fn conversion (a library
routine), the FP8 attention oracle against torch's float64 scaled-dot-product
attention on independently dequantized inputs, and the Max_offset recurrence
of "Online Softmax 算法详解" section 6 against closed forms.

Every check is a function of the implementation it checks, so the planted
mistakes at the end can show that each check catches a plausible error.
"""
import math

import numpy as np
import pytest
import torch

from oracle import fp8 as F
from oracle import softmax_ref as sr
from online_softmax_03_amd import workloads as W


def _torch_decode(codes) -> np.ndarray:
    t = torch.as_tensor(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def _torch_round(x) -> np.ndarray:
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


# ---------------------------------------------------------------- checkers

def check_decode(decode) -> bool:
    codes = np.arange(256)
    got = decode(codes)
    ref = _torch_decode(codes)
    if not np.array_equal(np.isnan(got), np.isnan(ref)):
        return False
    ok = ~np.isnan(ref)
    if not np.array_equal(got[ok], ref[ok]):
        return False
    # values the format's definition fixes by hand
    spot = {0x38: 1.0, 0x7E: 448.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6,
            0x0F: 1.875 * 2.0 ** -6, 0x40: 2.0, 0xC2: -2.5, 0x77: 1.875 * 2.0 ** 7, 0x78: 256.0}
    vals = decode(np.array(list(spot)))
    if not np.array_equal(vals, np.array(list(spot.values()))):
        return False
    z = decode(np.array([0x00, 0x80]))
    return z[0] == 0.0 and z[1] == 0.0 and not np.signbit(z[0]) and np.signbit(z[1]) and \
        bool(np.isnan(decode(np.array([0x7F, 0xFF]))).all())


def check_round(rnd) -> bool:
    g = np.random.default_rng(7)
    finite = _torch_decode(np.arange(0, 127))
    mids = (finite[:-1] + finite[1:]) / 2                    # exact ties
    x = np.concatenate([
        g.standard_normal(4000) * 60, g.standard_normal(2000) * 0.01, g.uniform(-460, 460, 2000),
        mids, -mids, finite, -finite, [0.0, 1e-30, 2.0 ** -10, 3 * 2.0 ** -11, 447.9, 463.9]])
    x = x.astype(np.float32).astype(np.float64)               # torch converts from float32
    got, ref = rnd(x), _torch_round(x)
    if not np.array_equal(got, ref):
        return False
    over = rnd(np.array([464.0, 500.0, -464.0, np.nan]))      # no saturation
    return bool(np.isnan(over).all())


def check_attention(att) -> bool:
    """FP8 attention against torch SDPA (float64) on inputs dequantized by
    torch's own float8 conversion, with non-unit descales, causal and key
    padding."""
    g = torch.Generator().manual_seed(11)
    B, H, N, d = 2, 2, 37, 16
    ds = (2.0 ** -6, 0.03, 2.0 ** -5)
    q8 = (torch.randn(B, H, N, d, generator=g) * 64).to(torch.float8_e4m3fn)
    k8 = (torch.randn(B, H, N, d, generator=g) * 30).to(torch.float8_e4m3fn)
    v8 = (torch.randn(B, H, N, d, generator=g) * 32).to(torch.float8_e4m3fn)
    scale = 0.25
    mask = torch.ones(B, N, dtype=torch.uint8)
    mask[1, 20:] = 0
    for causal in (False, True):
        for m in (None, mask):
            O, L, fm = att(q8, k8, v8, scale, *ds, causal=causal, mask=m)
            qd, kd, vd = (t.to(torch.float64) * s for t, s in zip((q8, k8, v8), ds))
            allow = torch.ones(N, N, dtype=torch.bool)
            if causal:
                allow = torch.tril(allow)
            allow = allow[None, None].expand(B, H, N, N).clone()
            if m is not None:
                allow &= m.bool()[:, None, None, :]
            ref = torch.nn.functional.scaled_dot_product_attention(qd, kd, vd, attn_mask=allow, scale=scale)
            s = torch.where(allow, scale * qd @ kd.transpose(-1, -2), torch.tensor(-math.inf, dtype=torch.float64))
            lse = torch.logsumexp(s, dim=-1)
            if fm.any() or not np.allclose(O, ref.numpy(), rtol=0, atol=1e-12):
                return False
            if not np.allclose(L, lse.numpy(), rtol=0, atol=1e-12):
                return False
    return True


def check_offset_model(model) -> bool:
    """The Max_offset recurrence against closed forms.

    Scores s = -j ln 2 for j in J = {0..9, 11..17, 19, 20}, in decreasing
    order (so the maximum, 0, comes first and nothing is rescaled), give
    exp(s - m) = 2^-j. With offset 8, P' = 2^(8-j) is an E4M3 value for
    j <= 17 (smallest subnormal 2^-9) and rounds to 0 for j = 19, 20 (below
    the 2^-10 midpoint). With offset 0, P = 2^-j survives only for j <= 9.
    The row sum is taken before rounding, so the LSE is ln sum 2^-j either way.
    """
    J = np.array(list(range(0, 10)) + list(range(11, 18)) + [19, 20])
    s = -J * math.log(2.0)
    v = np.stack([np.ones(J.size), J.astype(np.float64)], axis=1)
    w = 2.0 ** -J.astype(np.float64)
    lse_exact = math.log(w.sum())
    for off, keep in ((8, 17), (0, 9)):
        kept = np.where(J <= keep, w, 0.0)
        expect = np.array([kept.sum(), (kept * J).sum()]) / w.sum()
        for block in (1, 3, J.size):
            out, lse = model(s, v, block, off)
            if abs(lse - lse_exact) > 1e-12 or not np.allclose(out, expect, rtol=1e-12, atol=0):
                return False
    return True


# ---------------------------------------------------------------- pins

def test_decode_matches_the_format_and_torch():
    assert check_decode(F.e4m3_decode)


def test_round_matches_torch_including_ties_and_overflow():
    assert check_round(F.e4m3_round)


def test_encode_round_trips_every_code():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    vals = F.e4m3_decode(codes)
    assert np.array_equal(F.e4m3_round(vals), vals)
    enc = F.e4m3_encode(vals)
    # -0.0 and +0.0 keep their sign bit
    assert np.array_equal(enc, codes)


def test_fp8_attention_against_torch_sdpa():
    assert check_attention(F.attention_fp8)


def test_fp8_attention_on_selected_rows():
    x = W.generate(W.FP8_WORKLOADS[0].with_shape(B=1, H=2, N=96))
    O, L, fm = F.attention_fp8(x["q"], x["k"], x["v"], x["scale"], *x["descale"], causal=True)
    rows = np.array([0, 5, 95, 96, 150, 191])
    Os, Ls, fms = F.attention_fp8(x["q"], x["k"], x["v"], x["scale"], *x["descale"], causal=True, rows=rows)
    assert np.array_equal(Os, O.reshape(-1, O.shape[-1])[rows])
    assert np.array_equal(Ls, L.reshape(-1)[rows])
    # causal row 0 sees only key 0: O = dv * v_0 exactly, LSE = the one score
    v0 = F.e4m3_decode(x["v"][0, 0, 0]) * x["descale"][2]
    assert np.array_equal(O[0, 0, 0], v0)


def test_max_offset_recurrence_closed_form():
    assert check_offset_model(F.online_attention_e4m3)


def test_max_offset_reduces_the_rounding_error():
    """Section 6.1 of "Online Softmax 算法详解": with P in [0, 1] E4M3 spends
    most of its codes outside the range P uses, and small probabilities fall
    into the subnormals or to zero; scaling by 2^8 (section 6.2) moves them
    into the normal range. Rows of 4096 scores ~ N(0, 2^2) with V = 1 (the
    first column; the special case whose exact output is 1) and V ~ U(0, 1):
    with offset 0 the many small terms are lost and the output is biased low;
    with offset 8 the error stays within the rounding bound below and is
    several times smaller on average."""
    g = np.random.default_rng(3)
    e8, e0 = [], []
    for _ in range(10):
        n = 4096
        s = g.standard_normal(n) * 2.0
        v = np.concatenate([np.ones((n, 1)), g.uniform(0, 1, (n, 3))], axis=1)
        p, _, l, lse = sr.safe_softmax(s)
        exact = p @ v
        # per term |round(P') - P'| <= 2^-4 P' (normal range) + 2^-10 (the
        # subnormal half-spacing); divided by l' = 2^8 l
        bound = 2.0 ** -4 * (p @ np.abs(v)) + 2.0 ** -10 * np.abs(v).sum(axis=0) / (2.0 ** 8 * l)
        o8, l8 = F.online_attention_e4m3(s, v, 64, 8)
        o0, l0 = F.online_attention_e4m3(s, v, 64, 0)
        assert abs(l8 - lse) <= 1e-12 and abs(l0 - lse) <= 1e-12
        assert np.all(np.abs(o8 - exact) <= bound)
        assert o0[0] < 1.0 - 1e-3          # offset 0 loses mass: biased low
        e8.append(np.abs(o8 - exact).max())
        e0.append(np.abs(o0 - exact).max())
    assert np.mean(e8) * 4 < np.mean(e0)


# ---------------------------------------------------------------- planted mistakes

def _decode_bias8(b):
    return F.e4m3_decode(b) / 2.0


def _decode_subnormal_wrong(b):
    b = np.asarray(b)
    v = F.e4m3_decode(b)
    sub = ((b >> 3) & 0xF) == 0
    return np.where(sub, v / 2.0, v)


def _decode_no_nan(b):
    b = np.asarray(b).astype(np.int64)
    v = F.e4m3_decode(b)
    return np.where((b & 0x7F) == 0x7F, np.where(b & 0x80, -480.0, 480.0), v)


def _round_ties_away(x):
    """Ties go to the larger magnitude instead of the even code."""
    x = np.asarray(x, dtype=np.float64)
    vals = F._all_values()
    a = np.abs(x)
    hi = np.clip(np.searchsorted(vals, a), 1, vals.size - 1)
    tie = (a > vals[0]) & (a == (vals[hi - 1] + vals[hi]) / 2)
    return np.where(tie, np.copysign(vals[hi], x), F.e4m3_round(x))


def _round_saturating(x):
    x = np.asarray(x, dtype=np.float64)
    r = F.e4m3_round(x)
    return np.where(np.abs(x) >= F.E4M3_OVERFLOW, np.copysign(448.0, x), r)


def _att_no_descale_v(q, k, v, scale, dq=1.0, dk=1.0, dv=1.0, **kw):
    return F.attention_fp8(q, k, v, scale, dq, dk, 1.0, **kw)


def _att_descale_k_squared(q, k, v, scale, dq=1.0, dk=1.0, dv=1.0, **kw):
    return F.attention_fp8(q, k, v, scale, dq, dk * dk, dv, **kw)


def _model_sum_of_rounded(s, v, block, off):
    """l summed from the rounded P' instead of the float P'."""
    s = np.asarray(s, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    m, l, O = -math.inf, 0.0, np.zeros(v.shape[1])
    for j0 in range(0, s.size, block):
        sb, vb = s[j0:j0 + block], v[j0:j0 + block]
        m_new = max(m, float(np.max(sb)))
        alpha = 0.0 if m == -math.inf else math.exp(m - m_new)
        l, O = l * alpha, O * alpha
        p = F.e4m3_round(np.exp(sb - m_new) * 2.0 ** off)
        l += float(p.sum())
        O += p @ vb
        m = m_new
    return O / l, m + math.log(l / 2.0 ** off)


def _model_no_compensation(s, v, block, off):
    out, lse = F.online_attention_e4m3(s, v, block, off)
    return out, lse + off * math.log(2.0)


@pytest.mark.parametrize("check,mutant", [
    (check_decode, _decode_bias8),
    (check_decode, _decode_subnormal_wrong),
    (check_decode, _decode_no_nan),
    (check_round, _round_ties_away),
    (check_round, _round_saturating),
    (check_attention, _att_no_descale_v),
    (check_attention, _att_descale_k_squared),
    (check_offset_model, _model_sum_of_rounded),
    (check_offset_model, _model_no_compensation),
])
def test_planted_mistakes_are_caught(check, mutant):
    assert not check(mutant)
