"""Parity of the FP8 (E4M3) attention forward with the float64 oracle (needs a
GPU).

The oracle is the plain attention of the dequantized inputs. The kernel
rounds the probabilities to E4M3 for the P V product, so the tolerance is
derived per row from that rounding: with P' = 2^Max_offset * exp(s - m_ref)
(m_ref at most the row maximum) rounded to nearest, each term is off by at
most 2^-4 P' (3 mantissa bits) plus 2^-10 (half the subnormal spacing); the
row sum l' >= 2^Max_offset * l, l = sum_j exp(s_j - max_j s_j), is taken from
the unrounded values. Hence per row and output column

    |dO| <= dv * ((2^-4 + 2^-10) sum_j p_j |v_j| + 2^-10 sum_j |v_j| / (2^off l))
            + (half an ulp of the output dtype) |O|,

the extra 2^-10 sum p|v| covering float32 accumulation over up to 2^13 keys.
LSE is formed from the unrounded sum: |dLSE| <= 1e-3. Fully masked rows are
O = 0 and LSE = -inf exactly. O and LSE are pre-filled with NaN.
"""

import numpy as np
import pytest
import torch

from oracle import fp8 as F
from online_softmax_03_amd import attention as A
from online_softmax_03_amd import workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

BASE = W.FP8_WORKLOADS[0]
# half an ulp, relative: bf16 keeps 8 significant bits, fp16 11, fp32 24
OUT_ULP = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11, "f32": 2.0 ** -24}
LSE_TOL = 1e-3


def run_fp8(x, max_offset=8):
    dev = torch.device("cuda:0")
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    mask = None if x["mask"] is None else x["mask"].to(dev)
    out_dt = W.DTYPES[x["out_dtype"]]
    o = torch.full(q.shape, float("nan"), dtype=out_dt, device=dev)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=dev)
    A.attention_fwd_fp8(q, k, v, scale=x["scale"], descale_q=x["descale"][0], descale_k=x["descale"][1],
                        descale_v=x["descale"][2], causal=x["causal"], key_padding_mask=mask,
                        out_dtype=out_dt, max_offset=max_offset, out=o, lse=lse)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def _abs_codes(t):
    """E4M3 codes of |v|: the sign bit cleared."""
    return (t.contiguous().view(torch.uint8) & 0x7F).contiguous()


def reference_rows(x, b, h, rows):
    """Oracle O, LSE, fully-masked flags, and the per-row error bound terms
    (sum_j p_j |v_j| * dv, sum_j |v_j| * dv / l) for query rows `rows` of
    head (b, h)."""
    sl = lambda t: t[b:b + 1, h:h + 1]  # noqa: E731
    mask = None if x["mask"] is None else x["mask"][b:b + 1]
    ds = x["descale"]
    Oref, Lref, fm = F.attention_fp8(sl(x["q"]), sl(x["k"]), sl(x["v"]), x["scale"], *ds, causal=x["causal"],
                                     mask=mask, rows=rows)
    Pabs, _, _ = F.attention_fp8(sl(x["q"]), sl(x["k"]), _abs_codes(sl(x["v"])), x["scale"], *ds,
                                 causal=x["causal"], mask=mask, rows=rows)
    # l = sum_j exp(s_j - max s) needs the row maximum of the scaled scores
    q = F.e4m3_decode(sl(x["q"]))[0, 0]
    k = F.e4m3_decode(sl(x["k"]))[0, 0]
    vabs = np.abs(F.e4m3_decode(sl(x["v"]))[0, 0]) * ds[2]
    N = q.shape[0]
    keyok = np.ones(N, dtype=bool) if mask is None else (mask[0].numpy() != 0)
    sumv_over_l = np.zeros((len(rows), q.shape[1]))
    for n, i in enumerate(rows):
        allow = keyok.copy()
        if x["causal"]:
            allow[i + 1:] = False
        if not allow.any():
            continue
        s = (x["scale"] * ds[0] * ds[1]) * (k[allow] @ q[i])
        l = float(np.exp(s - s.max()).sum())
        sumv_over_l[n] = vabs[allow].sum(axis=0) / l
    return Oref, Lref, fm, Pabs, sumv_over_l


def compare_fp8(O, L, ref, out_dtype, max_offset, what):
    Oref, Lref, fm, Pabs, sumv_over_l = ref
    assert not np.isnan(O).any(), f"{what}: NaN in O"
    assert not np.isnan(L).any(), f"{what}: NaN in LSE"
    dead = np.isneginf(L)
    assert np.array_equal(dead, fm), f"{what}: fully masked rows differ ({dead.sum()} vs {fm.sum()})"
    assert np.all(O[fm] == 0.0), f"{what}: O not exactly 0 on fully masked rows"
    tol = ((2.0 ** -4 + 2.0 ** -10) * Pabs + 2.0 ** -10 * sumv_over_l / 2.0 ** max_offset
           + OUT_ULP[out_dtype] * np.abs(Oref) + 1e-6)
    err = np.abs(O - Oref)
    worst = float((err / tol).max()) if err.size else 0.0
    assert worst <= 1.0, f"{what}: error {err.max():.3e} exceeds the rounding bound (ratio {worst:.2f})"
    live = ~fm
    errL = float(np.abs(L[live] - Lref[live]).max()) if live.any() else 0.0
    assert errL <= LSE_TOL, f"{what}: max |dLSE| = {errL:.3e} > {LSE_TOL}"
    return float(err.max()) if err.size else 0.0, errL, worst


def check_all_rows(x, max_offset=8, what=""):
    O, L = run_fp8(x, max_offset)
    B, H, N, d = x["q"].shape
    errs = []
    for b in range(B):
        for h in range(H):
            ref = reference_rows(x, b, h, np.arange(N))
            errs.append(compare_fp8(O[b, h], L[b, h], ref, x["out_dtype"], max_offset, f"{what} b={b} h={h}"))
    e = tuple(max(t[i] for t in errs) for i in range(3))
    U.log(f"  {what}: max|dO|={e[0]:.2e} max|dLSE|={e[1]:.2e} worst err/bound={e[2]:.2f}")
    return e


SMALL = [
    # (id, shape overrides, key lengths or None)
    ("causal_n333", dict(B=1, H=3, N=333), None),
    ("causal_n64", dict(B=2, H=1, N=64), None),
    ("noncausal_n190", dict(B=1, H=2, N=190, causal=False), None),
    ("noncausal_n1", dict(B=1, H=1, N=1, causal=False), None),
    ("causal_n65_f16out", dict(B=1, H=2, N=65, out_dtype="f16"), None),
    ("noncausal_n130_f32out", dict(B=1, H=2, N=130, causal=False, out_dtype="f32"), None),
    ("keypad_n257", dict(B=6, H=1, N=257, causal=False), [0, 1, 63, 64, 65, 257]),
    ("keypad_causal_n200", dict(B=3, H=2, N=200), [0, 100, 200]),
    ("causal_h32_n300", dict(B=2, H=16, N=300), None),  # tiles dealt over groups of 4 heads
    ("unit_descale_n300", dict(B=1, H=2, N=300, q_dist=("normal", 1.0), k_dist=("normal", 1.0),
                               v_dist=("normal", 1.0), descale=(1.0, 1.0, 1.0)), None),
]


@pytest.mark.parametrize("max_offset", [8, 0])
@pytest.mark.parametrize("ident,over,lens", SMALL, ids=[s[0] for s in SMALL])
def test_small_shapes_every_row(ident, over, lens, max_offset):
    w = BASE.with_shape(**over)
    x = W.generate(w, lens=None if lens is None else torch.tensor(lens, dtype=torch.int64))
    U.log(f"case fp8 {ident} offset={max_offset}: B,H,N={w.B},{w.H},{w.N} -> {w.out_dtype} causal={w.causal}")
    check_all_rows(x, max_offset, f"fp8 {ident} off={max_offset}")


def test_general_key_mask():
    """A non-contiguous key mask (every third key dropped, plus a hole)."""
    w = BASE.with_shape(B=2, H=2, N=290, causal=False)
    x = W.generate(w)
    m = torch.ones(2, 290, dtype=torch.uint8)
    m[:, ::3] = 0
    m[1, 100:180] = 0
    x["mask"] = m
    U.log("case fp8 general mask")
    check_all_rows(x, 8, "fp8 general mask")


def test_offset_8_beats_offset_0_on_positive_values():
    """"Online Softmax 算法详解" section 6.1 on the GPU: long rows of spread-out
    scores (real Q ~ N(0, 2^2): stored N(0, 64^2), descale 2^-5) and
    V ~ U(0, 1) (stored U(0, 32), descale 2^-5). With P in [0, 1]
    the many small probabilities round to zero and the output is biased low;
    with the offset they keep their value."""
    w = BASE.with_shape(B=1, H=2, N=2048, causal=False, v_dist=("uniform", 0.0, 32.0),
                        descale=(2.0 ** -5, 2.0 ** -6, 2.0 ** -5))
    x = W.generate(w)
    e8 = check_all_rows(x, 8, "fp8 U(0,1) values off=8")
    e0 = check_all_rows(x, 0, "fp8 U(0,1) values off=0")
    assert e8[0] * 2 < e0[0]


def test_headline_fp8_workload_sampled_rows():
    """The FP8 headline workload (B=2, H=32, N=8192, d=128, causal) at full
    size; the oracle computes sampled rows one by one."""
    x = W.generate(BASE)
    U.log(f"case {BASE.name}: full size, sampled rows")
    O, L = run_fp8(x, 8)
    B, H, N, d = x["q"].shape
    rows = U.sample_rows(B, H, N, 96, seed=5, causal=True)
    worst = []
    for bh in sorted(set((rows // N).tolist())):
        b, h = divmod(bh, H)
        rr = rows[(rows // N) == bh] - bh * N
        ref = reference_rows(x, b, h, rr)
        worst.append(compare_fp8(O[b, h][rr], L[b, h][rr], ref, x["out_dtype"], 8, f"{BASE.name} head {bh}"))
    e = tuple(max(t[i] for t in worst) for i in range(3))
    U.log(f"  {BASE.name}: {len(rows)} rows, max|dO|={e[0]:.2e} max|dLSE|={e[1]:.2e} worst err/bound={e[2]:.2f}")


def _draw(i):
    r = np.random.default_rng(60000 + i)
    return dict(causal=bool(r.integers(2)), B=int(r.integers(1, 4)), H=int(r.integers(1, 4)),
                N=max(1, int(np.exp(r.uniform(0.0, np.log(400.0))))), out=["bf16", "f16", "f32"][int(r.integers(3))],
                qk=float(r.choice([16.0, 32.0, 64.0])), offset=[8, 0][int(r.integers(2))],
                mask=["none", "padding", "general"][int(r.integers(3))], seed=61000 + i)


RANDOM = [_draw(i) for i in range(60)]


@pytest.mark.parametrize("i", range(len(RANDOM)))
def test_random_shapes_every_row(i):
    """Seeded random draws: causal or not, 1-3 batches of 1-3 heads, length
    log-uniform in 1 ... 400, output dtype, stored logit spread (descale
    2^-6), Max_offset 8 or 0, and no key mask, a padding mask (random
    lengths) or a random non-contiguous one; every row against the oracle
    within the per-row rounding bound."""
    c = RANDOM[i]
    w = BASE.with_shape(B=c["B"], H=c["H"], N=c["N"], causal=c["causal"], out_dtype=c["out"],
                        q_dist=("normal", c["qk"]), k_dist=("normal", c["qk"]), seed=c["seed"])
    g = torch.Generator().manual_seed(c["seed"] + 1)
    lens = None
    if c["mask"] == "padding":
        lens = torch.randint(0, c["N"] + 1, (c["B"],), generator=g, dtype=torch.int64)
    x = W.generate(w, lens=lens)
    if c["mask"] == "general":
        x["mask"] = (torch.rand((c["B"], c["N"]), generator=g) < 0.6).to(torch.uint8)
    U.log(f"case fp8 random {i}: {c}")
    check_all_rows(x, c["offset"], f"fp8 random {i}")
