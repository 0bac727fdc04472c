"""Parity of the HIP row softmax (fa_softmax_fwd) with the float64 oracle
(needs a GPU).

Every row of the small cases is compared element by element; the lengths
cover each register-resident and register + LDS shape on both sides of its
capacity, both streamed forms (a length that is not a whole number of
16-byte vectors, and rows longer than registers and LDS hold), masked entries, rows with a single live
entry and rows with none. The two full-size workloads are compared on sampled
rows. y and LSE are pre-filled with NaN so that an unwritten element fails.

Tolerances, from the arithmetic: the kernel works in float32 and rounds y
once to the output dtype, so |dy| <= rel * y + abs with rel = 4e-3 for bf16
output (half an ulp is at most 2^-8 of the value), 1e-3 for fp16 (2^-11, plus the
float32 terms), 2e-5 for fp32 (exp2 of an argument carrying up to ~100 * 2^-24
absolute error, and the sum's rounding); abs covers fp16 subnormals. LSE is
a float32 output, ln of a normaliser summed over up to 2^17 terms plus the
maximum: |dLSE| <= 1e-4 + 2^-22 |LSE| (the second term is two ulps of the
float32 result itself, which dominates for inputs near 3e4).
Rows with no finite entry must match exactly: y = 0 and LSE = -inf.
"""
import numpy as np
import pytest
import torch

import oracle
from online_softmax_03_amd import softmax as S
from online_softmax_03_amd import workloads as W
from tests.gpu_util import log

pytestmark = pytest.mark.gpu

Y_TOL = {"bf16": (4e-3, 1e-30), "f16": (1e-3, 1e-7), "f32": (2e-5, 1e-30)}
LSE_TOL = 1e-4
LSE_REL = 2.0 ** -22
PAIRS = [("bf16", "bf16"), ("bf16", "f32"), ("f16", "f16"), ("f16", "f32"), ("f32", "f32")]
BASE = W.SOFTMAX_WORKLOADS[0]


def run_gpu(x: torch.Tensor, out_dtype: str, inplace=False):
    dev = torch.device("cuda:0")
    xd = x.to(dev)
    lse = torch.full(x.shape[:-1], float("nan"), dtype=torch.float32, device=dev)
    if inplace:
        y, _ = S.softmax_rows(xd, out=xd, lse=lse)
    else:
        y = torch.full(x.shape, float("nan"), dtype=W.DTYPES[out_dtype], device=dev)
        S.softmax_rows(xd, out_dtype=W.DTYPES[out_dtype], out=y, lse=lse)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def compare(y, lse, x, out_dtype, what):
    yref, lref, dead = oracle.softmax_rows(x.double().numpy())
    assert not np.isnan(y).any(), f"{what}: NaN in y"
    assert not np.isnan(lse).any(), f"{what}: NaN in LSE"
    assert np.array_equal(np.isneginf(lse), dead), f"{what}: dead rows differ"
    assert np.all(y[dead] == 0.0), f"{what}: y not exactly 0 on rows with no finite entry"
    rel, ab = Y_TOL[out_dtype]
    err = np.abs(y - yref)
    bound = rel * np.abs(yref) + ab
    worst = float((err / bound).max()) if err.size else 0.0
    assert worst <= 1.0, f"{what}: |dy| exceeds {rel}*y+{ab} by {worst:.2f}x (max |dy| {err.max():.3e})"
    live = ~dead
    el = float(np.abs(lse[live] - lref[live]).max()) if live.any() else 0.0
    lbound = LSE_TOL + LSE_REL * np.abs(lref[live])
    assert np.all(np.abs(lse[live] - lref[live]) <= lbound), f"{what}: max |dLSE| = {el:.3e}"
    return float(err.max()) if err.size else 0.0, el


# register-resident capacities (16-bit elements): 512 ... 65536; register +
# LDS shapes: 131072 and 165888 (16-bit), 98304 and 132096 (fp32); each
# also one vector over, which moves to the next shape or the streamed form
COLS = [1, 3, 4, 8, 24, 64, 100, 512, 520, 1024, 1032, 2048, 2056, 4096, 4104, 8192, 8200, 16384, 16392,
        32768, 32776, 65536, 65544, 70001, 98304, 98308, 100000, 131072, 131076, 131080, 132096, 132100,
        163840, 165888, 165896]


@pytest.mark.parametrize("cols", COLS)
@pytest.mark.parametrize("pair", PAIRS, ids=["->".join(p) for p in PAIRS])
def test_rows_every_element(pair, cols):
    rows = 7 if cols <= 8200 else 3
    w = BASE.with_shape(rows=rows, cols=cols, in_dtype=pair[0], out_dtype=pair[1], masked_frac=0.1,
                        seed=3000 + cols)
    x = W.generate_softmax(w)
    x[0] = float("-inf")                 # no finite entry
    if rows > 2:
        x[2] = float("-inf")
        x[2, cols // 2] = 1.5            # a single live entry
    log(f"case softmax {pair[0]}->{pair[1]} rows={rows} cols={cols}")
    y, lse = run_gpu(x, pair[1])
    e = compare(y, lse, x, pair[1], f"{pair} cols={cols}")
    log(f"  max|dy|={e[0]:.2e} max|dLSE|={e[1]:.2e}")


@pytest.mark.parametrize("in_dtype", ["bf16", "f32"])
def test_large_magnitudes_and_ragged_row_count(in_dtype):
    """Values around +-3e4 (the max must be subtracted first) and a row count
    that does not fill the last workgroup."""
    w = BASE.with_shape(rows=13, cols=96, in_dtype=in_dtype, out_dtype=in_dtype, dist=("uniform", -40.0, 40.0),
                        seed=3100)
    x = W.generate_softmax(w).float()
    x[:6] += 3.0e4
    x[6:] -= 3.0e4
    x = x.to(W.DTYPES[in_dtype])
    y, lse = run_gpu(x, in_dtype)
    compare(y, lse, x, in_dtype, f"magnitudes {in_dtype}")


@pytest.mark.parametrize("pair", [("bf16", "bf16"), ("f32", "f32"), ("f16", "f16")])
@pytest.mark.parametrize("cols", [512, 70001, 131072])
def test_in_place(pair, cols):
    w = BASE.with_shape(rows=5, cols=cols, in_dtype=pair[0], out_dtype=pair[1], seed=3200)
    x = W.generate_softmax(w)
    y, lse = run_gpu(x, pair[1], inplace=True)
    compare(y, lse, x, pair[1], f"in place {pair} cols={cols}")


# The register + LDS forms run one workgroup per compute unit (256) that walks
# rows r, r + 256, ...: 517 rows give each workgroup two or three rows, and
# the rows with no finite entry or a single one sit in the second and third
# passes of their workgroups.
ROW_WALK = [(("bf16", "bf16"), 131072, False), (("f16", "f32"), 165888, False), (("f32", "f32"), 98304, False),
            (("f32", "f32"), 132096, True), (("bf16", "bf16"), 163840, True)]


@pytest.mark.parametrize("pair,cols,inplace", ROW_WALK,
                         ids=[f"{p[0]}->{p[1]}-{c}{'-inplace' if ip else ''}" for p, c, ip in ROW_WALK])
def test_register_lds_row_walk(pair, cols, inplace):
    rows = 517
    w = BASE.with_shape(rows=rows, cols=cols, in_dtype=pair[0], out_dtype=pair[1], masked_frac=0.1,
                        seed=3400 + cols)
    x = W.generate_softmax(w)
    x[300] = float("-inf")               # second pass of workgroup 44
    x[513] = float("-inf")               # third pass of workgroup 1
    x[513, 17] = -2.0
    x[516] = float("-inf")               # third pass of the last workgroup with three rows
    log(f"case softmax row walk {pair[0]}->{pair[1]} rows={rows} cols={cols} inplace={inplace}")
    y, lse = run_gpu(x, pair[1], inplace=inplace)
    e = compare(y, lse, x, pair[1], f"row walk {pair} cols={cols} inplace={inplace}")
    log(f"  max|dy|={e[0]:.2e} max|dLSE|={e[1]:.2e}")


def test_without_lse():
    w = BASE.with_shape(rows=4, cols=256, seed=3300)
    x = W.generate_softmax(w)
    y, lse = S.softmax_rows(x.cuda(), want_lse=False)
    torch.cuda.synchronize()
    assert lse is None
    yref, _, _ = oracle.softmax_rows(x.double().numpy())
    assert np.abs(y.float().cpu().numpy() - yref).max() <= 4e-3


@pytest.mark.parametrize("name", [w.name for w in W.SOFTMAX_WORKLOADS])
def test_full_size_sampled_rows(name):
    """The benchmark workloads at full size: sampled rows against the oracle,
    and every row summing to 1 within the output rounding."""
    w = W.SOFTMAX_BY_NAME[name]
    log(f"case {name}: rows={w.rows} cols={w.cols}")
    x = W.generate_softmax(w)
    y, lse = run_gpu(x, w.out_dtype)
    g = np.random.default_rng(11)
    rows = np.union1d(g.choice(w.rows, size=48, replace=False), [0, w.rows - 1])
    compare(y[rows], lse[rows], x[torch.as_tensor(rows)], w.out_dtype, name)
    sums = y.sum(axis=1)
    rel = Y_TOL[w.out_dtype][0]
    assert np.abs(sums - 1.0).max() <= rel, f"{name}: row sums off by {np.abs(sums - 1).max():.2e}"


def _draw_softmax(i):
    r = np.random.default_rng(15000 + i)
    pair = PAIRS[int(r.integers(len(PAIRS)))]
    cols = int(np.exp(r.uniform(0.0, np.log(170000.0))))
    rows = int(r.integers(1, 12)) if cols <= 20000 else int(r.integers(1, 4))
    lo = float(r.uniform(-60.0, 0.0))
    return dict(pair=pair, rows=rows, cols=max(1, cols), masked_frac=float(r.choice([0.0, 0.1, 0.9])),
                dist=("uniform", lo, lo + float(r.uniform(0.1, 60.0))), seed=16000 + i)


SOFTMAX_RANDOM = [_draw_softmax(i) for i in range(200)]


@pytest.mark.parametrize("i", range(len(SOFTMAX_RANDOM)))
def test_random_rows(i):
    """Seeded random shapes (column counts log-uniform up to 170000, so every
    kernel form and its boundaries get drawn), dtype pairs, value ranges and
    masked fractions, every element against the oracle."""
    c = SOFTMAX_RANDOM[i]
    w = BASE.with_shape(rows=c["rows"], cols=c["cols"], in_dtype=c["pair"][0], out_dtype=c["pair"][1],
                        masked_frac=c["masked_frac"], dist=c["dist"], seed=c["seed"])
    x = W.generate_softmax(w)
    log(f"case softmax random {i}: {c}")
    y, lse = run_gpu(x, c["pair"][1])
    compare(y, lse, x, c["pair"][1], f"softmax random {i}: {c}")
