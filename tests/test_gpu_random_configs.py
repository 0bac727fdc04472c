"""Seeded random configurations of every entry point, compared with the
oracle on every row / element (needs a GPU).

The hand-picked cases elsewhere cover each feature on its own; these draw
combinations (head dim, dtypes, causal, padding or general key masks, every
compiled tile, split counts, gradient dtype, FP8 offset) at small ragged
sizes from a fixed seed, so a combination nobody listed still meets the same
parity bar. The draws are deterministic; a failing case prints its index and
parameters.
"""
import numpy as np
import pytest
import torch

from online_softmax_03_amd import attention as A
from online_softmax_03_amd import capi
from online_softmax_03_amd import workloads as W
from tests import gpu_util as U
from tests import test_gpu_bwd as TB
from tests import test_gpu_fp8 as T8

pytestmark = pytest.mark.gpu

BASE = {w.name: w for w in W.WORKLOADS}["bf16_causal_n8192_d128"]


def _tiles(d):
    out = [None]
    for br in (64, 128, 256, 512):
        for bc in (32, 64, 128):
            if capi.fa_tile_supported(d, capi.FA_DTYPE_BF16, capi.FA_DTYPE_BF16, (br, bc)) == 0:
                out.append((br, bc))
    return out


def _mask(g, kind, B, N):
    if kind == "none":
        return None, None
    if kind == "pad":
        lens = torch.from_numpy(g.integers(0, N + 1, B)).to(torch.int64)
        return W.mask_from_lengths(lens, N), lens
    m = (torch.from_numpy(g.random((B, N))) > g.uniform(0.2, 0.9)).to(torch.uint8)
    return m, None


def _draw(i, g):
    d = int(g.choice([64, 128]))
    dt = str(g.choice(["bf16", "f16"]))
    return dict(d=d, in_dtype=dt, out_dtype=str(g.choice([dt, "f32"])), causal=bool(g.integers(2)),
                B=int(g.integers(1, 4)), H=int(g.integers(1, 4)), N=int(g.integers(1, 520)),
                mask=str(g.choice(["none", "pad", "general"])), seed=5000 + i)


FWD = [_draw(i, np.random.default_rng(9000 + i)) for i in range(64)]


def _forward(c, g, label):
    w = BASE.with_shape(B=c["B"], H=c["H"], N=c["N"], d=c["d"], in_dtype=c["in_dtype"], out_dtype=c["out_dtype"],
                        causal=c["causal"], seed=c["seed"])
    x = W.generate(w)
    x["mask"], x["lens"] = _mask(g, c["mask"], c["B"], c["N"])
    tiles = _tiles(c["d"])
    tile = tiles[int(g.integers(len(tiles)))]
    splits = [None, None, 2, 3, 5][int(g.integers(5))]
    if splits is not None:
        tile = None
    what = f"{label}: {c} tile={tile} splits={splits}"
    U.log(what)
    U.check_full(x, tile=tile, what=what, num_splits=splits)


@pytest.mark.parametrize("i", range(len(FWD)))
def test_random_forward(i):
    _forward(FWD[i], np.random.default_rng(9100 + i), f"random forward {i}")


BWD = [_draw(100 + i, np.random.default_rng(9200 + i)) for i in range(20)]


def _backward(c, g, label):
    w = BASE.with_shape(B=c["B"], H=c["H"], N=c["N"], d=c["d"], in_dtype=c["in_dtype"], out_dtype=c["in_dtype"],
                        causal=c["causal"], seed=c["seed"])
    x = W.generate(w)
    x["mask"], _ = _mask(g, c["mask"], c["B"], c["N"])
    do = W.generate_dout(w)
    ref, o, lse = TB._oracle_inputs(x, do)
    grad = [None, "f32"][int(g.integers(2))]
    U.log(f"{label}: {c} grad={grad}")
    got = TB.run_bwd(x, do, o, lse, grad_dtype=grad)
    TB.check(got, ref, c["in_dtype"], label)


@pytest.mark.parametrize("i", range(len(BWD)))
def test_random_backward(i):
    _backward(BWD[i], np.random.default_rng(9300 + i), f"random backward {i}")


def _draw_fp8(i, r):
    return dict(B=int(r.integers(1, 3)), H=int(r.integers(1, 4)), N=int(r.integers(1, 400)), causal=bool(r.integers(2)),
                mask=str(r.choice(["none", "pad", "general"])), out=str(r.choice(["bf16", "f16", "f32"])),
                offset=int(r.choice([8, 0])), seed=7000 + i)


FP8 = [_draw_fp8(j, np.random.default_rng(9400 + j)) for j in range(16)]


def _fp8(c, g, label):
    w = W.FP8_BY_NAME["fp8_causal_n8192_d128"].with_shape(B=c["B"], H=c["H"], N=c["N"], causal=c["causal"],
                                                        out_dtype=c["out"], seed=c["seed"])
    x = W.generate(w)
    x["mask"], _ = _mask(g, c["mask"], c["B"], c["N"])
    U.log(f"{label}: {c}")
    T8.check_all_rows(x, c["offset"], label)


@pytest.mark.parametrize("i", range(len(FP8)))
def test_random_fp8(i):
    _fp8(FP8[i], np.random.default_rng(9500 + i), f"random fp8 {i}")


# A wider sweep from other seeds, in chunks so that each test reports on its
# own: 16 chunks of 100 forward, 15 backward and 15 FP8 configurations.
SWEEP_CHUNKS, SWEEP_FWD, SWEEP_BWD, SWEEP_FP8 = 16, 100, 15, 15


@pytest.mark.parametrize("k", range(SWEEP_CHUNKS))
def test_random_sweep_chunk(k):
    for j in range(SWEEP_FWD):
        i = k * SWEEP_FWD + j
        _forward(_draw(i, np.random.default_rng(31000 + i)), np.random.default_rng(41000 + i), f"sweep forward {i}")
    for j in range(SWEEP_BWD):
        i = k * SWEEP_BWD + j
        _backward(_draw(100000 + i, np.random.default_rng(32000 + i)), np.random.default_rng(42000 + i),
                  f"sweep backward {i}")
    for j in range(SWEEP_FP8):
        i = k * SWEEP_FP8 + j
        _fp8(_draw_fp8(10000 + i, np.random.default_rng(33000 + i)), np.random.default_rng(43000 + i),
             f"sweep fp8 {i}")
