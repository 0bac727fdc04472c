"""Seeded random draws of the attention forward against the float64 oracle,
every row (needs a GPU).

Each draw picks a head dim (64, 128), an input dtype (bf16, fp16) and an
output dtype (the input's or fp32), causal or not, 1-3 batches of 1-4 heads,
a sequence length log-uniform in 1 ... 640 (so single keys, ragged tails and
several tiles all come up), logit and value spreads, and a key mask: none, a
padding mask with random lengths (0 and N included), or a random
non-contiguous mask. A quarter of the draws force a random compiled tile
shape, another quarter go through the split-KV entry point with a random part
count (0 = the library's). The bar is the parity bar of the other tests: O
within 2e-2 (bf16) / 5e-3 (fp16), LSE within 1e-3, the fully masked rows
exactly (O = 0, LSE = -inf), no NaN; O and LSE are pre-filled with NaN.
"""
import numpy as np
import pytest
import torch

from online_softmax_03_amd import workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

BASE = W.BY_NAME["bf16_causal_n8192_d128"]


def _tiles(d, in_dtype, out_dtype):
    from online_softmax_03_amd import capi
    code = {"bf16": capi.FA_DTYPE_BF16, "f16": capi.FA_DTYPE_F16, "f32": capi.FA_DTYPE_F32}
    return [(br, bc) for br in (64, 128, 256, 512) for bc in (32, 64, 128)
            if capi.fa_tile_supported(d, code[in_dtype], code[out_dtype], (br, bc)) == 0]


def _draw(i):
    r = np.random.default_rng(40000 + i)
    d = int(r.choice([64, 128]))
    in_dtype = ["bf16", "f16"][int(r.integers(2))]
    out_dtype = [in_dtype, "f32"][int(r.integers(2))]
    causal = bool(r.integers(2))
    B, H = int(r.integers(1, 4)), int(r.integers(1, 5))
    N = max(1, int(np.exp(r.uniform(0.0, np.log(640.0)))))
    qk = float(r.choice([0.5, 1.0, 2.0, 3.0]))
    v = 1.0 if in_dtype == "bf16" else 0.577
    mask = ["none", "padding", "general"][int(r.integers(3))]
    route = ["default", "default", "tile", "split"][int(r.integers(4))]
    return dict(d=d, in_dtype=in_dtype, out_dtype=out_dtype, causal=causal, B=B, H=H, N=N, qk=qk, v=v, mask=mask,
                route=route, pick=int(r.integers(1 << 30)), seed=41000 + i)


DRAWS = [_draw(i) for i in range(400)]


@pytest.mark.parametrize("i", range(len(DRAWS)))
def test_random_forward_every_row(i):
    c = DRAWS[i]
    w = BASE.with_shape(B=c["B"], H=c["H"], N=c["N"], d=c["d"], in_dtype=c["in_dtype"], out_dtype=c["out_dtype"],
                        causal=c["causal"], q_dist=("normal", c["qk"]), k_dist=("normal", c["qk"]),
                        v_dist=("normal", c["v"]), key_padding=False, seed=c["seed"])
    g = torch.Generator().manual_seed(c["seed"] + 1)
    lens = None
    if c["mask"] == "padding":
        lens = torch.randint(0, c["N"] + 1, (c["B"],), generator=g, dtype=torch.int64)
    x = W.generate(w, lens=lens)
    if c["mask"] == "general":
        keep = float(torch.rand((), generator=g)) * 0.8 + 0.1
        x["mask"] = (torch.rand((c["B"], c["N"]), generator=g) < keep).to(torch.uint8)
    tile, splits = None, None
    if c["route"] == "tile":
        options = _tiles(c["d"], c["in_dtype"], c["out_dtype"])
        tile = options[c["pick"] % len(options)]
    elif c["route"] == "split":
        splits = c["pick"] % 9  # 0: the library's count
    U.log(f"case forward random {i}: {c} tile={tile} splits={splits}")
    U.check_full(x, tile=tile, num_splits=splits, what=f"forward random {i}")
