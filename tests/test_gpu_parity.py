"""Parity of the HIP attention forward with the float64 oracle (needs a GPU).

Small shapes are compared element by element on every row; they span several
tiles and end in ragged tails. At full size the bf16 d = 64 and fp16
key-padded workloads are compared on every row; the causal d = 128 ones on
one row of every 32-row block of every head, which the oracle computes one by
one, and on the exact fully masked set over every row. Every run pre-fills O and
LSE with NaN, so an element the kernel fails to write shows up as NaN.
"""
import math

import numpy as np
import pytest
import torch

from online_softmax_03_amd import attention as A
from online_softmax_03_amd import workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

C = {w.name: w for w in W.WORKLOADS}
TINY, C2, C3, C4, C5 = (w.name for w in W.WORKLOADS)

SMALL = [
    # (id, base workload, shape overrides, key lengths or None)
    ("bf16_f32out_d64_n300", C2, dict(B=2, H=3, N=300), None),
    ("bf16_d64_n200_bf16out", C2, dict(B=1, H=2, N=200, out_dtype="bf16"), None),
    ("bf16_causal_d128_n333", C3, dict(B=1, H=4, N=333), None),
    ("bf16_causal_d128_n64", C3, dict(B=2, H=1, N=64), None),
    ("bf16_noncausal_d128_n190", C3, dict(B=1, H=2, N=190, causal=False), None),
    ("bf16_causal_long_logits_n700", C4, dict(B=1, H=2, N=700), None),
    ("f16_keypad_d64_n257", C5, dict(B=6, H=2, N=257), [0, 1, 63, 64, 256, 257]),
    ("f16_keypad_causal_d128_f32out_n130", C5,
     dict(B=3, H=2, N=130, d=128, causal=True, out_dtype="f32"), [0, 5, 130]),
    ("f16_d64_n1", C5, dict(B=1, H=1, N=1, key_padding=False), None),
    ("bf16_causal_d64_n2", C2, dict(B=1, H=1, N=2, causal=True), None),
    ("bf16_d128_n31", C3, dict(B=1, H=1, N=31), None),
    ("f16_d64_n33_keypad", C5, dict(B=2, H=1, N=33), [32, 33]),
    # causal launches over 32 and 16 heads deal their query tiles over groups
    # of 4 and 2 heads
    ("bf16_causal_d128_h32_n300", C3, dict(B=2, H=16, N=300), None),
    ("f16_keypad_causal_d64_h16_n600", C5, dict(B=2, H=8, N=600, causal=True), [600, 417]),
]


@pytest.mark.parametrize("ident,base,over,lens", SMALL, ids=[s[0] for s in SMALL])
def test_small_shapes_every_row(ident, base, over, lens):
    w = C[base].with_shape(**over)
    x = W.generate(w, lens=None if lens is None else torch.tensor(lens, dtype=torch.int64))
    U.log(f"case {ident}: B,H,N,d={w.B},{w.H},{w.N},{w.d} {w.in_dtype}->{w.out_dtype} causal={w.causal}")
    U.check_full(x, what=ident)


def test_tiny_f32_workload_every_row():
    """The fp32 workload (B=1, H=1, N=256, d=64, B_c=64) on the fp32 MFMA path:
    O within 1e-4 and LSE within 1e-5 of the float64 oracle."""
    w = C[TINY]
    x = W.generate(w)
    U.log(f"case {TINY}: tile (128, {w.block_c})")
    O, L = U.run_gpu(x, tile=(128, w.block_c))
    import oracle
    Oref, Lref, fm = oracle.attention(x["q"], x["k"], x["v"], x["scale"], False)
    eo, el = U.compare(O, L, Oref, Lref, fm, "f32", TINY)
    U.log(f"  {TINY}: max|dO|={eo:.2e} max|dLSE|={el:.2e}")
    assert el <= 1e-5


@pytest.mark.parametrize("d,causal,lens", [(64, True, None), (128, False, None), (128, True, [0, 77])])
def test_f32_path_shapes(d, causal, lens):
    w = C[TINY].with_shape(B=2 if lens else 1, H=2, N=150, d=d, causal=causal)
    x = W.generate(w, lens=None if lens is None else torch.tensor(lens))
    U.check_full(x, what=f"f32 d={d} causal={causal} lens={lens}")


WORKED = [
    # scores, values: the pages' worked examples as row 0 of an attention
    ([2.0, 4.0, 1.0, 3.0], [1.0, 1.0, 1.0, 1.0]),
    ([1.0, 2.0, 5.0, 3.0], [1.0, -1.0, 2.0, 0.5]),
    ([1.0, 2.0, 3.0, 10.0], [1.0, 1.0, 1.0, 1.0]),
    ([0.0, 5.0], [2.0, 3.0]),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", range(len(WORKED)))
def test_worked_examples_as_attention(case, dtype):
    """q_0 = e_0, k_j = s_j e_0, scale 1: row 0's scores are the example's.
    All values are exact in bf16 and fp16. LSE and O follow in closed form."""
    s, vals = WORKED[case]
    n, d = len(s), 64
    dt = W.DTYPES[dtype]
    q = torch.zeros(1, 1, n, d)
    k = torch.zeros(1, 1, n, d)
    v = torch.zeros(1, 1, n, d)
    q[0, 0, 0, 0] = 1.0
    k[0, 0, :, 0] = torch.tensor(s)
    v[0, 0, :, 0] = torch.tensor(vals)
    x = dict(q=q.to(dt), k=k.to(dt), v=v.to(dt), mask=None, scale=1.0, causal=False,
             in_dtype=dtype, out_dtype="f32")
    O, L = U.run_gpu(x)
    m = max(s)
    l = sum(math.exp(t - m) for t in s)
    assert abs(L[0, 0, 0] - (m + math.log(l))) <= U.LSE_TOL
    ref = sum(math.exp(t - m) * y for t, y in zip(s, vals)) / l
    assert abs(O[0, 0, 0, 0] - ref) <= U.O_TOL[dtype]
    assert np.all(O[0, 0, 0, 1:] == 0)
    U.check_full(x, what=f"worked example {case} {dtype}")


@pytest.mark.parametrize("name", [C2, C5])
def test_full_size_every_row(name):
    """The bf16 d = 64 and the fp16 key-padded workloads at full size, every
    row against the oracle: O and LSE to tolerance, and the fully masked rows
    (C5's batch of key length 0) exactly, with O = 0 and LSE = -inf there."""
    w = C[name]
    U.log(f"case {name}: full size B,H,N,d={w.B},{w.H},{w.N},{w.d}, every row")
    x = W.generate(w)
    U.check_full(x, what=name)


@pytest.mark.parametrize("name", [C3, C4])
def test_full_size_rows_of_every_block(name):
    """The causal d = 128 workloads at full size. The oracle computes one row
    of every 32-row block of every head (a block is one wave's share of a
    query tile; the row within it is drawn at random) plus the first and last
    rows of a few heads. On every row: no NaN in O or LSE, and LSE = -inf on
    exactly the oracle's fully masked set (empty under a causal mask without
    padding: key 0 is allowed to every row)."""
    w = C[name]
    U.log(f"case {name}: full size B,H,N,d={w.B},{w.H},{w.N},{w.d}, one row per block")
    x = W.generate(w)
    g = np.random.default_rng(17)
    heads = np.arange(w.B * w.H)
    blocks = np.arange(0, w.N, 32)
    per_block = (heads[:, None] * w.N + blocks[None, :] +
                 g.integers(0, 32, size=(heads.size, blocks.size))).reshape(-1)
    rows = np.union1d(per_block, U.sample_rows(w.B, w.H, w.N, 96, seed=5, causal=True))
    O, L, _ = U.check_sampled(x, rows, what=name)
    assert not np.isnan(O).any() and not np.isnan(L).any()
    import oracle
    fm = oracle.fully_masked_rows(w.B, w.H, w.N, w.causal, x["mask"])
    assert np.array_equal(np.isneginf(L), fm)
    # row 0 of every head attends to key 0 only: O = v_0
    v0 = x["v"][:, :, 0].double().numpy()
    assert np.abs(O[:, :, 0] - v0).max() <= U.O_TOL[w.in_dtype]


def test_largest_sequence_at_d128():
    """N = 4194303, the largest N with N*d*4 < 2^31 at d = 128: Q and O rows
    up to 1 GB from the head's start, K and V read from their last 8192 rows,
    the only keys the mask allows (so the launch does 1.8e13 FLOP). Q is one
    drawn 8192-row block repeated along N; K and V are zero outside the
    allowed keys. The oracle sees the same rows against the 8192 allowed keys
    (non-causal: the set of keys a row attends is all that matters)."""
    dev = torch.device("cuda:0")
    L, d = 8192, 128
    N = (2**31 - 1) // (d * 4)
    w = C[C3].with_shape(B=1, H=1, N=L, causal=False)
    x = W.generate(w)
    U.log(f"case largest N: B,H,N,d=1,1,{N},{d}, keys [{N - L}, {N}) allowed")
    q = x["q"].to(dev).repeat(1, 1, -(-N // L), 1)[:, :, :N].contiguous()
    k = torch.zeros((1, 1, N, d), dtype=q.dtype, device=dev)
    v = torch.zeros_like(k)
    k[:, :, N - L:] = x["k"].to(dev)
    v[:, :, N - L:] = x["v"].to(dev)
    mask = torch.zeros((1, N), dtype=torch.uint8, device=dev)
    mask[:, N - L:] = 1
    o = torch.full(q.shape, float("nan"), dtype=q.dtype, device=dev)
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=dev)
    A.attention_fwd(q, k, v, scale=w.scale, causal=False, key_padding_mask=mask, out=o, lse=lse)
    torch.cuda.synchronize()
    g = np.random.default_rng(11)
    rows = np.unique(np.concatenate([[0, 1, L - 1, L, N // 2, N - L - 1, N - L, N - 2, N - 1],
                                     g.integers(0, N, 40)]))
    qs = torch.zeros((1, 1, L, d), dtype=x["q"].dtype)
    qs[0, 0, :len(rows)] = x["q"][0, 0][torch.from_numpy(rows % L)]
    Oref, Lref, fm = U.oracle.attention(qs, x["k"], x["v"], x["scale"], False, None, rows=np.arange(len(rows)))
    ridx = torch.from_numpy(rows).to(dev)
    Og = o[0, 0].index_select(0, ridx).float().cpu().numpy().astype(np.float64)
    Lg = lse[0, 0].index_select(0, ridx).cpu().numpy().astype(np.float64)
    e = U.compare(Og, Lg, Oref, Lref, fm, "bf16", "largest N")
    U.log(f"  {len(rows)} rows up to {N - 1}: max|dO|={e[0]:.2e} max|dLSE|={e[1]:.2e}")
    assert not torch.isnan(o).any() and not torch.isnan(lse).any()


def test_long_causal_sequence_sampled_rows():
    """Causal d = 128 at N = 262144 (one head, 2048 query tiles, K/V offsets
    up to 64 MB), sampled rows against the oracle."""
    w = C[C3].with_shape(B=1, H=1, N=262144)
    x = W.generate(w)
    U.log(f"case causal N={w.N}")
    rows = U.sample_rows(w.B, w.H, w.N, 48, seed=13, causal=True)
    O, L, _ = U.check_sampled(x, rows, what="causal N=262144")
    assert not np.isnan(O).any() and not np.isnan(L).any()


def test_nondefault_stream_and_repeat():
    w = C[C2].with_shape(B=1, H=2, N=256)
    x = W.generate(w)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        O1, L1 = U.run_gpu(x)
    O2, L2 = U.run_gpu(x)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


@pytest.mark.parametrize("B,H,N,causal,tile", [(1, 16, 4096, False, (256, 64)), (1, 12, 8192, True, (256, 64)),
                                              (1, 8, 8192, True, (128, 32))])
def test_default_tile_is_the_shape_rule(B, H, N, causal, tile):
    """Without a tile, fa_fwd runs the tile fa_default_tile names for the
    shape: bit-identical to fa_fwd_ex with that tile, and the oracle agrees
    on sampled rows."""
    from online_softmax_03_amd import capi
    w = C[C3].with_shape(B=B, H=H, N=N, causal=causal)
    assert capi.fa_default_tile(B, H, N, 128, capi.FA_DTYPE_BF16, capi.FA_DTYPE_BF16, int(causal), 0) == (0, tile)
    x = W.generate(w)
    U.log(f"case default tile B,H,N={B},{H},{N} causal={causal} -> {tile}")
    O1, L1 = U.run_gpu(x)
    O2, L2 = U.run_gpu(x, tile=tile)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)
    U.check_sampled(x, U.sample_rows(B, H, N, 48, 5 + N, causal), what=f"default tile {tile}")


@pytest.mark.parametrize("d,dtype,causal", [(64, "f16", False), (128, "bf16", True), (64, "bf16", True),
                                            (128, "f16", False)])
def test_general_key_mask(d, dtype, causal):
    """A key mask whose valid entries are not contiguous (random, plus an
    all-padded batch and a single valid key) takes the per-key lookup path."""
    N, B, H = 211, 4, 2
    w = C[C5].with_shape(B=B, H=H, N=N, d=d, in_dtype=dtype, out_dtype=dtype, causal=causal,
                         key_padding=False)
    x = W.generate(w)
    g = torch.Generator().manual_seed(77 + d)
    mask = (torch.rand((B, N), generator=g) > 0.5).to(torch.uint8)
    mask[1] = 0                      # every key padded
    mask[2] = 0
    mask[2, 150] = 1                 # a single valid key (causal rows < 150 see none)
    mask[3, ::7] = 1                 # sparse, non-contiguous
    x["mask"] = mask
    U.check_full(x, what=f"general mask d={d} {dtype} causal={causal}")


def _all_tiles():
    from online_softmax_03_amd import capi
    out = []
    for d in (64, 128):
        for br in (64, 128, 256, 512):
            for bc in (32, 64, 128):
                if capi.fa_tile_supported(d, capi.FA_DTYPE_BF16, capi.FA_DTYPE_BF16, (br, bc)) == 0:
                    out.append((d, br, bc))
    return out


@pytest.mark.parametrize("d,br,bc", _all_tiles())
@pytest.mark.parametrize("causal", [False, True])
def test_every_tile_shape(d, br, bc, causal):
    """Every compiled (block_r, block_c) through fa_fwd_ex, with a ragged N
    and a padding mask on one batch."""
    w = C[C3].with_shape(B=2, H=2, N=301, d=d, causal=causal)
    x = W.generate(w, lens=torch.tensor([301, 97]))
    U.check_full(x, tile=(br, bc), what=f"tile {br}x{bc} d={d} causal={causal}")


# Logit patterns whose row maxima grow by far more than 2^8 (in exp2 units)
# after a row's first key tile, so the running state is rescaled: in every
# tile ("ramp", by 2^16 or more per tile), once in the second or third tile
# ("spike_early"), only in the last tile ("spike_last") and in half of the
# workgroups ("mixed": batch 0 random, batch 1 ramp). The ramp reaches 2^150
# over 300 keys, far past the float32 range of an unrescaled sum.
GROWTH = ["ramp", "spike_early", "spike_last", "mixed"]


def _growing_logits(x, pattern):
    q, k = x["q"].clone(), x["k"].clone()
    N = q.shape[2]
    if pattern in ("ramp", "mixed"):
        sel = slice(None) if pattern == "ramp" else slice(1, 2)
        q[sel] = 0
        q[sel, ..., 0] = 1
        k[sel, ..., 0] = (4.0 * torch.arange(N, dtype=torch.float32)).to(k.dtype)
    else:
        key = N - 1 if pattern == "spike_last" else 70
        q[..., 0] = 8
        k[..., key, 0] = 60
    y = dict(x)
    y["q"], y["k"] = q.contiguous(), k.contiguous()
    return y


@pytest.mark.parametrize("pattern", GROWTH)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("base,over", [(C3, dict(B=2, H=2, N=300)),
                                       (C2, dict(B=2, H=2, N=300)),
                                       (C5, dict(B=2, H=2, N=300, key_padding=False))],
                         ids=["bf16_d128", "bf16_d64_f32out", "f16_d64"])
def test_growing_logits_rescale(base, over, causal, pattern):
    w = C[base].with_shape(causal=causal, **over)
    x = _growing_logits(W.generate(w), pattern)
    what = f"{base} {pattern} causal={causal}"
    U.log(f"case {what}: B,H,N,d={w.B},{w.H},{w.N},{w.d}")
    U.check_full(x, what=what)


@pytest.mark.parametrize("pattern", ["ramp", "spike_last"])
@pytest.mark.parametrize("base", [C3, C2])
def test_growing_logits_split_kv(base, pattern):
    w = C[base].with_shape(B=1, H=2, N=300, causal=True)
    x = _growing_logits(W.generate(w), pattern)
    U.log(f"case {base} {pattern} split-KV 3 parts")
    U.check_full(x, what=f"{base} {pattern} split 3", num_splits=3)
