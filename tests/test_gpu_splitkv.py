"""Parity of the split-KV forward (fa_fwd_splitkv: key ranges processed by
separate workgroups, then merged) with the float64 oracle and with the
single-pass path (needs a GPU).

The merge is exact up to rounding (the online-softmax states combine
associatively), so the split path is held to the same bar as fa_fwd. Split
counts above the number of key tiles leave parts with no key at all; causal
rows near the top leave most parts empty; a batch with every key padded
leaves every part empty. The workspace is pre-filled with NaN bytes, so a
partial the attention pass fails to write poisons the merged result.
"""
import numpy as np
import pytest
import torch

from online_softmax_03_amd import attention as A
from online_softmax_03_amd import capi
from online_softmax_03_amd import workloads as W
from tests import gpu_util as U

pytestmark = pytest.mark.gpu

C = {w.name: w for w in W.WORKLOADS}
TINY, C2, C3, C4, C5 = (w.name for w in W.WORKLOADS)

SMALL = [
    # (id, base workload, shape overrides, key lengths or None, split counts)
    ("bf16_causal_d128_n333", C3, dict(B=1, H=3, N=333), None, (1, 2, 3, 7, 64)),
    ("bf16_noncausal_d128_n190_f32out", C3, dict(B=2, H=1, N=190, causal=False, out_dtype="f32"), None, (2, 5)),
    ("bf16_d64_n300_f32out", C2, dict(B=2, H=2, N=300), None, (2, 4, 9)),
    ("bf16_d64_n200_bf16out", C2, dict(B=1, H=2, N=200, out_dtype="bf16"), None, (3,)),
    ("bf16_causal_long_logits_n700", C4, dict(B=1, H=2, N=700), None, (2, 6)),
    ("f16_keypad_d64_n257", C5, dict(B=6, H=2, N=257), [0, 1, 63, 64, 256, 257], (2, 3, 64)),
    ("f16_keypad_causal_d128_f32out_n130", C5,
     dict(B=3, H=2, N=130, d=128, causal=True, out_dtype="f32"), [0, 5, 130], (2, 4)),
    ("f16_d64_n1", C5, dict(B=1, H=1, N=1, key_padding=False), None, (1, 4)),
    ("bf16_d128_n31", C3, dict(B=1, H=1, N=31), None, (2,)),
    ("f32_d64_n256", TINY, dict(B=1, H=2, N=256), None, (2, 3)),
    ("f32_causal_d128_n200_keypad", TINY, dict(B=2, H=1, N=200, d=128, causal=True), [0, 77], (2, 5)),
]


@pytest.mark.parametrize("ident,base,over,lens,splits", SMALL, ids=[s[0] for s in SMALL])
def test_small_shapes_every_row(ident, base, over, lens, splits):
    w = C[base].with_shape(**over)
    x = W.generate(w, lens=None if lens is None else torch.tensor(lens, dtype=torch.int64))
    for s in splits:
        U.log(f"case {ident} splits={s}: B,H,N,d={w.B},{w.H},{w.N},{w.d} {w.in_dtype}->{w.out_dtype} "
              f"causal={w.causal}")
        U.check_full(x, what=f"{ident} splits={s}", num_splits=s)


@pytest.mark.parametrize("d,dtype,causal", [(64, "f16", False), (128, "bf16", True)])
def test_general_key_mask(d, dtype, causal):
    """A non-contiguous key mask, an all-padded batch and a single valid key."""
    N, B, H = 211, 4, 2
    w = C[C5].with_shape(B=B, H=H, N=N, d=d, in_dtype=dtype, out_dtype=dtype, causal=causal,
                         key_padding=False)
    x = W.generate(w)
    g = torch.Generator().manual_seed(91 + d)
    mask = (torch.rand((B, N), generator=g) > 0.5).to(torch.uint8)
    mask[1] = 0
    mask[2] = 0
    mask[2, 150] = 1
    mask[3, ::7] = 1
    x["mask"] = mask
    for s in (2, 5):
        U.check_full(x, what=f"general mask d={d} {dtype} causal={causal} splits={s}", num_splits=s)


def test_matches_single_pass_at_full_size():
    """The headline shape (B=2, H=32, N=8192, d=128, bf16, causal) with two
    parts: sampled rows against the oracle, every row against fa_fwd."""
    w = C[C3]
    U.log(f"case {C3} splits=2: full size B,H,N,d={w.B},{w.H},{w.N},{w.d}")
    x = W.generate(w)
    rows = U.sample_rows(w.B, w.H, w.N, 64, seed=9, causal=w.causal)
    O, L, _ = U.check_sampled(x, rows, what=f"{C3} splits=2", num_splits=2)
    O1, L1 = U.run_gpu(x)
    dO = float(np.abs(O - O1).max())
    dL = float(np.abs(L - L1).max())
    U.log(f"  split vs single pass: max|dO|={dO:.2e} max|dLSE|={dL:.2e}")
    assert dO <= U.O_TOL["bf16"] and dL <= U.LSE_TOL


def test_auto_split_count_on_a_small_grid():
    """One batch, two heads, N=4096: 64 workgroups unsplit, so the library's
    choice splits; the result meets the bar on sampled rows."""
    w = C[C3].with_shape(B=1, H=2, N=4096)
    s = capi.fa_splitkv_num_splits(w.B, w.H, w.N, w.d, capi.FA_DTYPE_BF16, w.causal)
    U.log(f"case auto split: B,H,N,d={w.B},{w.H},{w.N},{w.d} -> {s} parts")
    assert s > 1
    x = W.generate(w)
    rows = U.sample_rows(w.B, w.H, w.N, 64, seed=4, causal=True)
    U.check_sampled(x, rows, what="auto split", num_splits=0)


def test_workspace_reuse_larger_then_smaller():
    """Two calls in a row on one workspace, the second smaller and with fewer
    parts: the second result depends only on its own inputs."""
    dev = torch.device("cuda:0")
    w1 = C[C3].with_shape(B=1, H=2, N=500)
    w2 = C[C3].with_shape(B=1, H=1, N=130, causal=False)
    ws = torch.full((capi.fa_splitkv_workspace_bytes(1, 2, 500, 128, 6),), 0xFF, dtype=torch.uint8, device=dev)
    for w, s in ((w1, 6), (w2, 3)):
        x = W.generate(w)
        q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
        o, lse = A.attention_fwd(q, k, v, scale=x["scale"], causal=x["causal"], num_splits=s, workspace=ws)
        torch.cuda.synchronize()
        import oracle
        Oref, Lref, fm = oracle.attention(x["q"], x["k"], x["v"], x["scale"], x["causal"])
        U.compare(o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64),
                  Oref, Lref, fm, "bf16", f"reuse N={w.N} splits={s}")


def test_workspace_too_small_is_rejected_before_launch():
    dev = torch.device("cuda:0")
    w = C[C3].with_shape(B=1, H=1, N=64)
    x = W.generate(w)
    q, k, v = (x[n].to(dev) for n in ("q", "k", "v"))
    need = capi.fa_splitkv_workspace_bytes(1, 1, 64, 128, 2)
    ws = torch.empty(need - 16, dtype=torch.uint8, device=dev)
    with pytest.raises(A.FaError) as e:
        A.attention_fwd(q, k, v, causal=True, num_splits=2, workspace=ws)
    assert e.value.status == capi.FA_ERR_WORKSPACE


@pytest.mark.parametrize("shape,d,dtype", [((1, 1, 32768), 128, "bf16"), ((1, 1, 32769), 128, "bf16"),
                                           ((1, 2, 8191), 64, "f16")])
def test_proportional_parts_long_causal(shape, d, dtype):
    """Causal launches with at most 256 query tiles split each tile's keys
    in proportion to its causal extent (256 query tiles of 128 rows at
    N = 32768; a ragged last tile at N = 8191, d = 64); one more query tile
    (N = 32769, 257 tiles) takes equal parts again: sampled rows against
    the oracle, every row against fa_fwd."""
    B, H, N = shape
    w = C[C3].with_shape(B=B, H=H, N=N, d=d, in_dtype=dtype, out_dtype=dtype, causal=True)
    s = capi.fa_splitkv_num_splits(B, H, N, d, U.A._DT[W.DTYPES[dtype]], True)
    U.log(f"case proportional split: B,H,N,d={B},{H},{N},{d} {dtype} -> {s} parts")
    assert s > 1
    x = W.generate(w)
    rows = U.sample_rows(B, H, N, 96, seed=17, causal=True)
    O, L, _ = U.check_sampled(x, rows, what=f"proportional split N={N} d={d}", num_splits=0)
    O1, L1 = U.run_gpu(x)
    dO = float(np.abs(O - O1).max())
    dL = float(np.abs(L - L1).max())
    U.log(f"  split vs single pass: max|dO|={dO:.2e} max|dLSE|={dL:.2e}")
    assert dO <= U.O_TOL[dtype] and dL <= U.LSE_TOL
