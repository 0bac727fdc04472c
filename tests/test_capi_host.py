"""Host-only checks of the C ABI: the library loads, exports every function
include/fa.h declares, and rejects every invalid argument with the documented
status before touching the device (so these run without a GPU).

Every call below carries exactly one invalid argument that validation
rejects; none of them reaches a kernel launch.
"""
import ctypes
import os
import re

import pytest

from online_softmax_03_amd import capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

BF16, F16, F32 = capi.FA_DTYPE_BF16, capi.FA_DTYPE_F16, capi.FA_DTYPE_F32
P = 1 << 20  # a 16-byte-aligned stand-in address; never dereferenced in these tests


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(capi.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(capi.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_strerror_names_every_status():
    names = {s: capi.fa_strerror(s) for s in range(-12, 1)}
    assert names[0] == "ok"
    assert len(set(names.values())) == len(names)
    assert capi.fa_strerror(-99) == "unknown status"


def _fwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=128, d=128, scale=0.125, causal=0,
             key_padding_mask=None, in_dtype=BF16, out_dtype=BF16, stream=None)
    a.update(kw)
    tile = a.pop("tile", None)
    return capi.fa_fwd_ex(*a.values(), tile=tile)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), capi.FA_ERR_NULL), (dict(k=None), capi.FA_ERR_NULL),
    (dict(v=None), capi.FA_ERR_NULL), (dict(o=None), capi.FA_ERR_NULL),
    (dict(lse=None), capi.FA_ERR_NULL),
    (dict(B=0), capi.FA_ERR_SHAPE), (dict(H=-1), capi.FA_ERR_SHAPE), (dict(N=0), capi.FA_ERR_SHAPE),
    (dict(d=96), capi.FA_ERR_HEADDIM), (dict(d=0), capi.FA_ERR_HEADDIM), (dict(d=256), capi.FA_ERR_HEADDIM),
    (dict(in_dtype=BF16, out_dtype=F16), capi.FA_ERR_DTYPE), (dict(in_dtype=7), capi.FA_ERR_DTYPE),
    (dict(in_dtype=F16, out_dtype=BF16), capi.FA_ERR_DTYPE),
    (dict(scale=0.0), capi.FA_ERR_SCALE), (dict(scale=-0.5), capi.FA_ERR_SCALE),
    (dict(scale=float("nan")), capi.FA_ERR_SCALE), (dict(scale=float("inf")), capi.FA_ERR_SCALE),
    (dict(q=P + 8), capi.FA_ERR_ALIGN), (dict(o=P + 2), capi.FA_ERR_ALIGN), (dict(lse=P + 2), capi.FA_ERR_ALIGN),
    (dict(tile=(96, 64)), capi.FA_ERR_TILE), (dict(tile=(128, 48)), capi.FA_ERR_TILE),
    (dict(tile=(-32, 64)), capi.FA_ERR_TILE),
    (dict(B=1 << 16, H=1 << 16, N=1 << 16), capi.FA_ERR_SHAPE),
    # a row index times the bytes of a float32 row must fit in 31 bits: N = 2^22
    # is one past the largest sequence at d = 128, N = 2^23 at d = 64
    (dict(N=1 << 22), capi.FA_ERR_SHAPE), (dict(N=1 << 23, d=64), capi.FA_ERR_SHAPE),
])
def test_invalid_arguments_rejected_on_host(kw, status):
    assert _fwd(**kw) == status


def test_fa_fwd_is_fa_fwd_ex_with_default_tile():
    assert capi.fa_fwd(None, P, P, P, P, 1, 1, 8, 64, 0.1, 0, None, BF16, BF16, None) == capi.FA_ERR_NULL
    assert capi.fa_fwd(P, P, P, P, P, 1, 1, 8, 64, 0.1, 0, None, BF16, F16, None) == capi.FA_ERR_DTYPE


def test_default_tile_and_supported_tiles():
    st, t = capi.fa_default_tile(2, 32, 8192, 128, BF16, BF16, 1, 0)
    assert st == capi.FA_OK and t[0] % 32 == 0 and t[1] % 32 == 0
    assert capi.fa_tile_supported(128, BF16, BF16, t) == capi.FA_OK
    assert capi.fa_tile_supported(128, BF16, BF16, (0, 0)) == capi.FA_OK
    assert capi.fa_tile_supported(128, BF16, BF16, (96, 64)) == capi.FA_ERR_TILE
    assert capi.fa_default_tile(1, 1, 8192, 96, BF16, BF16, 1, 0)[0] == capi.FA_ERR_HEADDIM
    assert capi.fa_default_tile(1, 1, 0, 128, BF16, BF16, 1, 0)[0] == capi.FA_ERR_SHAPE
    assert capi.fa_default_tile(0, 1, 64, 128, BF16, BF16, 1, 0)[0] == capi.FA_ERR_SHAPE
    assert capi.fa_default_tile(1, 0, 64, 128, BF16, BF16, 1, 0)[0] == capi.FA_ERR_SHAPE
    for d in (64, 128):
        for pair in ((BF16, BF16), (BF16, F32), (F16, F16), (F16, F32), (F32, F32)):
            for B, H, N, causal in ((1, 1, 4096, 0), (2, 32, 8192, 1), (1, 8, 32768, 1), (4, 16, 2048, 0)):
                st, t = capi.fa_default_tile(B, H, N, d, *pair, causal, 0)
                assert st == capi.FA_OK and capi.fa_tile_supported(d, *pair, t) == capi.FA_OK


@pytest.mark.parametrize("B,H,N,causal,tile", [
    # 16-bit d = 128: 256 x 64 for long key loops over a grid that covers the CUs
    (1, 8, 32768, 1, (256, 64)), (1, 12, 8192, 1, (256, 64)), (1, 16, 8192, 1, (256, 64)),
    (1, 8, 16384, 1, (256, 64)), (4, 16, 4096, 0, (256, 64)), (1, 8, 8192, 0, (256, 64)),
    (2, 16, 8192, 0, (256, 64)),
    # short loops, 256 and fewer causal workgroups of 256 rows, or more than
    # 1024 of them: 128 x 32
    (2, 32, 8192, 1, (128, 32)), (2, 32, 16384, 1, (128, 32)), (1, 8, 8192, 1, (128, 32)),
    (1, 4, 16384, 1, (128, 32)), (2, 32, 6144, 1, (128, 32)), (4, 32, 4096, 1, (128, 32)),
    (8, 16, 2048, 0, (128, 32)), (1, 4, 8192, 0, (128, 32)), (2, 32, 8192, 0, (128, 32)),
    (1, 1, 256, 0, (128, 32)),
])
def test_default_tile_follows_the_shape_rule(B, H, N, causal, tile):
    for dt in (BF16, F16):
        for has_mask in (0, 1):
            assert capi.fa_default_tile(B, H, N, 128, dt, dt, causal, has_mask) == (capi.FA_OK, tile)
    # d = 64 and fp32 inputs keep their one base tile
    assert capi.fa_default_tile(B, H, N, 64, BF16, BF16, causal, 0) == (capi.FA_OK, (256, 64))
    assert capi.fa_default_tile(B, H, N, 128, F32, F32, causal, 0) == (capi.FA_OK, (128, 64))


def test_splitkv_workspace_bytes():
    # [S][B*H*N][d] float32 partial outputs, then [S][B*H*N] float32 LSEs
    assert capi.fa_splitkv_workspace_bytes(2, 3, 100, 64, 4) == 4 * 2 * 3 * 100 * (64 + 1) * 4
    assert capi.fa_splitkv_workspace_bytes(1, 1, 1, 128, 1) == (128 + 1) * 4
    for bad in ((0, 1, 8, 64, 2), (1, 1, 0, 64, 2), (1, 1, 8, 96, 2), (1, 1, 8, 64, 0),
                (1, 1, 8, 64, capi.FA_MAX_SPLITS + 1), (1 << 16, 1 << 16, 1 << 16, 64, 1)):
        assert capi.fa_splitkv_workspace_bytes(*bad) == 0, bad


def test_splitkv_num_splits_heuristic():
    # equal parts per query tile: a full grid needs no split; a small one
    # splits until its parts fill the 768 (d = 128, 16-bit) or 512 (d = 64)
    # resident workgroup slots, keeping at least four key tiles per part, and
    # into at most 8 parts
    n = capi.fa_splitkv_num_splits
    assert n(2, 32, 8192, 128, BF16, 0) == 1
    assert n(1, 16, 8192, 128, BF16, 0) == 1   # 1024 workgroups
    assert n(1, 8, 8192, 128, BF16, 0) == 2    # 512 -> 1024
    assert n(1, 4, 8192, 128, BF16, 0) == 3    # 256 -> 768
    assert n(1, 2, 8192, 128, BF16, 0) == 6    # 128 -> 768
    assert n(1, 8, 2048, 64, BF16, 0) == 8     # 64 -> 512 (32 key tiles / 8)
    assert n(1, 1, 8192, 128, BF16, 0) == 8    # 64 -> 512: at most 8 parts
    assert n(1, 1, 2048, 64, BF16, 0) == 8     # capped: 32 key tiles, 4 per part
    for B, H, N, d in [(1, 2, 4096, 128), (1, 1, 8192, 128), (3, 5, 1000, 64), (1, 1, 300, 128)]:
        s = n(B, H, N, d, BF16, 0)
        br, bc, slots = (128, 32, 768) if d == 128 else (256, 64, 512)
        grid, tiles = B * H * -(-N // br), -(-N // bc)
        assert 1 <= s <= 8
        assert s == 1 or tiles // s >= 4                       # every part keeps four key tiles
        assert grid * s >= slots or s == 8 or tiles // (s + 1) < 4   # and no fewer parts would do
        assert s == 1 or grid * (s - 1) < slots
    assert n(1, 1, 64, 128, BF16, 0) == 1  # too few key tiles to split
    # causal, at most 256 query tiles: parts in proportion to the causal
    # extent (about half the workgroups of equal parts), counted until they
    # reach 9/16 of the slots (432 at d = 128), at most 12
    assert n(1, 1, 8192, 128, BF16, 1) == 12   # 374 workgroups at 12 (u = 6: 24 key tiles per part)
    assert n(1, 2, 8192, 128, BF16, 1) == 6    # 2 x 219 = 438
    assert n(1, 4, 8192, 128, BF16, 1) == 3    # 4 x 126 = 504 (4 x 96 = 384 at 2)
    assert n(1, 8, 4096, 128, BF16, 1) == 3    # 256 query tiles: still proportional
    assert n(1, 8, 8192, 128, BF16, 1) == 2    # 512 query tiles: equal parts, as without the mask
    assert n(2, 32, 8192, 128, BF16, 1) == 1
    assert n(1, 1, 64, 128, BF16, 1) == 1      # two key tiles: no split
    # fp32 inputs (64-key tiles on the fp32 MFMA) split down to one tile per part
    assert n(1, 1, 256, 64, capi.FA_DTYPE_F32, 0) == 4
    assert n(1, 1, 256, 64, capi.FA_DTYPE_F32, 1) == 4
    assert n(1, 1, 64, 64, capi.FA_DTYPE_F32, 0) == 1
    assert n(1, 1, 0, 128, BF16, 0) == capi.FA_ERR_SHAPE
    assert n(1, 1, 64, 80, BF16, 1) == capi.FA_ERR_HEADDIM
    assert n(1, 1, 64, 64, 9, 0) == capi.FA_ERR_DTYPE


def _split(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=128, d=128, scale=0.125, causal=0,
             key_padding_mask=None, in_dtype=BF16, out_dtype=BF16, num_splits=2, workspace=P,
             workspace_bytes=1 << 30, stream=None)
    a.update(kw)
    return capi.fa_fwd_splitkv(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), capi.FA_ERR_NULL), (dict(lse=None), capi.FA_ERR_NULL),
    (dict(N=0), capi.FA_ERR_SHAPE), (dict(d=32), capi.FA_ERR_HEADDIM),
    (dict(out_dtype=F16), capi.FA_ERR_DTYPE), (dict(scale=float("nan")), capi.FA_ERR_SCALE),
    (dict(v=P + 4), capi.FA_ERR_ALIGN),
    (dict(num_splits=0), capi.FA_ERR_SPLITS), (dict(num_splits=capi.FA_MAX_SPLITS + 1), capi.FA_ERR_SPLITS),
    (dict(workspace=None), capi.FA_ERR_WORKSPACE), (dict(workspace=P + 8), capi.FA_ERR_WORKSPACE),
    (dict(workspace_bytes=2 * 128 * 129 * 4 - 1), capi.FA_ERR_WORKSPACE),
    (dict(B=1 << 16, H=1 << 16, N=1 << 16), capi.FA_ERR_SHAPE),
])
def test_splitkv_invalid_arguments_rejected_on_host(kw, status):
    assert _split(**kw) == status


def _sm(**kw):
    a = dict(x=P, y=P, lse=P, rows=4, cols=64, in_dtype=BF16, out_dtype=BF16, stream=None)
    a.update(kw)
    return capi.fa_softmax_fwd(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), capi.FA_ERR_NULL), (dict(y=None), capi.FA_ERR_NULL),
    (dict(rows=0), capi.FA_ERR_SHAPE), (dict(cols=0), capi.FA_ERR_SHAPE), (dict(rows=-3), capi.FA_ERR_SHAPE),
    (dict(rows=1 << 31), capi.FA_ERR_SHAPE), (dict(rows=1 << 30, cols=1 << 11), capi.FA_ERR_SHAPE),
    (dict(in_dtype=BF16, out_dtype=F16), capi.FA_ERR_DTYPE), (dict(in_dtype=F32, out_dtype=BF16), capi.FA_ERR_DTYPE),
    (dict(in_dtype=5), capi.FA_ERR_DTYPE),
    (dict(x=P + 2), capi.FA_ERR_ALIGN), (dict(y=P + 8), capi.FA_ERR_ALIGN), (dict(lse=P + 1), capi.FA_ERR_ALIGN),
])
def test_softmax_invalid_arguments_rejected_on_host(kw, status):
    assert _sm(**kw) == status


def test_bwd_workspace_bytes():
    assert capi.fa_bwd_workspace_bytes(2, 3, 100) == 2 * 3 * 2 * 64 * 4 * 2  # ceil(100/64)=2 -> 4 groups
    assert capi.fa_bwd_workspace_bytes(1, 1, 64) == 64 * 2 * 4
    assert capi.fa_bwd_workspace_bytes(1, 1, 0) == 0
    assert capi.fa_bwd_workspace_bytes(1 << 16, 1 << 16, 1 << 16) == 0


def _bwd(**kw):
    a = dict(q=P, k=P, v=P, o=P, dout=P, lse=P, dq=P, dk=P, dv=P, B=1, H=1, N=128, d=128, scale=0.125, causal=0,
             key_padding_mask=None, in_dtype=BF16, grad_dtype=BF16, workspace=P, workspace_bytes=1 << 30,
             stream=None)
    a.update(kw)
    return capi.fa_bwd(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), capi.FA_ERR_NULL), (dict(dout=None), capi.FA_ERR_NULL), (dict(lse=None), capi.FA_ERR_NULL),
    (dict(dv=None), capi.FA_ERR_NULL), (dict(N=0), capi.FA_ERR_SHAPE), (dict(d=96), capi.FA_ERR_HEADDIM),
    (dict(in_dtype=F32, grad_dtype=F32), capi.FA_ERR_DTYPE), (dict(grad_dtype=F16), capi.FA_ERR_DTYPE),
    (dict(scale=-1.0), capi.FA_ERR_SCALE), (dict(o=P + 8), capi.FA_ERR_ALIGN), (dict(lse=P + 2), capi.FA_ERR_ALIGN),
    (dict(workspace=None), capi.FA_ERR_WORKSPACE), (dict(workspace_bytes=128 * 2 * 4 - 4), capi.FA_ERR_WORKSPACE),
    (dict(B=1 << 16, H=1 << 16, N=1 << 16), capi.FA_ERR_SHAPE),
])
def test_bwd_invalid_arguments_rejected_on_host(kw, status):
    assert _bwd(**kw) == status


def _fp8(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=128, d=128, scale=0.125, descale_q=1.0, descale_k=1.0,
             descale_v=1.0, causal=0, key_padding_mask=None, out_dtype=BF16, max_offset=8, stream=None)
    a.update(kw)
    return capi.fa_fwd_fp8(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), capi.FA_ERR_NULL), (dict(v=None), capi.FA_ERR_NULL), (dict(lse=None), capi.FA_ERR_NULL),
    (dict(B=0), capi.FA_ERR_SHAPE), (dict(N=-1), capi.FA_ERR_SHAPE), (dict(d=64), capi.FA_ERR_HEADDIM),
    (dict(out_dtype=9), capi.FA_ERR_DTYPE),
    (dict(scale=0.0), capi.FA_ERR_SCALE), (dict(descale_q=-1.0), capi.FA_ERR_SCALE),
    (dict(descale_k=float("inf")), capi.FA_ERR_SCALE), (dict(descale_v=float("nan")), capi.FA_ERR_SCALE),
    (dict(max_offset=4), capi.FA_ERR_OFFSET), (dict(max_offset=-8), capi.FA_ERR_OFFSET),
    (dict(k=P + 8), capi.FA_ERR_ALIGN), (dict(lse=P + 2), capi.FA_ERR_ALIGN),
    (dict(B=1 << 16, H=1 << 16, N=1 << 16), capi.FA_ERR_SHAPE),
])
def test_fp8_invalid_arguments_rejected_on_host(kw, status):
    assert _fp8(**kw) == status


def _noalloc(**kw):
    a = dict(q=P, k=P, v=P, o=P, lse=P, B=1, H=1, N=128, d=128, scale=0.125, causal=0,
             key_padding_mask=None, in_dtype=BF16, out_dtype=BF16, num_splits=2, stream=None)
    a.update(kw)
    return capi.fa_fwd_splitkv_noalloc(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), capi.FA_ERR_NULL), (dict(o=None), capi.FA_ERR_NULL),
    (dict(H=0), capi.FA_ERR_SHAPE), (dict(d=80), capi.FA_ERR_HEADDIM),
    (dict(in_dtype=F16, out_dtype=BF16), capi.FA_ERR_DTYPE), (dict(scale=0.0), capi.FA_ERR_SCALE),
    (dict(k=P + 4), capi.FA_ERR_ALIGN),
    (dict(num_splits=0), capi.FA_ERR_SPLITS), (dict(num_splits=capi.FA_MAX_SPLITS + 1), capi.FA_ERR_SPLITS),
    # partials beyond the fixed scratch: 2 parts of 64 * 8192 rows at d = 128 (541 MB)
    (dict(H=64, N=8192, num_splits=2), capi.FA_ERR_SCRATCH),
    # one row past the limit: S * rows * (d + 1) * 4 bytes > 64 MiB
    (dict(N=(capi.FA_NOALLOC_SCRATCH_BYTES // (129 * 4)) // 2 + 1, num_splits=2), capi.FA_ERR_SCRATCH),
])
def test_noalloc_invalid_arguments_rejected_on_host(kw, status):
    """Every rejection, the size limit of the fixed scratch included, happens
    before the entry point makes any HIP call."""
    assert _noalloc(**kw) == status
