"""The occupancy the host code assumes, checked against the built library.

The launch rules in fa_api.hip size grids by the workgroups one compute unit
holds at once (the split-KV part count, the equal-progress priority flag),
and the design keeps the hot kernels free of register spills. Both rest on
the register, LDS and scratch use the compiler chose, which the code objects
inside libfa.so record in their AMDGPU metadata note. These tests read that
note (offload bundle -> gfx950 ELF -> NT_AMDGPU_METADATA, msgpack) and check
the figures the host logic depends on. No GPU is needed.

gfx950 has a unified register file of 512 registers per lane and SIMD; a
wave's allocation is the register block count of its kernel descriptor
(compute_pgm_rsrc1 bits 5:0, blocks of 8 registers, architectural and
accumulation registers together), so waves per SIMD = 512 // that, at most 8.
The descriptor can allocate more than the metadata's `.vgpr_count` when LDS
already caps the occupancy (the compiler then widens the register budget).
"""
import shutil
import struct
import subprocess

import pytest

from online_softmax_03_amd import capi

msgpack = pytest.importorskip("msgpack")

LDS_PER_CU = 160 * 1024
NT_AMDGPU_METADATA = 32
SHT_SYMTAB = 2
SHT_NOTE = 7
KD_RSRC1 = 48  # byte offset of compute_pgm_rsrc1 in a kernel descriptor


def _sections(elf: bytes):
    shoff = struct.unpack_from("<Q", elf, 0x28)[0]
    shnum, shstrndx = struct.unpack_from("<HH", elf, 0x3C)
    hdr = [struct.unpack_from("<IIQQQQIIQQ", elf, shoff + 64 * i) for i in range(shnum)]
    strtab = hdr[shstrndx][4]
    out = []
    for h in hdr:
        start = strtab + h[0]
        out.append((elf[start:elf.index(b"\0", start)].decode(), h[1], h[4], h[5]))
    return out


def _descriptor_registers(co: bytes):
    """{kernel symbol: registers its descriptor allocates per lane}."""
    shoff = struct.unpack_from("<Q", co, 0x28)[0]
    shnum = struct.unpack_from("<H", co, 0x3C)[0]
    hdr = [struct.unpack_from("<IIQQQQIIQQ", co, shoff + 64 * i) for i in range(shnum)]
    out = {}
    for symtab in (h for h in hdr if h[1] == SHT_SYMTAB):
        strtab = hdr[symtab[6]]
        for k in range(symtab[5] // 24):
            name_off, _info, _other, shndx, value, _size = struct.unpack_from("<IBBHQQ", co, symtab[4] + 24 * k)
            start = strtab[4] + name_off
            name = co[start:co.index(b"\0", start)].decode()
            if name.endswith(".kd") and 0 < shndx < len(hdr):
                sec = hdr[shndx]
                rsrc1 = struct.unpack_from("<I", co, sec[4] + (value - sec[3]) + KD_RSRC1)[0]
                out[name[:-3]] = ((rsrc1 & 0x3F) + 1) * 8
    return out


def _kernels_of_code_object(co: bytes):
    found = []
    regs = _descriptor_registers(co)
    for _name, kind, off, size in _sections(co):
        if kind != SHT_NOTE:
            continue
        q, end = off, off + size
        while q < end:
            namesz, descsz, ntype = struct.unpack_from("<III", co, q)
            q += 12
            owner = co[q:q + namesz]
            q += (namesz + 3) & ~3
            desc = co[q:q + descsz]
            q += (descsz + 3) & ~3
            if ntype == NT_AMDGPU_METADATA and owner.startswith(b"AMDGPU"):
                for k in msgpack.unpackb(desc, raw=False)["amdhsa.kernels"]:
                    k["allocated"] = regs[k[".name"]]
                    found.append(k)
    return found


def _library_kernels():
    lib = open(capi.LIB_PATH, "rb").read()
    fatbin = [s for s in _sections(lib) if s[0] == ".hip_fatbin"]
    assert fatbin, "libfa.so carries no .hip_fatbin section"
    _, _, off, size = fatbin[0]
    blob = lib[off:off + size]
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    kernels, i = [], 0
    while (j := blob.find(magic, i)) >= 0:
        n = struct.unpack_from("<Q", blob, j + len(magic))[0]
        p = j + len(magic) + 8
        for _ in range(n):
            eoff, esize, tlen = struct.unpack_from("<QQQ", blob, p)
            p += 24
            triple = blob[p:p + tlen].decode()
            p += tlen
            if triple.endswith("gfx950") and esize:
                kernels += _kernels_of_code_object(blob[j + eoff:j + eoff + esize])
        i = j + 1
    return kernels


@pytest.fixture(scope="module")
def kernels():
    cxxfilt = shutil.which("c++filt")
    if cxxfilt is None:
        pytest.skip("c++filt is not installed")
    ks = _library_kernels()
    names = subprocess.run([cxxfilt], input="\n".join(k[".name"] for k in ks), capture_output=True,
                           text=True, check=True).stdout.splitlines()
    assert len(names) == len(ks)
    table = {}
    for k, name in zip(ks, names):
        assert k["allocated"] >= k[".vgpr_count"], name  # .vgpr_count includes any AGPRs
        table[name.split("(")[0].removeprefix("void ")] = dict(
            waves=min(8, 512 // k["allocated"]), vgprs=k[".vgpr_count"], allocated=k["allocated"],
            lds=k[".group_segment_fixed_size"], scratch=k[".private_segment_fixed_size"],
            threads=k[".max_flat_workgroup_size"])
    return table


def _select(table, prefix, **flags):
    """Kernels whose demangled name starts with prefix and whose template
    arguments, split at commas, match flags given as {position: text}."""
    out = {}
    for name, r in table.items():
        if not name.startswith(prefix + "<"):
            continue
        args = [a.strip() for a in name[len(prefix) + 1:-1].split(",")]
        if all(args[int(pos[1:])] == val for pos, val in flags.items()):
            out[name] = r
    return out


def _wgs_per_cu(r):
    waves_per_wg = r["threads"] // 64
    by_regs = 4 * r["waves"] // waves_per_wg
    by_lds = LDS_PER_CU // max(r["lds"], 1)
    return min(by_regs, by_lds)


def test_every_kernel_is_found(kernels):
    assert len(kernels) > 200
    for prefix in ("fa::attn_fwd_kernel", "fa::attn_fwd_f32_kernel", "fa::attn_fwd_fp8_kernel",
                   "fa::attn_merge_kernel", "fa::attn_bwd_dq_kernel", "fa::attn_bwd_dkdv_kernel",
                   "fa::attn_bwd_fused_kernel", "fa::attn_bwd_prep_kernel", "fa::softmax_resident_kernel",
                   "fa::softmax_resident_lds_kernel", "fa::softmax_stream_kernel"):
        assert _select(kernels, prefix), prefix


def test_headline_kernel_runs_three_waves_per_simd(kernels):
    r = kernels["fa::attn_fwd_kernel<128, 32, 4, fa::BF16, fa::BF16, true, false, false>"]
    assert r["waves"] == 3 and r["scratch"] == 0 and _wgs_per_cu(r) == 3


@pytest.mark.parametrize("ti,d,block_c,nw,resident", [
    ("fa::BF16", 128, 32, 4, 3), ("fa::F16", 128, 32, 4, 3),
    ("fa::BF16", 64, 64, 8, 2), ("fa::F16", 64, 64, 8, 2),
])
def test_split_forms_hold_the_assumed_workgroups_per_cu(kernels, ti, d, block_c, nw, resident):
    """fa_splitkv_num_splits counts 256 x resident_wgs_per_cu slots for the
    default tile's split forms (fourth template flag true)."""
    forms = _select(kernels, "fa::attn_fwd_kernel", a0=str(d), a1=str(block_c), a2=str(nw), a3=ti, a7="true")
    assert len(forms) == 4
    for name, r in forms.items():
        assert _wgs_per_cu(r) >= resident, (name, r)


@pytest.mark.parametrize("ti,d,block_c,nw,resident", [
    ("fa::BF16", 128, 32, 4, 3), ("fa::F16", 128, 32, 4, 3),
    ("fa::BF16", 64, 64, 8, 2), ("fa::F16", 64, 64, 8, 2),
])
def test_unmasked_noncausal_forms_hold_the_assumed_workgroups_per_cu(kernels, ti, d, block_c, nw, resident):
    """The equal-progress flag is set for non-causal launches without a key
    mask whose whole grid fits 256 x resident_wgs_per_cu workgroups."""
    forms = _select(kernels, "fa::attn_fwd_kernel", a0=str(d), a1=str(block_c), a2=str(nw), a3=ti,
                    a5="false", a6="false", a7="false")
    assert len(forms) == 2  # the input dtype as output, and fp32 output
    for name, r in forms.items():
        assert _wgs_per_cu(r) >= resident, (name, r)


@pytest.mark.parametrize("ti", ["fa::BF16", "fa::F16"])
def test_every_form_of_the_d128_default_tile_runs_three_waves_per_simd(kernels, ti):
    """Split-KV and key-masked forms carry a three-wave bound; the others
    stay below it by themselves."""
    forms = _select(kernels, "fa::attn_fwd_kernel", a0="128", a1="32", a2="4", a3=ti)
    assert len(forms) == 12  # {input dtype, fp32} output x causal x mask, and 4 split forms
    for name, r in forms.items():
        assert r["waves"] >= 3 and r["scratch"] == 0, (name, r)


@pytest.mark.parametrize("d,resident", [(64, 2), (128, 1)])
def test_fp32_input_tiles_hold_the_assumed_workgroups_per_cu(kernels, d, resident):
    forms = _select(kernels, "fa::attn_fwd_f32_kernel", a0=str(d), a1="64", a2="4")
    assert forms
    for name, r in forms.items():
        assert _wgs_per_cu(r) >= resident, (name, r)


def test_fused_d64_backward_fits_three_workgroups_per_cu(kernels):
    forms = _select(kernels, "fa::attn_bwd_fused_kernel")
    assert forms
    for name, r in forms.items():
        assert _wgs_per_cu(r) >= 3, (name, r)


# Kernels allowed a few bytes of scratch (register spill), each below 16 bytes
# per lane: the bf16 forms of the largest 16-bit shape of the LDS-backed row
# softmax.
SPILL_ALLOWED = {
    "fa::softmax_resident_lds_kernel<fa::BF16, fa::BF16, 768, 14, 13>",
    "fa::softmax_resident_lds_kernel<fa::BF16, fa::F32, 768, 14, 13>",
}


def test_no_kernel_spills_beyond_the_known_few(kernels):
    for name, r in kernels.items():
        if name in SPILL_ALLOWED:
            assert r["scratch"] < 16, (name, r)
        else:
            assert r["scratch"] == 0, (name, r)
