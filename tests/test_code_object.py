"""Resource use of the built gfx950 kernels, read on the host from the code
objects inside libmla.so (no GPU needed).

Guards stage 1's register budget: the instances that the dense bf16, fp8 and
per-token decodes and the sparse decode run at H = 128 hold no scratch memory.
A spilled value there is written back to HBM by the L2 and reloaded behind a
full memory wait once per segment, and every other stage-1 instance stays
within a few dozen bytes of scratch per lane.
"""
import os
import struct

import pytest

msgpack = pytest.importorskip("msgpack")

import mla_paged_latent_decode_amd as mla  # noqa: E402

SHT_NOTE = 7
NT_AMDGPU_METADATA = 32
BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def _sections(elf: bytes):
    """(name, type, bytes) of every section of a little-endian ELF64 file."""
    assert elf[:4] == b"\x7fELF" and elf[4] == 2 and elf[5] == 1, "not a little-endian ELF64 file"
    shoff, = struct.unpack_from("<Q", elf, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", elf, 0x3A)
    heads = [struct.unpack_from("<IIQQQQIIQQ", elf, shoff + i * shentsize) for i in range(shnum)]
    strtab = heads[shstrndx]
    names = elf[strtab[4]:strtab[4] + strtab[5]]
    out = []
    for name_off, typ, _flags, _addr, off, size, *_ in heads:
        name = names[name_off:names.index(b"\0", name_off)].decode()
        out.append((name, typ, elf[off:off + size]))
    return out


def _gfx950_code_objects(fatbin: bytes):
    """The gfx950 entries of the clang offload bundles concatenated in a
    .hip_fatbin section (one bundle per translation unit)."""
    pos = fatbin.find(BUNDLE_MAGIC)
    while pos >= 0:
        count, = struct.unpack_from("<Q", fatbin, pos + len(BUNDLE_MAGIC))
        at = pos + len(BUNDLE_MAGIC) + 8
        for _ in range(count):
            off, size, tlen = struct.unpack_from("<QQQ", fatbin, at)
            at += 24
            triple = fatbin[at:at + tlen].decode()
            at += tlen
            if triple.endswith("gfx950") and size:
                yield fatbin[pos + off:pos + off + size]
        pos = fatbin.find(BUNDLE_MAGIC, pos + 1)


def _kernel_metadata(code_object: bytes):
    """amdhsa.kernels of a code object's NT_AMDGPU_METADATA note (msgpack)."""
    for _name, typ, data in _sections(code_object):
        if typ != SHT_NOTE:
            continue
        at = 0
        while at + 12 <= len(data):
            namesz, descsz, ntype = struct.unpack_from("<III", data, at)
            name = data[at + 12:at + 12 + namesz].rstrip(b"\0")
            desc_at = at + 12 + (namesz + 3) // 4 * 4
            if ntype == NT_AMDGPU_METADATA and name == b"AMDGPU":
                return msgpack.unpackb(data[desc_at:desc_at + descsz], raw=False)["amdhsa.kernels"]
            at = desc_at + (descsz + 3) // 4 * 4
    return []


@pytest.fixture(scope="module")
def kernels():
    path = mla.library_path()
    if not os.path.exists(path):
        pytest.skip("libmla.so is not built (run __graft_entry__.build())")
    with open(path, "rb") as f:
        lib = f.read()
    fatbins = [data for name, _t, data in _sections(lib) if name == ".hip_fatbin"]
    assert fatbins, "libmla.so holds no .hip_fatbin section"
    out = {}
    for co in _gfx950_code_objects(fatbins[0]):
        for k in _kernel_metadata(co):
            out[k[".name"]] = k
    assert out, "no gfx950 kernel metadata found"
    return out


def _stage1(kernels, hpw, waves, d, dv, ring, narrow, gather, pt):
    """Metadata of mla_stage1<hpw, waves, d, dv, ring, narrow, gather, pt>."""
    key = (f"10mla_stage1ILi{hpw}ELi{waves}ELi{d}ELi{dv}ELi{ring}ELb{int(narrow)}"
           f"ELb{int(gather)}ELi{pt}EE")
    hits = [v for n, v in kernels.items() if key in n]
    assert len(hits) == 1, f"stage-1 instance {key} not found exactly once"
    return hits[0]


def test_every_kernel_fits_the_cu(kernels):
    for name, k in kernels.items():
        assert k[".group_segment_fixed_size"] <= 160 * 1024, name
        # on gfx950 the count spans both register files (VGPRs and AGPRs)
        assert k[".vgpr_count"] <= 512, name
        assert k[".wavefront_size"] == 64, name


@pytest.mark.parametrize("ring,narrow,gather,pt", [
    (3, False, False, 0),  # bf16 cache (dsv3, long-context, multi-token decode)
    (3, True, False, 0),   # per-tensor fp8 cache
    (2, True, False, 1),   # per-token fp8 cache
    (2, True, False, 2),   # per-token int8 cache
    (2, True, False, 3),   # per-token int4 cache
    (3, False, True, 0),   # sparse decode over a bf16 cache
])
def test_h128_stage1_holds_no_scratch(kernels, ring, narrow, gather, pt):
    k = _stage1(kernels, 32, 4, 576, 512, ring, narrow, gather, pt)
    assert k[".private_segment_fixed_size"] == 0, k[".name"]
    assert k.get(".vgpr_spill_count", 0) == 0, k[".name"]


def test_every_stage1_instance_spills_little(kernels):
    stage1 = {n: k for n, k in kernels.items() if "mla_stage1" in n}
    assert len(stage1) >= 64, len(stage1)
    worst = max(stage1.values(), key=lambda k: k[".private_segment_fixed_size"])
    assert worst[".private_segment_fixed_size"] <= 64, worst[".name"]
