"""CPU checks of the built library's gfx950 code objects, read from their AMDGPU metadata notes.

libpe.so carries one offload bundle per HIP source in its `.hip_fatbin` section. Each bundle holds
a gfx950 ELF whose NT_AMDGPU_METADATA note (msgpack) lists every kernel with its resources. The
kernels are fully unrolled register pipelines, so the checks are:
- no private (scratch) memory: no spills, and no arrays or argument structs copied to memory;
- LDS within the 160 KB of a gfx950 CU;
- registers within the 512 of a SIMD lane;
- wave64.
"""
import struct

import pytest

pe = pytest.importorskip("vlm_vision_patch_amd", reason="libpe.so not built")
msgpack = pytest.importorskip("msgpack")

BUNDLE_MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"
SHT_NOTE = 7
NT_AMDGPU_METADATA = 32


def elf_sections(b):
    """name -> (type, offset, size) of a little-endian ELF64 image."""
    assert b[:4] == b"\x7fELF" and b[4] == 2 and b[5] == 1
    shoff, = struct.unpack_from("<Q", b, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", b, 0x3A)
    hdrs = [struct.unpack_from("<IIQQQQIIQQ", b, shoff + i * shentsize) for i in range(shnum)]
    stroff = hdrs[shstrndx][4]
    out = {}
    for h in hdrs:
        name = b[stroff + h[0]: b.index(b"\0", stroff + h[0])].decode()
        out[name] = (h[1], h[4], h[5])
    return out


def code_objects(lib_bytes, arch="gfx950"):
    """The device ELF images for `arch` in every offload bundle of the host library."""
    _, off, size = elf_sections(lib_bytes)[".hip_fatbin"]
    fb = lib_bytes[off: off + size]
    out, pos = [], 0
    while True:
        i = fb.find(BUNDLE_MAGIC, pos)
        if i < 0:
            return out
        n_entries, = struct.unpack_from("<Q", fb, i + len(BUNDLE_MAGIC))
        p = i + len(BUNDLE_MAGIC) + 8
        for _ in range(n_entries):
            e_off, e_size, t_len = struct.unpack_from("<QQQ", fb, p)
            p += 24
            triple = fb[p: p + t_len].decode()
            p += t_len
            if triple.endswith(arch):
                out.append(fb[i + e_off: i + e_off + e_size])
        pos = i + len(BUNDLE_MAGIC)


def kernels_of(co):
    for typ, off, size in elf_sections(co).values():
        if typ != SHT_NOTE:
            continue
        q = off
        while q < off + size:
            namesz, descsz, ntype = struct.unpack_from("<III", co, q)
            q += 12
            name = co[q: q + namesz]
            q += (namesz + 3) & ~3
            desc = co[q: q + descsz]
            q += (descsz + 3) & ~3
            if name.startswith(b"AMDGPU") and ntype == NT_AMDGPU_METADATA:
                yield from msgpack.unpackb(desc, raw=False)["amdhsa.kernels"]


@pytest.fixture(scope="module")
def kernels():
    cos = code_objects(open(pe.LIB_PATH, "rb").read())
    assert len(cos) >= 6, "one gfx950 code object per HIP source"
    ks = [k for co in cos for k in kernels_of(co)]
    assert ks
    return ks


def test_kernel_families_present(kernels):
    names = " ".join(k[".name"] for k in kernels)
    for fam in ("pe_fwd32_kernel", "pe_fwd32_sk_kernel", "pe_fwd16_kernel", "pe_pack_kernel",
                "pe_layernorm_kernel"):
        assert fam in names, fam


def test_no_scratch_no_spills(kernels):
    bad = [(k[".name"], k[".private_segment_fixed_size"], k[".vgpr_spill_count"], k[".sgpr_spill_count"])
           for k in kernels
           if k[".private_segment_fixed_size"] or k[".vgpr_spill_count"] or k[".sgpr_spill_count"]
           or k.get(".uses_dynamic_stack", False)]
    assert not bad, bad[:5]


def test_resources_fit_a_cu(kernels):
    for k in kernels:
        assert k[".wavefront_size"] == 64, k[".name"]
        assert k[".group_segment_fixed_size"] <= 160 * 1024, k[".name"]
        assert k[".vgpr_count"] + k.get(".agpr_count", 0) <= 512, k[".name"]
        assert k[".kernarg_segment_size"] <= 4096, k[".name"]
