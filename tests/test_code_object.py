"""CPU checks of the built library's gfx950 code objects, read from their AMDGPU metadata notes.

libpe.so carries one offload bundle per HIP source in its `.hip_fatbin` section (read by bench.py's
gfx950_code_objects). Each bundle holds a gfx950 ELF whose NT_AMDGPU_METADATA note (msgpack) lists every kernel with its resources. The
kernels are fully unrolled register pipelines, so the checks are:
- no private (scratch) memory: no spills, and no arrays or argument structs copied to memory;
- LDS within the 160 KB of a gfx950 CU;
- registers within the 512 of a SIMD lane;
- wave64.
"""
import struct
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402  (its ELF and offload-bundle reader)

pe = pytest.importorskip("vlm_vision_patch_amd", reason="libpe.so not built")
msgpack = pytest.importorskip("msgpack")

SHT_NOTE = 7
NT_AMDGPU_METADATA = 32


def kernels_of(co):
    for h in bench.elf_sections(co)[0].values():
        typ, off, size = h[1], h[4], h[5]
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
    cos = [co for _, co in bench.gfx950_code_objects(open(pe.LIB_PATH, "rb").read())]
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
