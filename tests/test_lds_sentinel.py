"""The LDS sentinel debug build (libpe_sentinel.so: the same sources with -DPE_LDS_SENTINEL=1, made
by build.py next to libpe.so). Its kernels fill their LDS with NaN bytes before first use, so an
LDS read that comes before the matching write turns into a NaN in the output.

CPU: the debug library exports the same symbols, its LDS kernels differ from the shipped ones
(the fill is compiled in) while the LayerNorm kernel, which uses no LDS, is identical, and its
code objects fit a CU with no scratch memory.
GPU: tests/lds_sentinel_cases.py runs every LDS path against the oracle on the debug library, in
a process of its own (the library a process loads is fixed when the binding is imported).
"""
import ctypes
import os
import subprocess
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402  (kernel_code_hash, code-object reader)

pe = pytest.importorskip("vlm_vision_patch_amd", reason="libpe.so not built")

SENTINEL = os.path.join(ROOT, "vlm_vision_patch_amd", "libpe_sentinel.so")
LDS_KERNELS = ("pe_fwd32_kernel", "pe_fwd32_sk_kernel", "pe_fwd16_kernel")


def need_lib():
    assert os.path.exists(SENTINEL), "libpe_sentinel.so is not built: python __graft_entry__.py build"


def test_sentinel_library_exports_the_abi():
    need_lib()
    lib = ctypes.CDLL(SENTINEL)
    for n in pe.EXPORTS:
        assert hasattr(lib, n), n


def test_fill_only_in_the_debug_build():
    need_lib()
    for k in LDS_KERNELS:
        assert bench.kernel_code_hash(k, SENTINEL) != bench.kernel_code_hash(k, pe.LIB_PATH), k
    assert bench.kernel_code_hash("pe_layernorm_kernel", SENTINEL) == bench.kernel_code_hash("pe_layernorm_kernel",
                                                                                          pe.LIB_PATH)


def test_sentinel_code_objects_fit_a_cu():
    need_lib()
    from test_code_object import kernels_of
    cos = [co for _, co in bench.gfx950_code_objects(open(SENTINEL, "rb").read())]
    ks = [k for co in cos for k in kernels_of(co)]
    assert ks
    for k in ks:
        assert not k[".private_segment_fixed_size"] and not k[".vgpr_spill_count"], k[".name"]
        assert k[".group_segment_fixed_size"] <= 160 * 1024, k[".name"]
        assert k[".vgpr_count"] + k.get(".agpr_count", 0) <= 512, k[".name"]


@pytest.mark.gpu
@pytest.mark.timeout(420)
def test_parity_on_the_lds_sentinel_build():
    need_lib()
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("[case] LDS sentinel build: tests/lds_sentinel_cases.py", flush=True)
    env = dict(os.environ, PE_LIB_PATH=SENTINEL)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "tests", "lds_sentinel_cases.py")], env=env,
                       capture_output=True, text=True, timeout=400)
    print(r.stdout[-6000:], flush=True)
    print(r.stderr[-3000:], flush=True)
    assert r.returncode == 0, "a case failed on the LDS sentinel build"
    assert "all cases passed on " + SENTINEL in r.stdout
