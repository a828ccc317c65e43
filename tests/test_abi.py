"""C-ABI and host-logic tests that need no GPU: the library loads and exports every symbol that
include/pe.h declares; argument validation returns the documented codes without touching a
device; the fragment map is a bijection onto the patch elements."""
import ctypes
import os
import re
import subprocess

import pytest

from conftest import ROOT

pe = pytest.importorskip("vlm_vision_patch_amd", reason="libpe.so not built")

HEADER = os.path.join(ROOT, "include", "pe.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(pe_\w+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_symbol():
    names = header_functions()
    assert set(names) == set(pe.EXPORTS), names
    lib = ctypes.CDLL(pe.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n


def test_library_is_gfx950_code_object():
    data = open(pe.LIB_PATH, "rb").read()
    assert b"gfx950" in data


def test_config_struct_matches_header():
    """The binding's pe_config has the header's fields, in order, all int32."""
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct \{(.*?)\} pe_config;", src, flags=re.S).group(1)
    fields = re.findall(r"int32_t\s+(\w+)\s*;", body)
    assert fields == [f for f, _ in pe.pe_config._fields_]
    assert all(t is ctypes.c_int32 for _, t in pe.pe_config._fields_)
    assert ctypes.sizeof(pe.pe_config) == 4 * len(fields)


def test_num_rows_matches_page_shapes():
    assert pe.pe_num_rows([[1, 36, 54]]) == 1944          # mytransformer shape table
    assert pe.pe_num_rows([[1, 16, 64]]) == 1024          # Qwen2.5VL language-model page
    assert pe.pe_num_rows([[1, 72, 72]] * 64) == 331776
    assert pe.pe_num_rows([]) == 0
    with pytest.raises(pe.PEError) as ei:
        pe.pe_num_rows([[1, 0, 4]])
    assert ei.value.code == pe.PE_ERR_SHAPE
    assert "non-positive" in pe.last_error()


def test_num_rows_large_and_overflowing_grids():
    big = 2 ** 31 - 1
    assert pe.pe_num_rows([[big, big, 1]]) == big * big               # 4.6e18 still fits int64
    assert pe.pe_num_rows([[big, 1, 1]] * 3) == 3 * big
    assert pe.pe_num_rows([[big, big, 2]]) == 2 * big * big          # just below 2^63
    for grid in ([[big, big, big]], [[big, big, 3]], [[big, big, 1]] * 3):
        with pytest.raises(pe.PEError) as ei:
            pe.pe_num_rows(grid)
        assert ei.value.code == pe.PE_ERR_SHAPE
        assert "overflows" in pe.last_error()


def _cfg(**kw):
    c = dict(in_channels=3, temporal_patch_size=2, patch_size=14, embed_dim=1280, spatial_merge_size=2,
             weight_dtype=pe.PE_BF16, out_dtype=pe.PE_BF16, out_order=pe.PE_ORDER_MERGE_WINDOW)
    c.update(kw)
    return pe.pe_config(**c)


@pytest.mark.parametrize("kw,code", [
    (dict(in_channels=4), pe.PE_ERR_UNSUPPORTED),
    (dict(temporal_patch_size=1), pe.PE_ERR_UNSUPPORTED),
    (dict(patch_size=15), pe.PE_ERR_UNSUPPORTED),
    (dict(embed_dim=1000), pe.PE_ERR_UNSUPPORTED),
    (dict(embed_dim=0), pe.PE_ERR_UNSUPPORTED),
    (dict(weight_dtype=7), pe.PE_ERR_INVALID_ARG),
    (dict(out_dtype=-1), pe.PE_ERR_INVALID_ARG),
    (dict(out_order=5), pe.PE_ERR_INVALID_ARG),
    (dict(spatial_merge_size=0), pe.PE_ERR_INVALID_ARG),
    (dict(image_fold=2), pe.PE_ERR_INVALID_ARG),
    (dict(image_fold=1, weight_dtype=pe.PE_F32, out_dtype=pe.PE_F32), pe.PE_ERR_UNSUPPORTED),
])
def test_create_rejects_bad_config_before_touching_device(kw, code):
    h = ctypes.c_void_p(123)
    # the weight pointer is never dereferenced: validation fails first
    rc = pe.lib.pe_create(ctypes.byref(_cfg(**kw)), 0x1000, None, None, ctypes.byref(h))
    assert rc == code
    assert h.value is None
    assert pe.last_error()


def test_null_arguments():
    h = ctypes.c_void_p()
    assert pe.lib.pe_create(None, 0x1000, None, None, ctypes.byref(h)) == pe.PE_ERR_INVALID_ARG
    assert pe.lib.pe_create(ctypes.byref(_cfg()), None, None, None, ctypes.byref(h)) == pe.PE_ERR_INVALID_ARG
    assert pe.lib.pe_create(ctypes.byref(_cfg()), 0x1000, None, None, None) == pe.PE_ERR_INVALID_ARG
    g = (ctypes.c_int32 * 3)(1, 2, 2)
    assert pe.lib.pe_forward(None, 1, 0x1000, 1, g, None, 1, 0x2000, None) == pe.PE_ERR_INVALID_ARG
    assert pe.lib.pe_destroy(None) == pe.PE_OK
    assert pe.lib.pe_num_rows(None, 1) == pe.PE_ERR_INVALID_ARG
    assert pe.lib.pe_num_rows(g, -1) == pe.PE_ERR_INVALID_ARG


def test_fragment_map_is_a_bijection(tmp_path):
    exe = str(tmp_path / "frag_map_check")
    subprocess.check_call(["/opt/rocm/bin/hipcc", "-O1", "-std=c++17",
                           "-I", os.path.join(ROOT, "include"),
                           "-I", os.path.join(ROOT, "vlm_vision_patch_amd", "csrc"),
                           os.path.join(ROOT, "tests", "frag_map_check.cpp"), "-o", exe],
                          stderr=subprocess.DEVNULL)
    out = subprocess.run([exe], capture_output=True, text=True)
    print(out.stdout)
    assert out.returncode == 0 and out.stdout.strip().endswith("OK"), out.stdout
