"""A plain C caller of the library (tests/c_client/pe_client.c: include/pe.h and the HIP runtime
only, built with gcc as C11): the header compiles as C and the client links against libpe.so
(CPU), and on the GPU its PatchEmbed and merger LayerNorm outputs match the oracle."""
import math
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
import workloads
from conftest import ROOT

PKG = os.path.join(ROOT, "vlm_vision_patch_amd")
SRC = os.path.join(ROOT, "tests", "c_client", "pe_client.c")


def build_client(out_dir):
    exe = os.path.join(str(out_dir), "pe_client")
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-Wall", "-Werror", "-D__HIP_PLATFORM_AMD__",
                           "-I/opt/rocm/include", "-I", os.path.join(ROOT, "include"), SRC, "-o", exe,
                           "-L/opt/rocm/lib", "-lamdhip64", "-L", PKG, "-lpe",
                           "-Wl,-rpath,/opt/rocm/lib", "-Wl,-rpath," + PKG])
    return exe


def test_header_is_c_and_client_links(tmp_path):
    if not os.path.exists(os.path.join(PKG, "libpe.so")):
        pytest.skip("libpe.so not built")
    exe = build_client(tmp_path)
    out = subprocess.run(["nm", "-u", exe], capture_output=True, text=True).stdout
    for sym in ("pe_create", "pe_forward", "pe_layernorm", "pe_num_rows", "pe_destroy", "pe_last_error"):
        assert sym in out, sym


def bf16_bytes(t):
    return t.to(torch.bfloat16).contiguous().view(torch.int16).numpy().tobytes()


def from_bf16_bytes(b, shape):
    a = np.frombuffer(b, dtype=np.int16).copy()
    return torch.from_numpy(a).view(torch.bfloat16).reshape(shape).double().numpy()


@pytest.mark.gpu
def test_c_client_matches_oracle(tmp_path):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("[case] C client: one 8 x 12 image, P14, E256, bias, merge order, then LayerNorm", flush=True)
    P, E, t, h, w, F = 14, 256, 1, 8, 12, 1
    K = 3 * 2 * P * P
    x = workloads.random_tensor((F, 3, h * P, w * P), seed=6000, dtype=torch.bfloat16)
    wt = workloads.random_tensor((E, 3, 2, P, P), seed=6001, dtype=torch.bfloat16, dist="uniform", bound=1 / math.sqrt(K))
    b = workloads.random_tensor((E,), seed=6002, dtype=torch.bfloat16, dist="uniform", bound=1 / math.sqrt(K))
    gam = (1 + 0.1 * workloads.random_tensor((E,), seed=6003)).to(torch.bfloat16)
    bet = (0.1 * workloads.random_tensor((E,), seed=6004)).to(torch.bfloat16)
    d = str(tmp_path)
    for name, tens in (("frames.bin", x), ("weight.bin", wt), ("bias.bin", b), ("gamma.bin", gam), ("beta.bin", bet)):
        open(os.path.join(d, name), "wb").write(bf16_bytes(tens))
    open(os.path.join(d, "meta.txt"), "w").write("%d %d %d %d %d %d\n" % (P, E, t, h, w, F))
    exe = build_client(tmp_path)
    r = subprocess.run([exe, d], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0
    n = t * h * w
    got = from_bf16_bytes(open(os.path.join(d, "out.bin"), "rb").read(), (n, E))
    ref = oracle.forward(x, wt, b, grid=[[t, h, w]], frames=[F], order="merge", m=2)
    assert np.all(np.abs(got - ref) <= 1e-3 + 1e-2 * np.abs(ref))
    # LayerNorm of the client's bf16 rows: the oracle's rows rounded to bf16 may differ from the
    # library's in one ulp where the fp64 and fp32 sums straddle a midpoint; that moves the
    # normalized value by at most |gamma| * rstd * ulp
    pe_ref = oracle.round_via_f32(ref, "bf16")
    ln_ref = oracle.layer_norm(pe_ref, gam, bet, 1e-6)
    ln_got = from_bf16_bytes(open(os.path.join(d, "ln.bin"), "rb").read(), (n, E))
    mean = pe_ref.mean(axis=1, keepdims=True)
    rstd = 1.0 / np.sqrt(((pe_ref - mean) ** 2).mean(axis=1, keepdims=True) + 1e-6)
    ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(pe_ref), 1e-30))) - 7)
    tol = 1e-3 + 1e-2 * np.abs(ln_ref) + np.abs(oracle._f64(gam)) * rstd * ulp
    assert np.all(np.abs(ln_got - ln_ref) <= tol)


@pytest.mark.gpu
@pytest.mark.parametrize("n,in_dtype", [(256, torch.bfloat16), (8192, torch.bfloat16), (1024, torch.float32)])
def test_c_client_patch_rows_exact_buffer(tmp_path, n, in_dtype):
    """Patch rows in a device buffer of exactly N*K elements (N chosen so that it ends on a 4 KiB
    boundary): the loads of the last row's final fragment stay inside the row (the split-k kernel
    at N = 256, the large-tile kernel that stages rows through LDS at N = 8192; fp32 rows rounded on
    load), and the output matches the oracle."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print("[case] C client patch rows: N=%d %s, P14, E1280, bias, exact-size buffer" % (n, in_dtype), flush=True)
    P, E = 14, 1280
    K = 3 * 2 * P * P
    isz = 2 if in_dtype == torch.bfloat16 else 4
    assert (n * K * isz) % 4096 == 0
    x = workloads.random_tensor((n, K), seed=6100 + n, dtype=in_dtype)
    wt = workloads.random_tensor((E, 3, 2, P, P), seed=6101, dtype=torch.bfloat16, dist="uniform", bound=1 / math.sqrt(K))
    b = workloads.random_tensor((E,), seed=6102, dtype=torch.bfloat16, dist="uniform", bound=1 / math.sqrt(K))
    d = str(tmp_path)
    raw = bf16_bytes(x) if in_dtype == torch.bfloat16 else x.contiguous().numpy().tobytes()
    open(os.path.join(d, "rows.bin"), "wb").write(raw)
    open(os.path.join(d, "weight.bin"), "wb").write(bf16_bytes(wt))
    open(os.path.join(d, "bias.bin"), "wb").write(bf16_bytes(b))
    open(os.path.join(d, "rows_meta.txt"), "w").write("%d %d %d %d\n" % (P, E, n, 1 if in_dtype == torch.bfloat16 else 0))
    exe = build_client(tmp_path)
    r = subprocess.run([exe, d, "rows"], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr, flush=True)
    assert r.returncode == 0
    got = from_bf16_bytes(open(os.path.join(d, "rows_out.bin"), "rb").read(), (n, E))
    ref = oracle.forward(x, wt, b, grid=[[1, 1, n]], kind="patches", cast_input_to="bf16")
    assert np.all(np.abs(got - ref) <= 1e-3 + 1e-2 * np.abs(ref))
