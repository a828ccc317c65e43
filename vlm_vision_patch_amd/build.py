"""Build libpe.so (the gfx950 PatchEmbed library) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpe.so")
SOURCES = [os.path.join(CSRC, "pe_kernels.hip"), os.path.join(CSRC, "pe_api.cpp")]
HEADERS = [os.path.join(CSRC, "pe_internal.h"), os.path.join(ROOT, "include", "pe.h")]
ARCH = "gfx950"


def hipcc_cmd(out: str, extra=()):
    return ["/opt/rocm/bin/hipcc", "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            *extra, *SOURCES, "-o", out]


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS + [__file__])


def build(force: bool = True, verbose: bool = False) -> str:
    if not force and not stale():
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = hipcc_cmd(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that is harmless
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), flush=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(force=True, verbose=True)
    print(LIB)
    sys.exit(0)
