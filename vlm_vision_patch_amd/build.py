"""Build libpe.so (the gfx950 PatchEmbed library) in-tree with hipcc.

The forward kernels are split over translation units (one per patch size and input dtype) that
compile in parallel; the objects are then linked into one shared library.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libpe.so")
OBJDIR = os.path.join(PKG, "_build")
SOURCES = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "pe_api.cpp")]
HEADERS = sorted(glob.glob(os.path.join(CSRC, "*.h"))) + [os.path.join(ROOT, "include", "pe.h")]
ARCH = "gfx950"
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall"]


def compile_cmd(src: str, obj: str, extra=()):
    return ["/opt/rocm/bin/hipcc", *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            *extra, "-c", src, "-o", obj]


def link_cmd(objs, out: str):
    return ["/opt/rocm/bin/hipcc", "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", out]


def stale() -> bool:
    if not os.path.exists(LIB):
        return True
    t = os.path.getmtime(LIB)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS + [__file__])


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that is harmless
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l]
    return res.returncode, msgs


def build(force: bool = True, verbose: bool = False, jobs: int = 0) -> str:
    if not force and not stale():
        return LIB
    os.makedirs(OBJDIR, exist_ok=True)
    tag = "%d" % os.getpid()
    objs = [os.path.join(OBJDIR, os.path.basename(s) + "." + tag + ".o") for s in SOURCES]
    cmds = [compile_cmd(s, o) for s, o in zip(SOURCES, objs)]
    jobs = jobs or min(len(cmds), max(1, (os.cpu_count() or 1)), 8)
    try:
        with ThreadPoolExecutor(jobs) as ex:
            results = list(ex.map(_run, cmds))
        for cmd, (rc, msgs) in zip(cmds, results):
            if verbose:
                print(" ".join(cmd), flush=True)
            if rc != 0:
                raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
            if verbose and msgs:
                print("\n".join(msgs), flush=True)
        tmp = LIB + ".tmp" + tag
        rc, msgs = _run(link_cmd(objs, tmp))
        if rc != 0:
            raise RuntimeError("hipcc link failed:\n" + "\n".join(msgs))
        os.replace(tmp, LIB)
    finally:
        for o in objs:
            if os.path.exists(o):
                os.remove(o)
    return LIB


if __name__ == "__main__":
    build(force=True, verbose=True)
    print(LIB)
    sys.exit(0)
