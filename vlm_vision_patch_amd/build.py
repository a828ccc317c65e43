"""Build libpe.so (the gfx950 PatchEmbed library) in-tree with hipcc.

The forward kernels are split over translation units (one per patch size and input dtype) that
compile in parallel; the objects are then linked into one shared library.

build(sentinel=True) builds the same sources with -DPE_LDS_SENTINEL=1 into libpe_sentinel.so, a
debug library whose kernels fill their LDS with NaN before use (csrc/pe_device.h); the tests run
parity cases on it to catch LDS reads that come before their writes.
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
LIB_SENTINEL = os.path.join(PKG, "libpe_sentinel.so")
OBJDIR = os.path.join(PKG, "_build")
SOURCES = sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "pe_api.cpp"), os.path.join(CSRC, "pe_plan.cpp")]
HEADERS = sorted(glob.glob(os.path.join(CSRC, "*.h"))) + [os.path.join(ROOT, "include", "pe.h")]
ARCH = "gfx950"
FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wall"]


def compile_cmd(src: str, obj: str, extra=()):
    return ["/opt/rocm/bin/hipcc", *FLAGS, "-I", os.path.join(ROOT, "include"), "-I", CSRC,
            *extra, "-c", src, "-o", obj]


def link_cmd(objs, out: str):
    return ["/opt/rocm/bin/hipcc", "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", out]


def stale(lib: str = LIB) -> bool:
    if not os.path.exists(lib):
        return True
    t = os.path.getmtime(lib)
    return any(os.path.getmtime(p) > t for p in SOURCES + HEADERS + [__file__])


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature and says so; that is harmless
    msgs = [l for l in (res.stdout + res.stderr).splitlines() if "packed-fp32-ops" not in l]
    return res.returncode, msgs


def _jobs(sentinel: bool):
    lib = LIB_SENTINEL if sentinel else LIB
    tag = ("s%d" if sentinel else "%d") % os.getpid()
    objs = [os.path.join(OBJDIR, os.path.basename(s) + "." + tag + ".o") for s in SOURCES]
    extra = ["-DPE_LDS_SENTINEL=1"] if sentinel else []
    return lib, tag, objs, [compile_cmd(s, o, extra) for s, o in zip(SOURCES, objs)]


def _build_many(variants, verbose: bool, jobs: int):
    """Compile the objects of every (lib, tag, objs, cmds) in one pool (the largest translation
    units first, so the long ones overlap), then link each library."""
    os.makedirs(OBJDIR, exist_ok=True)
    cmds = [c for v in variants for c in v[3]]
    order = sorted(range(len(cmds)), key=lambda i: -os.path.getsize(cmds[i][cmds[i].index("-c") + 1]))
    jobs = jobs or min(len(cmds), max(1, (os.cpu_count() or 1)), 8)
    try:
        with ThreadPoolExecutor(jobs) as ex:
            done = dict(zip(order, ex.map(_run, [cmds[i] for i in order])))
        for i, cmd in enumerate(cmds):
            rc, msgs = done[i]
            if verbose:
                print(" ".join(cmd), flush=True)
            if rc != 0:
                raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
            if verbose and msgs:
                print("\n".join(msgs), flush=True)
        for lib, tag, objs, _ in variants:
            tmp = lib + ".tmp" + tag
            rc, msgs = _run(link_cmd(objs, tmp))
            if rc != 0:
                raise RuntimeError("hipcc link failed:\n" + "\n".join(msgs))
            os.replace(tmp, lib)
    finally:
        for v in variants:
            for o in v[2]:
                if os.path.exists(o):
                    os.remove(o)


def build(force: bool = True, verbose: bool = False, jobs: int = 0, sentinel: bool = False) -> str:
    """libpe.so (or, with sentinel, libpe_sentinel.so)."""
    v = _jobs(sentinel)
    if force or stale(v[0]):
        _build_many([v], verbose, jobs)
    return v[0]


def build_all(force: bool = True, verbose: bool = False, jobs: int = 0):
    """libpe.so and libpe_sentinel.so, compiled in one pool."""
    vs = [v for v in (_jobs(False), _jobs(True)) if force or stale(v[0])]
    if vs:
        _build_many(vs, verbose, jobs)
    return LIB, LIB_SENTINEL


if __name__ == "__main__":
    if "--sentinel" in sys.argv[1:]:
        print("\n".join(build_all(force=True, verbose=True)))
    else:
        print(build(force=True, verbose=True))
    sys.exit(0)
