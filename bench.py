"""Benchmark of the gfx950 vision PatchEmbed: one JSON line on stdout.

A step is one PatchEmbed forward (gather + matrix product + epilogue, one kernel launch per
<= 64 items) over one batch of synthetic input already resident in HBM. The timed region is
K steps captured back to back in a HIP graph and replayed once, bracketed by HIP events on the
stream they run on; `eager_ms_per_step` gives the same K steps launched one by one from Python.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 5] [--extra 2,3]
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import struct
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "PatchEmbed patches/s + TFLOP/s (% bf16 MFMA peak) on 1 MI355X"
PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 2.4 GHz x 4096 dense bf16 flop/clk/CU
PEAK_F32_MATRIX_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
LIBPE = os.path.join(ROOT, "vlm_vision_patch_amd", "libpe.so")


def elf_sections(b):
    """Section headers of a little-endian ELF64 image: ({name: header}, [headers]); a header is
    (name, type, flags, addr, offset, size, link, info, align, entsize)."""
    if b[:4] != b"\x7fELF" or b[4] != 2 or b[5] != 1:
        raise ValueError("not a little-endian ELF64 image")
    shoff, = struct.unpack_from("<Q", b, 0x28)
    shentsize, shnum, shstrndx = struct.unpack_from("<HHH", b, 0x3A)
    secs = [struct.unpack_from("<IIQQQQIIQQ", b, shoff + i * shentsize) for i in range(shnum)]
    so = secs[shstrndx][4]
    return {b[so + s[0]: b.index(b"\0", so + s[0])].decode(): s for s in secs}, secs


def gfx950_code_objects(b):
    """(offset in b, image) of each gfx950 code object of HIP shared library image b: the clang
    offload bundles (one per translation unit) in its .hip_fatbin section, uncompressed."""
    named, _ = elf_sections(b)
    if ".hip_fatbin" not in named:
        raise ValueError("no .hip_fatbin section")
    base, size = named[".hip_fatbin"][4], named[".hip_fatbin"][5]
    fat = b[base: base + size]
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    i = fat.find(magic)
    while i >= 0:
        n, = struct.unpack_from("<Q", fat, i + len(magic))
        p = i + len(magic) + 8
        for _ in range(n):
            off, size, tl = struct.unpack_from("<QQQ", fat, p)
            triple = fat[p + 24: p + 24 + tl].decode()
            p += 24 + tl
            if triple.endswith("gfx950") and size:
                yield base + i + off, fat[i + off: i + off + size]
        i = fat.find(magic, i + len(magic))


def kernel_symbols(b, kernel):
    """(name, offset in b, size) of every symbol of template pe::`kernel` in the gfx950 code of
    library image b: each instantiation's entry (machine code) and its descriptor (`.kd`:
    registers, LDS, launch bounds)."""
    prefix = "_ZN2pe%d%s" % (len(kernel), kernel)
    for base, co in gfx950_code_objects(b):
        named, secs = elf_sections(co)
        st, sn = named[".symtab"], named[".strtab"]
        for k in range(st[5] // 24):
            nmo, _info, _other, shndx, val, size = struct.unpack_from("<IBBHQQ", co, st[4] + 24 * k)
            if size == 0 or shndx == 0 or shndx >= len(secs):
                continue
            name = co[sn[4] + nmo: co.index(b"\0", sn[4] + nmo)].decode()
            if name.startswith(prefix):
                sec = secs[shndx]
                yield name, base + sec[4] + val - sec[3], size


def kernel_code_hash(kernel: str, lib: str = LIBPE) -> str:
    """Hash of the machine code of every instantiation of pe::`kernel` in the built library (each
    symbol's name and bytes, in name order). It keys HBM-traffic counters to the code they were
    taken on: a change to that kernel's code changes it; a comment or another kernel does not.
    A descriptor's entry offset (bytes 16-23 of the 64-byte `.kd`: the distance from the
    descriptor to the code) is left out, since it moves when another kernel of the same code object
    changes size."""
    b = open(lib, "rb").read()
    syms = sorted(kernel_symbols(b, kernel))
    if not syms:
        raise ValueError("no code for kernel %s in %s" % (kernel, lib))
    h = hashlib.sha256()
    for name, off, size in syms:
        body = b[off: off + size]
        if name.endswith(".kd") and size == 64:
            body = body[:16] + bytes(8) + body[24:]
        h.update(name.encode() + b"\0" + body)
    return h.hexdigest()[:16]


def algorithmic(wl, rows=False, add=False):
    """FLOPs and algorithmic HBM bytes of one step: unique input read once (one frame per image,
    every frame of a video; patch rows as given), packed weight, bias, output. rows: the same
    patches given as pre-flattened rows [N, K]."""
    import workloads
    esz = {"bf16": 2, "f32": 4}
    n = sum(t * h * w for (t, h, w) in wl.grid)
    flops = 2.0 * n * wl.k * wl.embed
    inp = 1
    for d in (wl.input_shape if not rows else (n, wl.k)):
        inp *= d
    byts = inp * esz[wl.in_dtype] + wl.embed * wl.k * esz[wl.w_dtype] + \
        (wl.embed * esz[wl.w_dtype] if wl.bias else 0) + n * wl.embed * esz[wl.out_dtype] * (2 if add else 1)
    return n, flops, byts


def time_workload(idx, steps, warmup, graph=True, rows=False, items=None, reps=10, cold=False, add=False,
                  fold=False, keep_out=False, stage=False):
    """rows: feed the workload's patches as pre-flattened rows [N, K] (the processor's
    pixel_values layout) instead of its frames: same N, weight and bias, synthetic N(0, 1) rows.
    items: keep only the first `items` items (one GPU's share of an item split).
    The graph of K steps is replayed `reps` times, each replay timed: median, p10 and p90 per step.
    cold: also time single launches after overwriting a 1 GiB buffer (L2 and the 256 MB
    Infinity Cache hold nothing of the inputs), median of `reps`.
    add: fuse the add of a synthetic [N, E] tensor (position embeddings) into the epilogue.
    fold: the approximate image-fold mode (single-frame items on W[:, :, 0] + W[:, :, 1] in bf16).
    stage: the opt-in LDS-staged gather of single images (stage_images).
    keep_out: also return the output of the last timed step (and the inputs and the addend, on the
    host), for the parity check of the timed output.
    The result holds the library's launch plan of one step (pe_forward_plan): which kernel runs,
    its tile and grid."""
    import torch
    import workloads
    import vlm_vision_patch_amd as pe

    wl = workloads.WORKLOADS[idx]
    dev = torch.device("cuda:0")
    x, w, b = workloads.generate(wl)
    if items is not None:
        wl = workloads.share(wl, items)
        x = x.reshape(-1)[:workloads.input_elements(wl)]
    n, flops, byts = algorithmic(wl, rows, add)
    kind = wl.kind
    grid, frames = [list(g) for g in wl.grid], list(wl.frames) or None
    if rows:
        x = workloads.random_tensor((n, wl.k), seed=1000 + idx, dtype=workloads.DTYPES[wl.in_dtype])
        kind, grid, frames = "patches", [[1, 1, n]], None
    host_in = (x, w, b, None) if keep_out else None
    x, w = x.to(dev), w.to(dev)
    b = b.to(dev) if b is not None else None
    mod = pe.PatchEmbed(w, b, order=wl.order, out_dtype=workloads.DTYPES[wl.out_dtype], image_fold=fold,
                        stage_images=stage)
    plan = mod.plan(grid, frames, kind=kind, in_dtype=x.dtype)
    out = torch.empty((n, wl.embed), dtype=workloads.DTYPES[wl.out_dtype], device=dev)
    addend = None
    if add:
        addend_host = (workloads.random_tensor((n, wl.embed), seed=3000 + idx) * 0.02).to(
            workloads.DTYPES[wl.out_dtype])
        addend = addend_host.to(dev)
        if keep_out:
            host_in = host_in[:3] + (addend_host,)
    s = torch.cuda.Stream(device=dev)   # default priority
    with torch.cuda.stream(s):
        for _ in range(warmup):
            mod(x, grid, frames, kind=kind, out=out, add=addend)
        # eager: K launches from Python
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(s)
        for _ in range(steps):
            mod(x, grid, frames, kind=kind, out=out, add=addend)
        e1.record(s)
        torch.cuda.synchronize()
        eager_ms = e0.elapsed_time(e1) / steps
    ms = eager_ms
    timing = "K eager launches between HIP events"
    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for _ in range(steps):
                mod(x, grid, frames, kind=kind, out=out, add=addend)
        per = []
        with torch.cuda.stream(s):
            g.replay()                       # untimed: first replay uploads the graph
            torch.cuda.synchronize()
            for _ in range(max(1, reps)):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(s)
                g.replay()
                e1.record(s)
                torch.cuda.synchronize()
                per.append(e0.elapsed_time(e1) / steps)
        per.sort()
        ms = per[len(per) // 2]
        stats = {"median_ms": round(ms, 6), "p10_ms": round(per[len(per) // 10], 6),
                 "p90_ms": round(per[min(len(per) - 1, (9 * len(per)) // 10)], 6), "replays": len(per)}
        timing = "K steps captured in one HIP graph; median over %d replays, each between HIP events" % len(per)
        del g
    else:
        stats = None
    cold_ms = None
    if cold:
        flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)   # 1 GiB
        cs = []
        with torch.cuda.stream(s):
            for i in range(max(1, reps)):
                flush.fill_(float(i))
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(s)
                mod(x, grid, frames, kind=kind, out=out, add=addend)
                e1.record(s)
                torch.cuda.synchronize()
                cs.append(e0.elapsed_time(e1))
        cs.sort()
        cold_ms = cs[len(cs) // 2]
        del flush
    mod.close()
    return dict(wl=wl, n=n, flops=flops, bytes=byts, ms=ms, eager_ms=eager_ms, timing=timing, rows=rows,
                stats=stats, cold_ms=cold_ms, plan=plan, out=out if keep_out else None, host_in=host_in,
                kind=kind, grid=grid, frames=frames)


def layernorm_alg_bytes(wl):
    """Algorithmic HBM bytes of one LayerNorm over the workload's [N, E] output rows: the rows read
    once and written once, gamma and beta, all in the output dtype."""
    esz = {"bf16": 2, "f32": 4}[wl.out_dtype]
    n = sum(t * h * w for (t, h, w) in wl.grid)
    return 2 * n * wl.embed * esz + 2 * wl.embed * esz


def time_merger_front(idx, steps, warmup=3, reps=5, eps=1e-6, eager=False):
    """The PatchMerger front end on the workload's output rows: pe_layernorm over [N, E] in the
    output dtype (synthetic rows and parameters), alone and after the PatchEmbed as one step
    (PatchEmbed, then the LayerNorm in place). Graph of K steps, median of `reps` replays (eager:
    K launches from Python between events, for counter runs)."""
    import torch
    import workloads
    import vlm_vision_patch_amd as pe

    wl = workloads.WORKLOADS[idx]
    dev = torch.device("cuda:0")
    odt = workloads.DTYPES[wl.out_dtype]
    n = sum(t * h * w for (t, h, w) in wl.grid)
    E = wl.embed
    rows = (workloads.random_tensor((n, E), seed=4000 + idx) * 0.6).to(odt).to(dev)
    y = torch.empty_like(rows)
    gam = (1.0 + 0.1 * workloads.random_tensor((E,), seed=4100 + idx)).to(odt).to(dev)
    bet = (0.1 * workloads.random_tensor((E,), seed=4200 + idx)).to(odt).to(dev)
    x, w, b = workloads.generate(wl)
    x, w = x.to(dev), w.to(dev)
    b = b.to(dev) if b is not None else None
    mod = pe.PatchEmbed(w, b, order=wl.order, out_dtype=odt)
    grid, frames = [list(g) for g in wl.grid], list(wl.frames) or None
    out = torch.empty((n, E), dtype=odt, device=dev)
    s = torch.cuda.Stream(device=dev)

    def ln_only():
        pe.layer_norm(rows, gam, bet, eps, out=y, stream=s.cuda_stream)

    def pipeline():
        mod(x, grid, frames, out=out, stream=s.cuda_stream)
        pe.layer_norm(out, gam, bet, eps, out=out, stream=s.cuda_stream)

    res = {}
    for name, fn in (("layernorm", ln_only), ("patch_embed_then_layernorm", pipeline)):
        if eager:
            with torch.cuda.stream(s):
                for _ in range(warmup):
                    fn()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda.synchronize()
                e0.record(s)
                for _ in range(steps):
                    fn()
                e1.record(s)
                torch.cuda.synchronize()
            res[name] = e0.elapsed_time(e1) / steps
            continue
        with torch.cuda.stream(s):
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=s):
                for _ in range(steps):
                    fn()
            g.replay()
            torch.cuda.synchronize()
            per = []
            for _ in range(reps):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(s)
                g.replay()
                e1.record(s)
                torch.cuda.synchronize()
                per.append(e0.elapsed_time(e1) / steps)
            del g
        per.sort()
        res[name] = per[len(per) // 2]
    mod.close()
    ln_bytes = layernorm_alg_bytes(wl)
    ln_ms = res["layernorm"]
    return {"what": "LayerNorm over E of the [N, E] %s rows (the PatchMerger front end; in merge-window "
                    "order the 2x2 concatenation is a view)" % wl.out_dtype,
            "n_rows": n, "embed": E, "ms_per_step": round(ln_ms, 5),
            "alg_bytes": ln_bytes, "gbs": round(ln_bytes / (ln_ms / 1e3) / 1e9, 1),
            "frac_hbm": round(ln_bytes / (ln_ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
            "patch_embed_then_layernorm_ms": round(res["patch_embed_then_layernorm"], 5),
            "patch_embed_then_layernorm_patches_per_s": round(n / (res["patch_embed_then_layernorm"] / 1e3), 1),
            "traffic": load_traffic("pe_layernorm_kernel", wl.name + "_layernorm"),
            "timing": "K eager launches between HIP events" if eager else "graph of K steps, median of replays",
            "steps": steps}


def time_linear(a, w2, b2, steps):
    """Milliseconds per torch.nn.functional.linear(a, w2, b2) (hipBLASLt), K eager calls between
    events after three untimed ones."""
    import torch
    for _ in range(3):
        y = torch.nn.functional.linear(a, w2, b2)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        y = torch.nn.functional.linear(a, w2, b2)
    e1.record()
    torch.cuda.synchronize()
    del y
    return e0.elapsed_time(e1) / steps


def time_linear_context(idx, steps=20):
    """hipBLASLt (torch.nn.functional.linear) on the same product with the patches already
    flattened into a contiguous [N, K] matrix: context for the gather-fused kernel, not a target."""
    import torch
    import workloads
    wl = workloads.WORKLOADS[idx]
    dev = torch.device("cuda:0")
    _, w, b = workloads.generate(wl)
    n = sum(t * h * ww for (t, h, ww) in wl.grid)
    dt = workloads.DTYPES[wl.w_dtype]
    a = workloads.random_tensor((n, wl.k), seed=2000 + idx, dtype=dt).to(dev)
    w2 = w.reshape(wl.embed, wl.k).to(dev)
    b2 = b.to(dev) if b is not None else None
    ms = time_linear(a, w2, b2, steps)
    del a
    return {"what": "torch.nn.functional.linear (hipBLASLt) on a contiguous [N, K] patch matrix, same "
                    "N, K, E, dtype and bias; the patchify gather not included", "ms_per_step": round(ms, 5),
            "tflops": round(2.0 * n * wl.k * wl.embed / (ms / 1e3) / 1e12, 2), "steps": steps}


def time_square_context(m=8192, steps=20):
    """hipBLASLt on an m x m x m bf16 product: what the vendor library reaches on a large square
    product on this chip, a practical ceiling for bf16 matrix-core work next to the nominal peak."""
    import torch
    import workloads
    dev = torch.device("cuda:0")
    a = workloads.random_tensor((m, m), seed=3001, dtype=torch.bfloat16).to(dev)
    w2 = workloads.random_tensor((m, m), seed=3002, dtype=torch.bfloat16).to(dev)
    ms = time_linear(a, w2, None, steps)
    del a, w2
    tf = 2.0 * m ** 3 / (ms / 1e3) / 1e12
    return {"what": "torch.nn.functional.linear (hipBLASLt) on a %d x %d x %d bf16 product, no bias" % (m, m, m),
            "ms_per_step": round(ms, 5), "tflops": round(tf, 2), "frac_matrix_peak": round(tf / PEAK_BF16_TFLOPS, 4),
            "steps": steps}


def cpu_info():
    """The host's CPU model and how many cores this process may use: the smallest of the affinity
    mask and the cgroup CPU quota (a container's CPU share), next to what os.cpu_count() says."""
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    nproc = os.cpu_count() or 1
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = nproc
    quota = None
    for path in ("/sys/fs/cgroup/cpu.max",):
        try:
            q, per = open(path).read().split()[:2]
            if q != "max":
                quota = max(1, math.ceil(int(q) / int(per)))
        except (OSError, ValueError):
            pass
    if quota is None:
        try:
            q = int(open("/sys/fs/cgroup/cpu/cpu.cfs_quota_us").read())
            per = int(open("/sys/fs/cgroup/cpu/cpu.cfs_period_us").read())
            if q > 0:
                quota = max(1, math.ceil(q / per))
        except (OSError, ValueError):
            pass
    usable = min(affinity, quota) if quota else affinity
    return {"model": model, "nproc": nproc, "affinity": affinity, "cgroup_quota": quota, "usable": usable}


def sample_rows(n, count, tile=256, seed=0):
    """A deterministic sample of `count` output rows of n (all rows if count >= n): the first and
    last rows, the rows on both sides of `tile`-row boundaries (up to a quarter of the sample), then
    evenly spread rows with a seeded jitter, topped up with seeded random rows where those collide."""
    import random
    if count >= n:
        return list(range(n))
    rng = random.Random(seed)
    picked = {0, n - 1}
    for edge in range(tile, n, tile):
        if len(picked) + 2 > count // 4:
            break
        picked.update((edge - 1, edge))
    left = count - len(picked)
    step = n / max(1, left)
    for i in range(left):
        picked.add(min(n - 1, int(i * step + rng.random() * step)))
    while len(picked) < count:
        picked.add(rng.randrange(n))
    return sorted(picked)


def _tolerance(wl, ref):
    import numpy as np
    if wl.out_dtype == "bf16":
        return 1e-3 + 1e-2 * np.abs(ref), "|err| <= 1e-3 + 1e-2 |ref|"
    return 5e-4, "|err| <= 5e-4"


def cpu_baseline(r, target_seconds=15.0):
    """The oracle, as it stands, timed on this host over a bounded sample of the workload's output
    rows (about `target_seconds` of CPU work, on every core this process may use), and the same rows
    of the timed GPU output compared with it (the parity of what was timed)."""
    import numpy as np
    import oracle
    wl = r["wl"]
    x, w, b, _ = r["host_in"]
    info = cpu_info()
    threads = info["usable"]
    n = r["n"]
    kw = dict(grid=r["grid"], frames=r["frames"], kind=r["kind"], order=wl.order, threads=threads)
    # exact fp64 copies once (the oracle would convert the whole input on every call), then the
    # stratified sample in chunks, in an order that spreads every prefix over the whole workload,
    # until the time bound or the end of the sample
    xd, wd, bd = oracle._f64(x), oracle._f64(w), (oracle._f64(b) if b is not None else None)
    order_rows = sample_rows(n, min(n, 400000), seed=2)
    perm = np.random.default_rng(3).permutation(len(order_rows))
    rows, refs = [], []
    t0 = time.perf_counter()
    chunk = 4 * threads
    done = 0
    while done < len(order_rows):
        part = sorted(order_rows[i] for i in perm[done:done + chunk])
        refs.append(oracle.forward(xd, wd, bd, rows=part, **kw))
        rows += part
        done += len(part)
        el = time.perf_counter() - t0
        if el >= target_seconds:
            break
        chunk = min(8192, chunk * 2)
    el = time.perf_counter() - t0
    ref = np.concatenate(refs)
    import torch
    got = r["out"].index_select(0, torch.tensor(rows, device=r["out"].device)).float().cpu().double().numpy()
    err = np.abs(got - ref)
    tol, tol_text = _tolerance(wl, ref)
    bad = int((err > tol).sum())
    sample = ("%s %d of the %d output rows of %s (drawn from a stratified sample: the first and last rows, both "
              "sides of 256-row tile edges, the rest spread evenly): fp64 direct Conv3d, %d threads, %.1f s" % (
                  "all" if len(rows) == n else "a sample of", len(rows), n, wl.name, threads, el))
    cpu = {"value": round(len(rows) / el, 1), "unit": "patches/s", "cores": threads, "kind": "oracle",
           "sample": sample, "cpu_model": info["model"], "nproc": info["nproc"],
           "cores_note": "cores = min(affinity mask %d, cgroup CPU quota %s) of the %d the host has" % (
               info["affinity"], info["cgroup_quota"], info["nproc"])}
    parity = {"rows_checked": len(rows), "max_abs_err": float(err.max()), "out_of_tolerance": bad,
              "tolerance": tol_text}
    return cpu, parity


def cpu_baseline_config(q, max_rows=8192, approximate=False):
    """Part of the cpu_baseline leg for a secondary line: the oracle timed on all output rows of the
    line's last timed step, or on `max_rows` stratified rows of a larger one, and those rows of the
    timed output compared with it. approximate: the image-fold line, whose sums differ from the
    exact Conv3d by the folded weight's rounding; its error is reported with no tolerance."""
    import numpy as np
    import torch
    import oracle
    wl = q["wl"]
    x, w, b, addend = q["host_in"]
    threads = cpu_info()["usable"]
    n = q["n"]
    rows = sample_rows(n, min(n, max_rows), seed=5)
    t0 = time.perf_counter()
    ref = oracle.forward(x, w, b, grid=q["grid"], frames=q["frames"], kind=q["kind"], order=wl.order,
                         rows=rows, addend=addend, threads=threads)
    el = time.perf_counter() - t0
    got = q["out"].index_select(0, torch.tensor(rows, device=q["out"].device)).float().cpu().double().numpy()
    err = np.abs(got - ref)
    out = {"rows_checked": len(rows), "of_rows": n, "oracle_s": round(el, 3),
           "oracle_patches_per_s": round(len(rows) / el, 1), "cores": threads, "max_abs_err": float(err.max())}
    if approximate:
        out["out_of_tolerance"] = None
        out["tolerance"] = "none: approximate mode, compared with the exact Conv3d"
    else:
        tol, tol_text = _tolerance(wl, ref)
        out["out_of_tolerance"] = int((err > tol).sum())
        out["tolerance"] = tol_text
    return out


def load_traffic(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE counters, if they were
    taken on the kernel's current machine code."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
        rec = d.get(workload)
        if rec and rec.get("code_hash") == kernel_code_hash(kernel):
            return rec["bytes_per_launch"]
    except Exception:
        return None
    return None


def pmc_per_dispatch(csv_dir, counter, kernel):
    """Mean over dispatches of `counter` for kernels whose name contains `kernel`, from the
    counter-collection CSV files rocprofv3 --pmc wrote under csv_dir (a dispatch's value is the sum
    of its rows: one per counter instance), and the dispatch count."""
    import csv
    per = {}
    for path in glob.glob(os.path.join(csv_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(path, newline="") as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter or kernel not in row.get("Kernel_Name", ""):
                    continue
                key = (path, row.get("Dispatch_Id"))
                per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
    if not per:
        raise SystemExit("no %s rows for kernel %s under %s" % (counter, kernel, csv_dir))
    return sum(per.values()) / len(per), len(per)


def summarize_pmc(workload, kernel, fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, cal_bytes, name=None):
    """HBM bytes per launch of `kernel` on `workload` from two rocprofv3 --pmc runs (FETCH_SIZE, then
    WRITE_SIZE, in KiB per dispatch), each scaled by what the same counter read for one plain device
    copy of cal_bytes bytes (bench.py --copy-calibrate), into profiles/traffic.json under the hash of
    the kernel's machine code in the built library."""
    import workloads
    wl = workloads.WORKLOADS[workload]
    if kernel == "pe_layernorm_kernel":  # the LayerNorm over the workload's output rows
        alg, name = layernorm_alg_bytes(wl), name or wl.name + "_layernorm"
    else:
        _, _, alg = algorithmic(wl)
    fk, nf = pmc_per_dispatch(fetch_dir, "FETCH_SIZE", kernel)
    wk, nw = pmc_per_dispatch(write_dir, "WRITE_SIZE", kernel)
    cf, _ = pmc_per_dispatch(cal_fetch_dir, "FETCH_SIZE", "copyBuffer")
    cw, _ = pmc_per_dispatch(cal_write_dir, "WRITE_SIZE", "copyBuffer")
    ff, wf = cal_bytes / (cf * 1024.0), cal_bytes / (cw * 1024.0)
    total = fk * 1024.0 * ff + wk * 1024.0 * wf
    rec = {"code_hash": kernel_code_hash(kernel), "kernel": kernel, "fetch_kib_per_launch": round(fk, 1),
           "write_kib_per_launch": round(wk, 1), "fetch_factor": round(ff, 4), "write_factor": round(wf, 4),
           "bytes_per_launch": int(round(total)), "algorithmic_bytes_per_launch": alg,
           "launches_counted": min(nf, nw)}
    p = os.path.join(ROOT, "profiles", "traffic.json")
    d = json.load(open(p)) if os.path.exists(p) else {}
    d[name or wl.name] = rec
    with open(p, "w") as f:
        json.dump(d, f, indent=1, sort_keys=True)
        f.write("\n")
    return rec


def parse_extra(spec):
    """One --extra entry: (workload, as patch rows, fused add, image fold, items kept or None,
    LDS-staged images). '5r' patch rows, '5a' fused add, '5f' fold, '5s8' the first 8 items, '5l'
    the opt-in LDS-staged gather."""
    as_rows, with_add, fold, stage = spec.endswith("r"), spec.endswith("a"), spec.endswith("f"), spec.endswith("l")
    share = int(spec.split("s")[1]) if "s" in spec else None
    return int(spec.rstrip("rafl").split("s")[0]), as_rows, with_add, fold, share, stage


def workloads_name(idx):
    import workloads
    return workloads.WORKLOADS[idx].name


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=5,
                    help="the headline workload (default 5: 64 images of 1008 x 1008, 331,776 patches, the "
                         "largest configuration and the one the bf16 matrix-core fraction is quoted on)")
    ap.add_argument("--extra", type=str, default="2,5r,5a,5n,5f,5l,2f,5s8,3,4,6,1",
                    help="comma-separated further workloads reported under 'also' ('' for none); "
                         "a trailing r feeds that workload's patches as pre-flattened rows, a trailing "
                         "a fuses the add of an [N, E] tensor, a trailing n times the PatchMerger "
                         "LayerNorm on its output rows, a trailing f runs the approximate image-fold "
                         "mode; sN keeps its first N items (one GPU's share of an N-way item split)")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the library-GEMM context line (hipBLASLt on the same product)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--eager", action="store_true",
                    help="time K launches from Python instead of a captured graph (for counter runs)")
    ap.add_argument("--copy-calibrate", type=int, default=0, metavar="BYTES",
                    help="only run one plain device-to-device copy of BYTES (counter calibration)")
    ap.add_argument("--summarize-pmc", nargs=7, metavar=("WORKLOAD", "KERNEL", "FETCH_DIR", "WRITE_DIR",
                                                          "CAL_FETCH_DIR", "CAL_WRITE_DIR", "CAL_BYTES"),
                    help="no GPU work: write the HBM bytes per launch of KERNEL on WORKLOAD from rocprofv3 "
                         "--pmc FETCH_SIZE / WRITE_SIZE output directories, calibrated by a copy's counters, "
                         "into profiles/traffic.json")
    args = ap.parse_args()
    if args.summarize_pmc:
        w_, k_, fd, wd, cfd, cwd, cb = args.summarize_pmc
        print(json.dumps(summarize_pmc(int(w_), k_, fd, wd, cfd, cwd, int(cb))), flush=True)
        return
    if args.gpus != 1:
        print("bench.py times one GPU only; --gpus %d is not supported (PatchEmbed rows are independent: "
              "across GPUs the items are dealt out, one handle per device, with no exchange)" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibrate:
        n = args.copy_calibrate // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n * 4}), flush=True)
        return

    cpu_leg = not args.no_cpu and not args.eager
    r = time_workload(args.workload, args.steps, args.warmup, graph=not args.eager, cold=not args.eager,
                      keep_out=cpu_leg)
    wl = r["wl"]
    t_s = r["ms"] / 1e3
    tflops = r["flops"] / t_s / 1e12
    gbs = r["bytes"] / t_s / 1e9
    bf16 = wl.w_dtype == "bf16"
    peak_fl = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_MATRIX_TFLOPS
    ai = r["flops"] / r["bytes"]
    ridge = peak_fl * 1e12 / (PEAK_HBM_GBS * 1e9)
    bound = "mfma" if ai >= ridge else "hbm"
    # the kernel that does the step's work, as the library planned it (pe_forward_plan): the launch
    # with the most output rows; the step's HIP-event time covers all of its launches
    plan = r["plan"]
    dom = max(plan, key=lambda L: L["n_rows"])
    kname = dom["kernel"]
    traffic = load_traffic(kname, wl.name)
    roof = {"bound": bound,
            "achieved": round(tflops if bound == "mfma" else gbs, 3),
            "peak": peak_fl if bound == "mfma" else PEAK_HBM_GBS,
            "unit": "TFLOP/s" if bound == "mfma" else "GB/s",
            "frac": round((tflops / peak_fl) if bound == "mfma" else (gbs / PEAK_HBM_GBS), 4),
            "traffic": traffic,
            "kernel": kname,
            "launch": {"tile": dom["tile"], "workgroups": dom["workgroups"], "a_mode": dom["a_mode"],
                       "launches_per_step": len(plan)},
            "per_launch": {"flops": r["flops"], "alg_bytes": r["bytes"], "avg_us": round(r["ms"] * 1e3, 3)},
            "hbm_frac": round(gbs / PEAK_HBM_GBS, 4),
            "frac_roofline_model": round(tflops / min(peak_fl, ai * PEAK_HBM_GBS / 1e3), 4)}
    also = {}
    per_config = {}
    for spec in [v.strip() for v in args.extra.split(",") if v.strip()]:
        if spec.endswith("n"):
            e = int(spec[:-1])
            also[workloads_name(e) + "_merger_layernorm"] = time_merger_front(e, max(5, min(args.steps, 50)),
                                                                               eager=args.eager)
            continue
        e, as_rows, with_add, fold, share, stage = parse_extra(spec)
        if e == args.workload and not (as_rows or with_add or fold or stage or share is not None):
            continue
        st = max(5, min(args.steps, 50))
        q = time_workload(e, st, 3, graph=not args.eager, rows=as_rows, items=share, reps=3, add=with_add,
                          fold=fold, stage=stage, keep_out=cpu_leg)
        qt = q["ms"] / 1e3
        qpk = PEAK_BF16_TFLOPS if q["wl"].w_dtype == "bf16" else PEAK_F32_MATRIX_TFLOPS
        qai = q["flops"] / q["bytes"]
        qdom = max(q["plan"], key=lambda L: L["n_rows"])
        key = (q["wl"].name + ("_as_patch_rows" if as_rows else "") + ("_plus_pos_embed" if with_add else "")
               + ("_image_fold_approx" if fold else "") + ("_lds_staged" if stage else ""))
        also[key] = {"patches_per_s": round(q["n"] / qt, 1), "ms_per_step": round(q["ms"], 5),
                              "tflops": round(q["flops"] / qt / 1e12, 2),
                              "frac_matrix_peak": round(q["flops"] / qt / 1e12 / qpk, 4),
                              "frac_hbm": round(q["bytes"] / qt / 1e9 / PEAK_HBM_GBS, 4),
                              # against the roofline model min(peak, AI x HBM bandwidth)
                              "frac_roofline_model": round(q["flops"] / qt / 1e12 / min(qpk, qai * PEAK_HBM_GBS / 1e3), 4),
                              "kernel": qdom["kernel"], "tile": qdom["tile"], "launches_per_step": len(q["plan"]),
                              "n_patches": q["n"], "steps": st,
                              # HBM bytes per launch from committed counters on this kernel code, if any
                              "traffic": load_traffic(qdom["kernel"], key) if len(q["plan"]) == 1 else None,
                              **({"approximate": "image fold: W[:, :, 0] + W[:, :, 1] rounded to bf16 once; "
                                                 "tflops counts the nominal Conv3d FLOPs, the matrix cores do "
                                                 "about half for images"} if fold else {})}
        if cpu_leg:
            # the cpu_baseline leg for this line: oracle time and parity of its timed output
            per_config[key] = cpu_baseline_config(q, approximate=fold)
        del q
    if not args.no_context and not args.eager:
        also["context_library_gemm_" + workloads_name(5)] = time_linear_context(5)
        also["context_library_gemm_square_8192"] = time_square_context()
    cpu, parity = cpu_baseline(r) if cpu_leg else (None, None)
    if cpu is not None:
        cpu["per_config"] = per_config
    line = {
        "metric": METRIC, "value": round(r["n"] / t_s, 1), "unit": "patches/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(r["ms"], 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32", "data": "synthetic",
        "config": {"workload": wl.name, "n_patches": r["n"], "k": wl.k, "embed": wl.embed,
                   "patch": wl.patch, "input": "%s %s" % (wl.kind, list(wl.input_shape)),
                   "grid_thw": [list(g) for g in wl.grid[:1]] + (["x%d" % len(wl.grid)] if len(wl.grid) > 1 else []),
                   "order": wl.order, "bias": wl.bias, "out_dtype": wl.out_dtype,
                   "parallelism": "single GPU"},
        "tflops": round(tflops, 3), "frac_bf16_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "eager_ms_per_step": round(r["eager_ms"], 6),
        "timing": r["timing"], "timing_stats": r["stats"],
        "cold_ms_per_step": round(r["cold_ms"], 6) if r["cold_ms"] is not None else None,
        "roofline": roof, "cpu_baseline": cpu,
        "parity_max_err": parity["max_abs_err"] if parity else None, "parity": parity,
        "also": also,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
