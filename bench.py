"""Benchmark of the gfx950 vision PatchEmbed: one JSON line on stdout.

A step is one PatchEmbed forward (gather + matrix product + epilogue, one kernel launch per
<= 64 items) over one batch of synthetic input already resident in HBM. The timed region is
K steps captured back to back in a HIP graph and replayed once, bracketed by HIP events on the
stream they run on; `eager_ms_per_step` gives the same K steps launched one by one from Python.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 2] [--extra 5]
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "PatchEmbed patches/s + TFLOP/s (% bf16 MFMA peak) on 1 MI355X"
PEAK_BF16_TFLOPS = 2516.6   # 256 CUs x 2.4 GHz x 4096 dense bf16 flop/clk/CU
PEAK_F32_MATRIX_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0
KERNEL_SOURCES = sorted(glob.glob(os.path.join(ROOT, "vlm_vision_patch_amd", "csrc", "*")))


def kernel_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        h.update(open(p, "rb").read())
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


def dominant_kernel(wl, num_cus=256):
    """Name of the kernel that does the step's work, by the library's tile choice for the largest
    launch (items that are all alike share one launch, others go 64 to a launch): in rounds of one
    workgroup per CU, 256 x 256 tiles cost ~30 us a round, 256 x 128 ~18 us and split-k ~8 us; the
    fewest (rounds x cost) wins. fp32 runs the 16x16 kernel."""
    if wl.w_dtype != "bf16":
        return "pe_fwd16_kernel"
    rows = [t * h * w for (t, h, w) in wl.grid]
    frames = list(wl.frames) or [None] * len(rows)
    if all(tuple(g) == tuple(wl.grid[0]) and f == frames[0] for g, f in zip(wl.grid, frames)):
        n = sum(rows)
    else:
        n = max(sum(rows[i:i + 64]) for i in range(0, len(rows), 64))
    E = wl.embed
    rounds = lambda tiles: -(-tiles // num_cus)
    rt = -(-n // 256)
    skn = 160 if E % 160 == 0 else 128
    c256 = rounds(rt * -(-E // 256)) * 30
    c128 = rounds(rt * -(-E // 128)) * 18
    csk = rounds(-(-n // 32) * -(-E // skn)) * 8
    return "pe_fwd32_kernel" if min(c256, c128) <= csk else "pe_fwd32_sk_kernel"


def time_workload(idx, steps, warmup, graph=True, rows=False, items=None, reps=10, cold=False, add=False,
                  fold=False):
    """rows: feed the workload's patches as pre-flattened rows [N, K] (the processor's
    pixel_values layout) instead of its frames: same N, weight and bias, synthetic N(0, 1) rows.
    items: keep only the first `items` items (one GPU's share of an item split).
    The graph of K steps is replayed `reps` times, each replay timed: median, p10 and p90 per step.
    cold: also time single launches after overwriting a 1 GiB buffer (L2 and the 256 MB
    Infinity Cache hold nothing of the inputs), median of `reps`.
    add: fuse the add of a synthetic [N, E] tensor (position embeddings) into the epilogue.
    fold: the approximate image-fold mode (single-frame items on W[:, :, 0] + W[:, :, 1] in bf16)."""
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
    x, w = x.to(dev), w.to(dev)
    b = b.to(dev) if b is not None else None
    mod = pe.PatchEmbed(w, b, order=wl.order, out_dtype=workloads.DTYPES[wl.out_dtype], image_fold=fold)
    out = torch.empty((n, wl.embed), dtype=workloads.DTYPES[wl.out_dtype], device=dev)
    addend = None
    if add:
        addend = (workloads.random_tensor((n, wl.embed), seed=3000 + idx) * 0.02).to(
            workloads.DTYPES[wl.out_dtype]).to(dev)
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
                stats=stats, cold_ms=cold_ms)


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
    esz = rows.element_size()
    ln_bytes = 2 * n * E * esz + 2 * E * esz
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
    for _ in range(3):
        y = torch.nn.functional.linear(a, w2, b2)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        y = torch.nn.functional.linear(a, w2, b2)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del y, a
    return {"what": "torch.nn.functional.linear (hipBLASLt) on a contiguous [N, K] patch matrix, same "
                    "N, K, E, dtype and bias; the patchify gather not included", "ms_per_step": round(ms, 5),
            "tflops": round(2.0 * n * wl.k * wl.embed / (ms / 1e3) / 1e12, 2), "steps": steps}


def cpu_baseline(idx, min_seconds=10.0):
    """The oracle, as it stands, timed on this host on repeats of the whole workload (or on its
    first rows when one pass would exceed the bound)."""
    import workloads
    import oracle
    wl = workloads.WORKLOADS[idx]
    x, w, b = workloads.generate(wl)
    n = sum(t * h * ww for (t, h, ww) in wl.grid)
    threads = max(1, min(os.cpu_count() or 1, 16))
    rows = None
    per_row = 2.0 * wl.k * wl.embed
    if n * per_row > 2e11:      # more than ~30 s on 16 cores: time the first rows only
        rows = list(range(int(2e11 / per_row)))
    done, t0 = 0, time.perf_counter()
    reps = 0
    while True:
        oracle.forward(x, w, b, grid=wl.grid, frames=list(wl.frames) or None, kind=wl.kind,
                       order=wl.order, rows=rows, threads=threads)
        done += n if rows is None else len(rows)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or rows is not None:
            break
    sample = ("%d passes over all %d rows" % (reps, n)) if rows is None else \
        ("first %d of %d rows" % (len(rows), n))
    return {"value": done / el, "unit": "patches/s", "cores": threads, "kind": "oracle",
            "sample": "%s of %s (fp64 direct Conv3d, %d threads, %.1f s)" % (sample, wl.name, threads, el)}


def load_traffic(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 FETCH_SIZE/WRITE_SIZE counters, if they were
    taken on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
        rec = d.get(workload)
        if rec and rec.get("kernel_hash") == kernel_hash():
            return rec["bytes_per_launch"]
    except Exception:
        return None
    return None


def workloads_name(idx):
    import workloads
    return workloads.WORKLOADS[idx].name


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--extra", type=str, default="5,5r,5a,5n,5f,2f,5s8,3,4,6,1",
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
    args = ap.parse_args()
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

    r = time_workload(args.workload, args.steps, args.warmup, graph=not args.eager, cold=not args.eager)
    wl = r["wl"]
    t_s = r["ms"] / 1e3
    tflops = r["flops"] / t_s / 1e12
    gbs = r["bytes"] / t_s / 1e9
    bf16 = wl.w_dtype == "bf16"
    peak_fl = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_MATRIX_TFLOPS
    ai = r["flops"] / r["bytes"]
    ridge = peak_fl * 1e12 / (PEAK_HBM_GBS * 1e9)
    bound = "mfma" if ai >= ridge else "hbm"
    kname = dominant_kernel(wl, torch.cuda.get_device_properties(0).multi_processor_count)
    traffic = load_traffic(kname, wl.name)
    roof = {"bound": bound,
            "achieved": round(tflops if bound == "mfma" else gbs, 3),
            "peak": peak_fl if bound == "mfma" else PEAK_HBM_GBS,
            "unit": "TFLOP/s" if bound == "mfma" else "GB/s",
            "frac": round((tflops / peak_fl) if bound == "mfma" else (gbs / PEAK_HBM_GBS), 4),
            "traffic": traffic,
            "kernel": kname,
            "per_launch": {"flops": r["flops"], "alg_bytes": r["bytes"], "avg_us": round(r["ms"] * 1e3, 3)},
            "hbm_frac": round(gbs / PEAK_HBM_GBS, 4)}
    also = {}
    for spec in [v.strip() for v in args.extra.split(",") if v.strip()]:
        if spec.endswith("n"):
            e = int(spec[:-1])
            also[workloads_name(e) + "_merger_layernorm"] = time_merger_front(e, max(5, min(args.steps, 50)),
                                                                               eager=args.eager)
            continue
        as_rows = spec.endswith("r")
        with_add = spec.endswith("a")
        fold = spec.endswith("f")
        share = int(spec.split("s")[1]) if "s" in spec else None
        e = int(spec.rstrip("raf").split("s")[0])
        if e == args.workload and not as_rows and share is None and not fold:
            continue
        st = max(5, min(args.steps, 50))
        q = time_workload(e, st, 3, graph=not args.eager, rows=as_rows, items=share, reps=3, add=with_add,
                          fold=fold)
        qt = q["ms"] / 1e3
        qpk = PEAK_BF16_TFLOPS if q["wl"].w_dtype == "bf16" else PEAK_F32_MATRIX_TFLOPS
        also[q["wl"].name + ("_as_patch_rows" if as_rows else "") + ("_plus_pos_embed" if with_add else "")
             + ("_image_fold_approx" if fold else "")] = {"patches_per_s": round(q["n"] / qt, 1), "ms_per_step": round(q["ms"], 5),
                              "tflops": round(q["flops"] / qt / 1e12, 2),
                              "frac_matrix_peak": round(q["flops"] / qt / 1e12 / qpk, 4),
                              "frac_hbm": round(q["bytes"] / qt / 1e9 / PEAK_HBM_GBS, 4),
                              "n_patches": q["n"], "steps": st,
                              **({"approximate": "image fold: W[:, :, 0] + W[:, :, 1] rounded to bf16 once; "
                                                 "tflops counts the nominal Conv3d FLOPs, the matrix cores do "
                                                 "about half for images"} if fold else {})}
    if not args.no_context and not args.eager:
        also["context_library_gemm_" + workloads_name(5)] = time_linear_context(5)
    cpu = None if args.no_cpu else cpu_baseline(args.workload)
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
        "roofline": roof, "cpu_baseline": cpu, "also": also,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
