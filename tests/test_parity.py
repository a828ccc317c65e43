"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the same seeded inputs.

Tolerances (fixed for the workloads and checked against the arithmetic: bf16 products, fp32 accumulation):
  * fp32 output from fp32 inputs: max |err| <= 5e-4 (unit-variance inputs);
  * bf16 output: |err| <= 1e-3 + 1e-2 * |ref| elementwise;
  * fp32 output from bf16 inputs: max |err| <= 5e-4;
  * integer-valued inputs: fp32 output bit-exact, bf16 output == round-to-nearest-even(ref).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def pe():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import vlm_vision_patch_amd
    return vlm_vision_patch_amd


def say(msg):
    print("[case] " + msg, flush=True)


def check(got, ref, out_dtype, what):
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    err = np.abs(got - ref)
    if out_dtype == torch.bfloat16:
        bad = err > 1e-3 + 1e-2 * np.abs(ref)
        assert not bad.any(), "%s: %d of %d outside 1e-3 + 1e-2|ref| (max err %.3g)" % (
            what, bad.sum(), bad.size, err.max())
    else:
        assert err.max() <= 5e-4, "%s: max err %.3g > 5e-4" % (what, err.max())
    return err.max()


def run(pe, name, x, w, b, grid, frames=None, kind="frames", order="raster", out_dtype=None,
        rows=None, add=None, inplace=False):
    say("%s: kind=%s order=%s grid=%s frames=%s x=%s w=%s bias=%s out=%s" % (
        name, kind, order, grid if len(grid) <= 4 else "%d items" % len(grid), frames if frames is None or len(frames) <= 4 else "...",
        tuple(x.shape), tuple(w.shape), b is not None, out_dtype))
    out_dtype = out_dtype or w.dtype
    mod = pe.PatchEmbed(w.to(DEV), b.to(DEV) if b is not None else None, order=order, out_dtype=out_dtype)
    if add is None:
        out = mod(x.to(DEV), grid, frames, kind=kind)
    else:
        add_dev = add.to(DEV).contiguous()
        out = mod(x.to(DEV), grid, frames, kind=kind, add=add_dev, out=add_dev if inplace else None)
    torch.cuda.synchronize()
    if rows is not None:
        got = out[torch.as_tensor(rows, device=DEV)].float().cpu().double().numpy()
    else:
        got = out.float().cpu().double().numpy()
    cast = None if x.dtype == w.dtype else {torch.bfloat16: "bf16", torch.float32: "f32"}[w.dtype]
    ref = oracle.forward(x, w, b, grid=grid, frames=frames, kind=kind, order=order, rows=rows,
                         cast_input_to=cast, addend=add)
    mod.close()
    return got, ref, out_dtype


# ---------------------------------------------------------------------------------------------
# the five workloads at full size, in the launch configuration the benchmark times
# ---------------------------------------------------------------------------------------------

def sampled_rows(n, seed, count):
    """Rows the oracle computes one by one: first/last rows, every 256-row tile edge, items'
    edges (5184-row images), plus a seeded random sample."""
    rng = np.random.default_rng(seed)
    edges = set([0, 1, n - 1, n - 2])
    for step in (64, 256, 5184):
        for e in range(step, n, step):
            edges.update((e - 1, e))
    picks = set(rng.choice(n, size=min(count, n), replace=False).tolist())
    rows = sorted(r for r in edges | picks if 0 <= r < n)
    return np.array(rows, dtype=np.int64)


@pytest.mark.parametrize("idx", [1, 2, 3, 4])
def test_workload_full(pe, idx):
    wl = workloads.WORKLOADS[idx]
    x, w, b = workloads.generate(wl)
    got, ref, od = run(pe, wl.name, x, w, b, list(wl.grid), list(wl.frames) or None,
                       kind=wl.kind, order=wl.order, out_dtype=workloads.DTYPES[wl.out_dtype])
    e = check(got, ref, od, wl.name)
    print("%s: max err %.3g" % (wl.name, e), flush=True)


def test_workload_5_sampled(pe):
    wl = workloads.WORKLOADS[5]
    x, w, b = workloads.generate(wl)
    rows = sampled_rows(331776, seed=5, count=1500)
    got, ref, od = run(pe, wl.name, x, w, b, list(wl.grid), list(wl.frames), kind=wl.kind,
                       order=wl.order, out_dtype=torch.bfloat16, rows=rows)
    e = check(got, ref, od, wl.name)
    print("%s: %d sampled rows, max err %.3g" % (wl.name, len(rows), e), flush=True)


@pytest.mark.timeout(1200)
def test_workload_5_all_rows(pe):
    """Every one of the 331,776 x 1280 outputs of the 64-image batch (the configuration the
    benchmark reports), element by element, in the benchmark's launch configuration: the oracle runs
    in chunks of four images' rows so that host memory stays bounded (N = t*h*w per item, items
    concatenated: "freechatgpt/mytransformer" section 3.2)."""
    import bench
    wl = workloads.WORKLOADS[5]
    x, w, b = workloads.generate(wl)
    n = sum(t * h * ww for (t, h, ww) in wl.grid)
    say("%s: all %d rows, oracle in chunks of 20736 rows" % (wl.name, n))
    mod = pe.PatchEmbed(w.to(DEV), b.to(DEV), order=wl.order, out_dtype=torch.bfloat16)
    out = mod(x.to(DEV), list(wl.grid), list(wl.frames))
    torch.cuda.synchronize()
    mod.close()
    # exact fp64 copies once, so that the chunks do not convert the inputs again
    xd, wd, bd = oracle._f64(x), oracle._f64(w), oracle._f64(b)
    threads = bench.cpu_info()["usable"]
    chunk, worst = 4 * 5184, 0.0
    for r0 in range(0, n, chunk):
        rows = np.arange(r0, min(n, r0 + chunk), dtype=np.int64)
        ref = oracle.forward(xd, wd, bd, grid=list(wl.grid), frames=list(wl.frames), order=wl.order, rows=rows,
                             threads=threads)
        got = out[r0:r0 + len(rows)].float().cpu().double().numpy()
        worst = max(worst, check(got, ref, torch.bfloat16, "%s rows %d..%d" % (wl.name, r0, r0 + len(rows) - 1)))
        print("rows %d..%d ok (max err so far %.3g)" % (r0, r0 + len(rows) - 1, worst), flush=True)
    print("%s: all %d rows within 1e-3 + 1e-2|ref|, max err %.3g" % (wl.name, n, worst), flush=True)


def test_workload_6_sampled(pe):
    """The Qwen3-VL-2B-shaped workload (P16, E1024, bias) over items of mixed sizes: every item's
    first and last rows plus a seeded sample."""
    wl = workloads.WORKLOADS[6]
    x, w, b = workloads.generate(wl)
    n = sum(t * h * ww for (t, h, ww) in wl.grid)
    starts = np.cumsum([0] + [t * h * ww for (t, h, ww) in wl.grid])
    edges = set()
    for s0, s1 in zip(starts[:-1], starts[1:]):
        edges.update((int(s0), int(s0) + 1, int(s1) - 2, int(s1) - 1))
    rows = np.array(sorted(edges | set(sampled_rows(n, 31, 700).tolist())), dtype=np.int64)
    got, ref, od = run(pe, wl.name, x, w, b, [list(g) for g in wl.grid], list(wl.frames), order=wl.order,
                       rows=rows)
    check(got, ref, od, wl.name)


def test_workload_5_raster_sampled(pe):
    """The same batch in raster order: the order is a free choice of the caller."""
    wl = workloads.WORKLOADS[5]
    x, w, b = workloads.generate(wl)
    rows = sampled_rows(331776, seed=6, count=500)
    got, ref, od = run(pe, wl.name + "_raster", x, w, b, list(wl.grid), list(wl.frames),
                       order="raster", out_dtype=torch.bfloat16, rows=rows)
    check(got, ref, od, wl.name + " raster")


# ---------------------------------------------------------------------------------------------
# edge cases: ragged tails, several tiles, multi-item tables, orders, dtypes, bias, E tails
# ---------------------------------------------------------------------------------------------

def make(seed, shape, dtype, dist="normal", bound=1.0):
    return workloads.random_tensor(shape, seed=seed, dtype=dtype, dist=dist, bound=bound)


CASES = [
    # name, P, E, items [(t,h,w,F)], order, in/w dtype, out dtype, bias
    ("image_ragged_raster", 14, 1280, [(1, 6, 10, 1)], "raster", torch.bfloat16, torch.bfloat16, False),
    ("image_ragged_merge", 14, 1280, [(1, 6, 10, 1)], "merge", torch.bfloat16, torch.bfloat16, True),
    ("video_odd_frames", 14, 256, [(2, 4, 4, 3)], "merge", torch.bfloat16, torch.bfloat16, True),
    ("mixed_items", 14, 512, [(1, 4, 6, 1), (3, 2, 4, 6), (1, 8, 2, 1), (2, 6, 6, 4)], "merge",
     torch.bfloat16, torch.bfloat16, True),
    ("mixed_items_raster", 14, 512, [(1, 3, 5, 1), (2, 3, 3, 3), (1, 7, 1, 1)], "raster",
     torch.bfloat16, torch.bfloat16, False),
    ("p16_e1152_tail", 16, 1152, [(1, 10, 12, 1), (1, 4, 4, 1)], "raster", torch.bfloat16, torch.bfloat16, True),
    ("p16_video_merge", 16, 1024, [(2, 6, 8, 4)], "merge", torch.bfloat16, torch.bfloat16, True),
    ("e16_minimum", 14, 16, [(1, 2, 2, 1)], "raster", torch.bfloat16, torch.bfloat16, True),
    ("e48_odd_blocks", 14, 48, [(1, 4, 4, 1)], "merge", torch.bfloat16, torch.bfloat16, False),
    ("bf16_in_f32_out", 14, 1280, [(1, 16, 20, 1)], "merge", torch.bfloat16, torch.float32, True),
    ("f32_frames", 14, 640, [(1, 6, 8, 1), (2, 4, 2, 4)], "merge", torch.float32, torch.float32, True),
    ("f32_p16_frames", 16, 320, [(1, 4, 6, 1)], "raster", torch.float32, torch.float32, False),
    ("single_patch", 14, 1280, [(1, 1, 1, 1)], "raster", torch.bfloat16, torch.bfloat16, True),
    ("large_merge_2k", 14, 1280, [(1, 40, 52, 1)], "merge", torch.bfloat16, torch.bfloat16, True),
    ("tall_video_big_tiles", 14, 1280, [(8, 24, 24, 16)], "merge", torch.bfloat16, torch.bfloat16, False),
    # one frame size, image-ness changing from item to item: a launch per run of images / videos
    ("images_and_videos_one_size", 14, 640, [(1, 4, 6, 1), (2, 4, 6, 3), (1, 4, 6, 1), (1, 4, 6, 2),
                                             (1, 4, 6, 1)], "merge", torch.bfloat16, torch.bfloat16, True),
    ("t1_two_frames", 14, 320, [(1, 6, 4, 2)], "raster", torch.bfloat16, torch.bfloat16, False),
    # wide embeddings: 32 column tiles of the split-k kernel, 16 of the large-tile kernel
    ("e4096_splitk", 14, 4096, [(1, 20, 24, 1)], "merge", torch.bfloat16, torch.bfloat16, True),
    ("e2304_p16_raster", 16, 2304, [(1, 12, 14, 1)], "raster", torch.bfloat16, torch.float32, True),
    # fp32 weight and input, bf16 output (fp32 products, one cast)
    ("f32_weight_bf16_out", 14, 640, [(1, 6, 8, 1), (2, 4, 2, 4)], "merge", torch.float32, torch.bfloat16, True),
    ("f32_p16_bf16_out_e384", 16, 384, [(1, 4, 6, 1), (1, 10, 2, 1)], "raster", torch.float32, torch.bfloat16,
     False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_frames_edge_cases(pe, case):
    name, P, E, items, order, dt, od, bias = case
    xs = [make(100 + i, (F, 3, h * P, w * P), dt) for i, (t, h, w, F) in enumerate(items)]
    x = torch.cat([a.reshape(-1) for a in xs])
    K = 3 * 2 * P * P
    w = make(200, (E, 3, 2, P, P), dt, "uniform", 1 / math.sqrt(K))
    b = make(201, (E,), dt, "uniform", 1 / math.sqrt(K)) if bias else None
    grid = [[t, h, ww] for (t, h, ww, F) in items]
    frames = [F for (*_, F) in items]
    got, ref, _ = run(pe, name, x, w, b, grid, frames, order=order, out_dtype=od)
    check(got, ref, od, name)


@pytest.mark.parametrize("P,N,dt,od", [(14, 1, torch.bfloat16, torch.bfloat16),
                                       (14, 333, torch.bfloat16, torch.bfloat16),
                                       (16, 777, torch.bfloat16, torch.float32),
                                       (14, 300, torch.float32, torch.float32),
                                       (16, 65, torch.float32, torch.float32),
                                       (14, 1024, torch.float32, torch.bfloat16),
                                       (16, 300, torch.float32, torch.bfloat16),
                                       (14, 20000, torch.bfloat16, torch.bfloat16),
                                       (16, 9000, torch.bfloat16, torch.bfloat16)])
def test_patch_rows(pe, P, N, dt, od):
    K = 3 * 2 * P * P
    x = make(300 + N, (N, K), dt)
    w = make(301, (1280, 3, 2, P, P), dt, "uniform", 1 / math.sqrt(K))
    b = make(302, (1280,), dt, "uniform", 1 / math.sqrt(K))
    rows = None if N <= 4000 else sampled_rows(N, 7, 500)
    got, ref, _ = run(pe, "patches_P%d_N%d" % (P, N), x, w, b, [[1, 1, N]], kind="patches",
                      out_dtype=od, rows=rows)
    check(got, ref, od, "patches")


@pytest.mark.parametrize("case", ["images_4x448_bias", "images_16x448", "rows_3000_E1168"])
def test_mid_size_tiles(pe, case):
    """Sizes where the launcher picks 256 x 128 tiles (between the split-k and the 256 x 256
    ranges), including a ragged row count and an embed width that leaves a partial column block."""
    if case.startswith("images"):
        k = 4 if case == "images_4x448_bias" else 16
        E, P = 1280, 14
        K = 3 * 2 * P * P
        x = make(700 + k, (k, 3, 448, 448), torch.bfloat16)
        w = make(701, (E, 3, 2, P, P), torch.bfloat16, "uniform", 1 / math.sqrt(K))
        b = make(702, (E,), torch.bfloat16, "uniform", 1 / math.sqrt(K)) if "bias" in case else None
        grid, n = [[1, 32, 32]] * k, k * 1024
        rows = sampled_rows(n, 11 + k, 400)
        got, ref, od = run(pe, case, x, w, b, grid, [1] * k, order="merge", rows=rows)
    else:
        E, P, n = 1168, 14, 3000
        K = 3 * 2 * P * P
        x = make(710, (n, K), torch.bfloat16)
        w = make(711, (E, 3, 2, P, P), torch.bfloat16, "uniform", 1 / math.sqrt(K))
        b = make(712, (E,), torch.bfloat16, "uniform", 1 / math.sqrt(K))
        rows = sampled_rows(n, 13, 400)
        got, ref, od = run(pe, case, x, w, b, [[1, 1, n]], kind="patches", rows=rows)
    check(got, ref, od, case)


@pytest.mark.parametrize("case", ["image_small_merge", "video_odd_frames", "images_mid", "images_8",
                                  "rows_small", "rows_large", "image_p16_bias"])
def test_fp32_input_bf16_weight(pe, case):
    """fp32 pixels on a bf16 weight: rounded to bf16 (nearest even) on load, as the module's
    input cast does; the oracle rounds the input the same way first."""
    P = 16 if "p16" in case else 14
    K = 3 * 2 * P * P
    E = 1152 if "p16" in case else 1280
    w = make(801, (E, 3, 2, P, P), torch.bfloat16, "uniform", 1 / math.sqrt(K))
    b = make(802, (E,), torch.bfloat16, "uniform", 1 / math.sqrt(K)) if "bias" in case or "video" in case else None
    rows = None
    if case.startswith("rows"):
        n = 300 if case == "rows_small" else 20000
        x = make(803 + n, (n, K), torch.float32)
        rows = None if n <= 4000 else sampled_rows(n, 17, 400)
        got, ref, od = run(pe, case, x, w, b, [[1, 1, n]], kind="patches", out_dtype=torch.bfloat16, rows=rows)
    else:
        if case == "image_small_merge":
            items = [(1, 16, 20, 1)]
        elif case == "video_odd_frames":
            items = [(2, 8, 6, 3), (1, 4, 4, 2)]
        elif case == "image_p16_bias":
            items = [(1, 28, 28, 1)]
        else:
            items = [(1, 32, 32, 1)] * (4 if case == "images_mid" else 8)
        x = torch.cat([make(810 + i, (F, 3, hh * P, ww * P), torch.float32).reshape(-1)
                       for i, (t, hh, ww, F) in enumerate(items)])
        grid = [[t, hh, ww] for (t, hh, ww, F) in items]
        n = sum(t * hh * ww for (t, hh, ww) in grid)
        rows = None if n <= 4000 else sampled_rows(n, 19, 400)
        got, ref, od = run(pe, case, x, w, b, grid, [F for (*_, F) in items], order="merge",
                           out_dtype=torch.bfloat16, rows=rows)
    check(got, ref, od, case)


def test_images_and_videos_large(pe):
    """Images and a video of one frame size at a size that uses the large-tile kernels: the
    library splits the call into launches by image-ness; rows sampled."""
    P, E = 14, 1280
    K = 3 * 2 * P * P
    items = [(1, 32, 32, 1)] * 3 + [(2, 32, 32, 4)] + [(1, 32, 32, 1)] * 3
    xs = [make(900 + i, (F, 3, h * P, ww * P), torch.bfloat16) for i, (t, h, ww, F) in enumerate(items)]
    x = torch.cat([a.reshape(-1) for a in xs])
    w = make(901, (E, 3, 2, P, P), torch.bfloat16, "uniform", 1 / math.sqrt(K))
    b = make(902, (E,), torch.bfloat16, "uniform", 1 / math.sqrt(K))
    grid = [[t, h, ww] for (t, h, ww, F) in items]
    n = sum(t * h * ww for (t, h, ww) in grid)
    got, ref, od = run(pe, "images_and_video_large", x, w, b, grid, [F for (*_, F) in items], order="merge",
                       rows=sampled_rows(n, 23, 500))
    check(got, ref, od, "images and video")


def test_concurrent_streams_one_handle(pe):
    """The handle is immutable: calls on two streams at once (different inputs, sizes and so
    kernels) give the same results as the oracle."""
    P, E = 14, 1280
    K = 3 * 2 * P * P
    w = make(950, (E, 3, 2, P, P), torch.bfloat16, "uniform", 1 / math.sqrt(K))
    b = make(951, (E,), torch.bfloat16, "uniform", 1 / math.sqrt(K))
    mod = pe.PatchEmbed(w.to(DEV), b.to(DEV), order="merge")
    x1 = make(952, (1, 3, 16 * P, 64 * P), torch.bfloat16)       # 1024 patches: split-k
    x2 = make(953, (8, 3, 32 * P, 32 * P), torch.bfloat16)       # 8192 patches: large tiles
    g1, g2 = [[1, 16, 64]], [[1, 32, 32]] * 8
    say("two streams: %s and %s" % (g1, "8 x [1, 32, 32]"))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    d1, d2 = x1.to(DEV), x2.to(DEV)
    torch.cuda.synchronize()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            o1 = mod(d1, g1, [1])
        with torch.cuda.stream(s2):
            o2 = mod(d2, g2, [1] * 8)
        outs.append((o1, o2))
    torch.cuda.synchronize()
    r1 = oracle.forward(x1, w, b, grid=g1, frames=[1], order="merge")
    rows2 = sampled_rows(8192, 29, 300)
    r2 = oracle.forward(x2, w, b, grid=g2, frames=[1] * 8, order="merge", rows=rows2)
    for o1, o2 in outs:
        check(o1.float().cpu().double().numpy(), r1, torch.bfloat16, "stream 1")
        check(o2[torch.as_tensor(rows2, device=DEV)].float().cpu().double().numpy(), r2, torch.bfloat16, "stream 2")
    mod.close()


def test_host_threads_share_one_handle(pe):
    """Several host threads call one handle at once, each on its own stream with its own request
    (ctypes releases the GIL during the call). Every result equals the same call made alone, bit
    for bit (the kernels are deterministic), and each thread reads back its own pe_last_error."""
    import ctypes
    import threading
    P, E = 14, 640
    K = 3 * 2 * P * P
    w = make(2800, (E, 3, 2, P, P), torch.bfloat16, "uniform", 1 / math.sqrt(K))
    b = make(2801, (E,), torch.bfloat16, "uniform", 1 / math.sqrt(K))
    mod = pe.PatchEmbed(w.to(DEV), b.to(DEV), order="merge")
    reqs = [([[1, 16, 64]], [1]), ([[1, 32, 32]] * 4, [1] * 4), ([[2, 8, 10]], [4]),
            ([[1, 6, 8], [1, 10, 4], [3, 2, 2]], [1, 1, 6])]
    say("host threads: %d requests on one handle" % len(reqs))
    xs = [make(2810 + i, (mod.input_elements(g, f),), torch.bfloat16).to(DEV) for i, (g, f) in enumerate(reqs)]
    alone = [mod(x, g, f) for x, (g, f) in zip(xs, reqs)]
    torch.cuda.synchronize()
    results = [[] for _ in reqs]
    errs = [None] * len(reqs)

    def worker(i):
        g, f = reqs[i]
        st = torch.cuda.Stream()
        with torch.cuda.stream(st):
            for k in range(16):
                results[i].append(mod(xs[i], g, f))
                if k == 8:
                    # item i of i + 1 has an odd width: validation fails before any launch
                    bad = (ctypes.c_int32 * (3 * (i + 1)))(*([1, 2, 2] * i + [1, 2, 3]))
                    rc = pe.lib.pe_forward(mod._h, 1, 0x1000, 1, bad, None, i + 1, 0x2000, None)
                    errs[i] = (rc, pe.last_error())
        st.synchronize()

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(reqs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    mod.close()
    for i in range(len(reqs)):
        assert len(results[i]) == 16, "thread %d did not finish" % i
        for o in results[i]:
            assert torch.equal(o, alone[i]), "thread %d: result differs from the call made alone" % i
        rc, msg = errs[i]
        assert rc == pe.PE_ERR_SHAPE and ("item %d:" % i) in msg, (i, rc, msg)
    # the results made alone are right
    r0 = oracle.forward(xs[0].cpu(), w, b, grid=reqs[0][0], frames=reqs[0][1], order="merge")
    check(alone[0].double().cpu().numpy(), r0, torch.bfloat16, "thread request 0")


def test_request_cache_of_the_binding(pe):
    """PatchEmbed keeps the marshalled arguments of each request by value: more distinct requests
    than it holds (it starts over when full), and a grid list changed in place between two calls,
    still give the oracle's results."""
    P, E = 14, 64
    K = 3 * 2 * P * P
    w = make(2900, (E, 3, 2, P, P), torch.bfloat16, "uniform", 1 / math.sqrt(K))
    mod = pe.PatchEmbed(w.to(DEV), order="merge")
    say("binding request cache: %d distinct grids, then a grid changed in place" % (mod._PLANS_MAX + 6))
    x = make(2901, (3 * 4 * P * 2 * (mod._PLANS_MAX + 6) * P,), torch.bfloat16)
    xd = x.to(DEV)
    for k in range(1, mod._PLANS_MAX + 7):
        g = [[1, 4, 2 * k]]
        n_el = 3 * 4 * P * 2 * k * P
        out = mod(xd[:n_el], g, [1])
        if k in (1, mod._PLANS_MAX, mod._PLANS_MAX + 1, mod._PLANS_MAX + 6):
            ref = oracle.forward(x[:n_el], w, None, grid=g, frames=[1], order="merge")
            check(out.double().cpu().numpy(), ref, torch.bfloat16, "grid %s" % g)
    g = [[1, 4, 6]]
    fr = [1]
    o1 = mod(xd[:3 * 4 * P * 6 * P], g, fr)
    g[0][2] = 8                               # same list object, new width
    o2 = mod(xd[:3 * 4 * P * 8 * P], g, fr)
    assert o2.shape[0] == 32 and o1.shape[0] == 24
    ref = oracle.forward(x[:3 * 4 * P * 8 * P], w, None, grid=[[1, 4, 8]], frames=[1], order="merge")
    check(o2.double().cpu().numpy(), ref, torch.bfloat16, "grid changed in place")
    mod.close()


MIXED = {
    # name: (items [(t, h, w, F)], dtype, order); frame sizes differ within one launch
    "images_large": ([(1, 72, 72, 1), (1, 32, 48, 1), (1, 16, 64, 1), (1, 56, 40, 1), (1, 24, 24, 1),
                      (1, 64, 64, 1), (1, 40, 30, 1), (1, 8, 8, 1)], torch.bfloat16, "merge"),
    "videos": ([(2, 8, 6, 4), (1, 12, 10, 2), (3, 4, 4, 5)], torch.bfloat16, "merge"),
    "images_f32_input": ([(1, 20, 30, 1), (1, 34, 18, 1), (1, 6, 4, 1)], torch.float32, "merge"),
    "images_raster": ([(1, 9, 13, 1), (1, 40, 33, 1), (1, 1, 1, 1), (1, 25, 7, 1)], torch.bfloat16, "raster"),
}


@pytest.mark.parametrize("case", sorted(MIXED))
def test_mixed_frame_sizes(pe, case):
    """Items of different frame sizes in one launch: each lane uses its own item's strides."""
    items, dt, order = MIXED[case]
    P, E = 14, 1280
    K = 3 * 2 * P * P
    xs = [make(1000 + i, (F, 3, h * P, ww * P), dt) for i, (t, h, ww, F) in enumerate(items)]
    x = torch.cat([a_.reshape(-1) for a_ in xs])
    w = make(1001, (E, 3, 2, P, P), torch.bfloat16, "uniform", 1 / math.sqrt(K))
    b = make(1002, (E,), torch.bfloat16, "uniform", 1 / math.sqrt(K))
    grid = [[t, h, ww] for (t, h, ww, F) in items]
    n = sum(t * h * ww for (t, h, ww) in grid)
    rows = None if n <= 3000 else sampled_rows(n, 37, 600)
    got, ref, od = run(pe, "mixed_" + case, x, w, b, grid, [F for (*_, F) in items], order=order,
                       out_dtype=torch.bfloat16, rows=rows)
    check(got, ref, od, "mixed " + case)


ADD_CASES = {
    # name: (kind, items [(t, h, w, F)] or rows N, weight dtype, out dtype, bias, in place)
    "image_splitk": ("frames", [(1, 16, 64, 1)], torch.bfloat16, torch.bfloat16, True, False),
    "images_256x128": ("frames", [(1, 32, 32, 1)] * 4, torch.bfloat16, torch.bfloat16, False, False),
    "rows_256x256": ("patches", 20000, torch.bfloat16, torch.bfloat16, True, False),
    "video_f32_out": ("frames", [(2, 8, 10, 4)], torch.bfloat16, torch.float32, True, False),
    "f32_weights": ("frames", [(1, 10, 12, 1), (1, 6, 4, 1)], torch.float32, torch.float32, True, False),
    "in_place": ("frames", [(1, 12, 20, 1)], torch.bfloat16, torch.bfloat16, True, True),
}


@pytest.mark.parametrize("case", sorted(ADD_CASES))
def test_forward_add(pe, case):
    """pe_forward_add: the PatchEmbed plus an [N, E] addend in output row order, added in fp32
    before the single rounding; the oracle adds it in fp64."""
    kind, items, wdt, od, bias, inplace = ADD_CASES[case]
    P, E = 14, 1280
    K = 3 * 2 * P * P
    w = make(1100, (E, 3, 2, P, P), wdt, "uniform", 1 / math.sqrt(K))
    b = make(1101, (E,), wdt, "uniform", 1 / math.sqrt(K)) if bias else None
    if kind == "patches":
        n = items
        x = make(1102, (n, K), wdt)
        grid, frames, order = [[1, 1, n]], None, "raster"
    else:
        xs = [make(1103 + i, (F, 3, h * P, ww * P), wdt) for i, (t, h, ww, F) in enumerate(items)]
        x = torch.cat([a_.reshape(-1) for a_ in xs])
        grid, frames, order = [[t, h, ww] for (t, h, ww, F) in items], [F for (*_, F) in items], "merge"
        n = sum(t * h * ww for (t, h, ww) in grid)
    add = make(1110, (n, E), od, "uniform", 0.5)
    rows = None if n <= 4000 else sampled_rows(n, 41, 500)
    got, ref, _ = run(pe, "add_" + case, x, w, b, grid, frames, kind=kind, order=order, out_dtype=od,
                      rows=rows, add=add, inplace=inplace)
    check(got, ref, od, "add " + case)


SPLIT_CASES = {
    # name: (kind, items [(t, h, w, F)] or rows N, with an addend); more than two rounds of 256 x 256
    # tiles with a last round under half full, rows checked around the last whole round's end
    "patch_rows": ("patches", 28160, False),
    "identical_images": ("frames", [(1, 64, 64, 1)] * 7, False),
    "mixed_images_tail_mid_item": ("frames", [(1, 72, 72, 1)] * 4 + [(1, 48, 64, 1)] * 3, False),
    "identical_images_add": ("frames", [(1, 64, 64, 1)] * 7, True),
}


@pytest.mark.parametrize("case", sorted(SPLIT_CASES))
def test_partial_last_round(pe, case):
    kind, items, with_add = SPLIT_CASES[case]
    P, E = 14, 1280
    K = 3 * 2 * P * P
    w = make(1200, (E, 3, 2, P, P), torch.bfloat16, "uniform", 1 / math.sqrt(K))
    b = make(1201, (E,), torch.bfloat16, "uniform", 1 / math.sqrt(K))
    if kind == "patches":
        n = items
        x = make(1202, (n, K), torch.bfloat16)
        grid, frames, order = [[1, 1, n]], None, "raster"
    else:
        xs = [make(1203 + i, (F, 3, h * P, ww * P), torch.bfloat16) for i, (t, h, ww, F) in enumerate(items)]
        x = torch.cat([a_.reshape(-1) for a_ in xs])
        grid, frames, order = [[t, h, ww] for (t, h, ww, F) in items], [F for (*_, F) in items], "merge"
        n = sum(t * h * ww for (t, h, ww) in grid)
    # rows around the split (the first row of the last whole-round row tile .. the end) plus a sample
    rt = (n + 255) // 256
    main_rows = (rt * 5 // 256) * 256 // 5 * 256
    near = set(range(max(0, main_rows - 300), min(n, main_rows + 300)))
    rows = np.array(sorted(near | set(sampled_rows(n, 43, 400).tolist())), dtype=np.int64)
    add = make(1210, (n, E), torch.bfloat16, "uniform", 0.5) if with_add else None
    got, ref, od = run(pe, "split_" + case, x, w, b, grid, frames, kind=kind, order=order, rows=rows, add=add)
    check(got, ref, od, "split " + case)


def test_wide_embedding_large_tiles(pe):
    """E = 4096 over 8192 patches: 512 tiles of 256 x 256 (16 column tiles), sampled rows."""
    P, E = 14, 4096
    K = 3 * 2 * P * P
    x = make(1300, (16, 3, 32 * P, 32 * P), torch.bfloat16)
    w = make(1301, (E, 3, 2, P, P), torch.bfloat16, "uniform", 1 / math.sqrt(K))
    b = make(1302, (E,), torch.bfloat16, "uniform", 1 / math.sqrt(K))
    rows = sampled_rows(8192, 47, 300)
    got, ref, od = run(pe, "e4096_video", x, w, b, [[8, 32, 32]], [16], order="merge", rows=rows)
    check(got, ref, od, "e4096 video")


@pytest.mark.parametrize("E,items,dt", [
    (65536, [(1, 4, 6, 1)], torch.bfloat16),            # the largest E pe_create accepts; split-k tiles
    (65520, [(1, 4, 6, 1)], torch.bfloat16),            # E not a multiple of 32: a ragged last column block
    (65536, [(1, 32, 64, 1)], torch.bfloat16),          # 2,048 rows: 256 x 256 tiles, 256 column tiles
    (65520, [(1, 6, 4, 1), (2, 2, 4, 3)], torch.float32),   # fp32 weight and input, an image and a video
])
def test_embedding_at_the_limit(pe, E, items, dt):
    """The widest embeddings pe_create accepts (E <= 65536, a multiple of 16), on sampled rows."""
    P = 14
    K = 3 * 2 * P * P
    xs = [make(1400 + i, (F, 3, h * P, w * P), dt) for i, (t, h, w, F) in enumerate(items)]
    x = torch.cat([a.reshape(-1) for a in xs])
    w = make(1401, (E, 3, 2, P, P), dt, "uniform", 1 / math.sqrt(K))
    b = make(1402, (E,), dt, "uniform", 1 / math.sqrt(K))
    grid = [[t, h, ww] for (t, h, ww, F) in items]
    frames = [F for (*_, F) in items]
    n = sum(t * h * ww for (t, h, ww, F) in items)
    rows = sampled_rows(n, 53, 64) if n > 64 else None
    got, ref, od = run(pe, "e%d_%s" % (E, "bf16" if dt == torch.bfloat16 else "f32"), x, w, b, grid, frames,
                       order="merge", rows=rows)
    check(got, ref, od, "E = %d" % E)


def test_many_items_split_launches(pe):
    """More items than one launch's item table holds: the library splits the launches."""
    P, E = 14, 256
    items = [(1, 2, 2 + 2 * (i % 3), 1) for i in range(150)]
    xs = [make(400 + i, (F, 3, h * P, w * P), torch.bfloat16) for i, (t, h, w, F) in enumerate(items)]
    x = torch.cat([a.reshape(-1) for a in xs])
    w = make(401, (E, 3, 2, P, P), torch.bfloat16, "uniform", 0.03)
    grid = [[t, h, ww] for (t, h, ww, F) in items]
    got, ref, od = run(pe, "150_items", x, w, None, grid, [1] * 150, order="merge")
    check(got, ref, od, "150 items")


IDENTICAL = {
    # name: item list; identical items go to one launch whatever their number, the rest of a
    # request keeps the 64-item table limit
    "200_identical_images": [(1, 4, 6, 1)] * 200,
    "70_identical_then_mixed": [(1, 4, 6, 1)] * 70 + [(1, 2, 4, 1), (2, 4, 2, 3)] + [(1, 4, 6, 1)] * 5,
    "66_identical_videos": [(2, 2, 4, 4)] * 66,
}


@pytest.mark.parametrize("case", sorted(IDENTICAL))
def test_identical_items_beyond_table(pe, case):
    items = IDENTICAL[case]
    P, E = 14, 320
    xs = [make(1400 + i, (F, 3, h * P, w * P), torch.bfloat16) for i, (t, h, w, F) in enumerate(items)]
    x = torch.cat([a.reshape(-1) for a in xs])
    w = make(1401, (E, 3, 2, P, P), torch.bfloat16, "uniform", 0.03)
    b = make(1402, (E,), torch.bfloat16, "uniform", 0.03)
    grid = [[t, h, ww] for (t, h, ww, F) in items]
    got, ref, od = run(pe, case, x, w, b, grid, [F for (*_, F) in items], order="merge")
    check(got, ref, od, case)


MERGE_SIZES = {
    # window size m: items (t, h, w, F); h and w multiples of m
    1: [(1, 3, 5, 1), (2, 2, 3, 4), (1, 7, 1, 1)],
    3: [(1, 6, 9, 1), (2, 3, 6, 3), (1, 30, 21, 1)],
    4: [(1, 8, 12, 1), (1, 4, 4, 1), (2, 4, 8, 4), (1, 32, 48, 1)],
    "3_identical": [(1, 6, 6, 1)] * 5,
}


@pytest.mark.parametrize("case", sorted(MERGE_SIZES, key=str))
def test_merge_window_sizes(pe, case):
    """Merge-window order for window sizes other than 2 (the row map takes m at run time)."""
    items = MERGE_SIZES[case]
    m = case if isinstance(case, int) else int(case.split("_")[0])
    P, E = 14, 320
    K = 3 * 2 * P * P
    xs = [make(2700 + i, (F, 3, h * P, w * P), torch.bfloat16) for i, (t, h, w, F) in enumerate(items)]
    x = torch.cat([a.reshape(-1) for a in xs])
    w = make(2701, (E, 3, 2, P, P), torch.bfloat16, "uniform", 1 / math.sqrt(K))
    b = make(2702, (E,), torch.bfloat16, "uniform", 1 / math.sqrt(K))
    grid = [[t, h, ww] for (t, h, ww, F) in items]
    frames = [F for (*_, F) in items]
    say("merge window m=%d: items %s" % (m, items if len(items) <= 4 else "%d x %s" % (len(items), items[0])))
    mod = pe.PatchEmbed(w.to(DEV), b.to(DEV), order="merge", spatial_merge_size=m)
    out = mod(x.to(DEV), grid, frames)
    torch.cuda.synchronize()
    mod.close()
    ref = oracle.forward(x, w, b, grid=grid, frames=frames, order="merge", m=m)
    check(out.double().cpu().numpy(), ref, torch.bfloat16, "merge m=%d" % m)


# ---------------------------------------------------------------------------------------------
# inputs beyond one launch's buffer range (32-bit offsets): the library splits the launch. The big
# input repeats a few seeded items with a period that does not divide the split point, so a wrong
# input or output offset in a later launch yields another item's values. The oracle runs once per
# distinct item on the sampled rows.
# ---------------------------------------------------------------------------------------------

LAUNCH_BYTES = 0xFFFFFFF0   # input bytes one launch addresses


def test_frames_beyond_launch_range(pe):
    P, E, hh, ww = 14, 1280, 72, 72
    n_img, period = 720, 7
    K = 3 * 2 * P * P
    item_elems = 3 * hh * P * ww * P
    per_launch = LAUNCH_BYTES // (item_elems * 2)           # 704 images of 1008 x 1008
    assert per_launch < n_img and per_launch % period != 0
    say("frames beyond the launch range: %d images of %dx%d, %.2f GB, split after %d" % (
        n_img, hh * P, ww * P, n_img * item_elems * 2 / 1e9, per_launch))
    imgs = [make(2600 + j, (1, 3, hh * P, ww * P), torch.bfloat16) for j in range(period)]
    w = make(2610, (E, 3, 2, P, P), torch.bfloat16, "uniform", 1 / math.sqrt(K))
    b = make(2611, (E,), torch.bfloat16, "uniform", 1 / math.sqrt(K))
    src = torch.stack([im.reshape(-1) for im in imgs]).to(DEV)
    x = src[torch.arange(n_img, device=DEV) % period].reshape(-1)
    del src
    mod = pe.PatchEmbed(w.to(DEV), b.to(DEV), order="merge")
    out = mod(x, [[1, hh, ww]] * n_img, [1] * n_img)
    torch.cuda.synchronize()
    mod.close()
    del x
    R = hh * ww
    rng = np.random.default_rng(2612)
    items = sorted({0, 1, per_launch - 2, per_launch - 1, per_launch, per_launch + 1, n_img - 1}
                   | set(rng.choice(n_img, 12, replace=False).tolist()))
    local = np.array(sorted({0, 1, 255, 256, R - 2, R - 1} | set(rng.choice(R, 20, replace=False).tolist())),
                     dtype=np.int64)
    refs = {j: oracle.forward(imgs[j], w, b, grid=[[1, hh, ww]], frames=[1], order="merge", rows=local)
            for j in sorted({i % period for i in items})}
    rows = np.concatenate([i * R + local for i in items])
    got = out[torch.as_tensor(rows, device=DEV)].double().cpu().numpy()
    del out
    torch.cuda.empty_cache()
    ref = np.concatenate([refs[i % period] for i in items])
    check(got, ref, torch.bfloat16, "frames beyond the launch range")


def test_patch_rows_beyond_launch_range(pe):
    P, E = 14, 1280
    K = 3 * 2 * P * P
    per_launch = LAUNCH_BYTES // (K * 2)                    # 1,826,091 rows of 2352 bytes
    n, period = per_launch + 73_909, 4099
    assert per_launch % period != 0
    say("patch rows beyond the launch range: %d rows, %.2f GB, split after %d" % (n, n * K * 2 / 1e9, per_launch))
    block = make(2620, (period, K), torch.bfloat16)
    w = make(2621, (E, 3, 2, P, P), torch.bfloat16, "uniform", 1 / math.sqrt(K))
    b = make(2622, (E,), torch.bfloat16, "uniform", 1 / math.sqrt(K))
    x = block.to(DEV)[torch.arange(n, device=DEV) % period]
    mod = pe.PatchEmbed(w.to(DEV), b.to(DEV))
    out = mod(x, [[1, 1, n]], kind="patches")
    torch.cuda.synchronize()
    mod.close()
    del x
    rng = np.random.default_rng(2623)
    rows = np.array(sorted({0, 1, per_launch - 2, per_launch - 1, per_launch, per_launch + 1, n - 2, n - 1}
                           | set(rng.choice(n, 200, replace=False).tolist())), dtype=np.int64)
    got = out[torch.as_tensor(rows, device=DEV)].double().cpu().numpy()
    del out
    torch.cuda.empty_cache()
    sel = block[torch.as_tensor(rows % period)]
    ref = oracle.forward(sel, w, b, grid=[[1, 1, len(rows)]], kind="patches")
    check(got, ref, torch.bfloat16, "patch rows beyond the launch range")


# ---------------------------------------------------------------------------------------------
# integer inputs: exact results (the R1 == R2 check on the "Optimize VLM PatchEmbed" page)
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("P,od", [(16, torch.float32), (14, torch.float32), (14, torch.bfloat16)])
def test_integer_inputs_exact(pe, P, od):
    N = 123
    K = 3 * 2 * P * P
    x = workloads.random_tensor((N, K), seed=120, dist="int", low=0, high=3).to(torch.bfloat16)
    w = workloads.random_tensor((1024, 3, 2, P, P), seed=121, dist="int", low=-2, high=3).to(torch.bfloat16)
    b = workloads.random_tensor((1024,), seed=122, dist="int", low=-5, high=6).to(torch.bfloat16)
    got, ref, _ = run(pe, "integers_P%d" % P, x, w, b, [[1, 1, N]], kind="patches", out_dtype=od)
    assert np.abs(ref).max() < 2 ** 24
    if od == torch.float32:
        assert np.array_equal(got, ref)
    else:
        want = torch.from_numpy(ref).to(torch.float32).to(torch.bfloat16).double().numpy()
        assert np.array_equal(got, want)


def test_integer_frames_exact_merge_order(pe):
    """Integer frames with a per-patch code make any row-order or gather mistake an exact miss."""
    P, t, h, w, F = 14, 2, 4, 6, 4
    x = workloads.random_tensor((F, 3, h * P, w * P), seed=130, dist="int", low=0, high=3).to(torch.bfloat16)
    wt = workloads.random_tensor((64, 3, 2, P, P), seed=131, dist="int", low=-2, high=3).to(torch.bfloat16)
    got, ref, _ = run(pe, "integer_frames_merge", x, wt, None, [[t, h, w]], [F], order="merge",
                      out_dtype=torch.float32)
    assert np.array_equal(got, ref)


# ---------------------------------------------------------------------------------------------
# single images staged through LDS (opt-in stage_images; bf16, P = 14, one frame size, large
# tiles): each wave loads whole pixel rows of 32 patches, the waves share them through LDS in the
# grouped k order. Every case checks first which path the plan runs it on.
# ---------------------------------------------------------------------------------------------

STAGED = {
    # name: items (h, w) of single images, merge size (0 = raster), E, out dtype, bias, fused add
    # (frame_sizes_differ: mixed frame sizes keep the register gather)
    "raster_ragged": ([(58, 142)], 0, 1280, torch.bfloat16, True, False),        # 8236 rows: tail of 44
    "merge2_ragged": ([(60, 138)], 2, 1280, torch.bfloat16, True, False),
    "merge4": ([(64, 120)], 4, 1280, torch.bfloat16, False, False),
    "merge3": ([(63, 126)], 3, 1280, torch.bfloat16, True, False),               # windows straddle waves
    "tiles_256x128": ([(64, 64)], 2, 1280, torch.bfloat16, True, False),
    "frame_sizes_differ": ([(40, 60), (36, 72), (50, 50), (2, 2)], 2, 1280, torch.bfloat16, True, False),
    "f32_out_e1152": ([(60, 140)], 2, 1152, torch.float32, True, False),
    "fused_add": ([(58, 142)], 2, 1280, torch.bfloat16, True, True),
    "identical_images": ([(36, 36)] * 9, 2, 1280, torch.bfloat16, True, False),
}


@pytest.mark.parametrize("case", sorted(STAGED))
def test_staged_images(pe, case):
    """stage_images = 1 against the oracle, and the same request on the default path."""
    items, m, E, od, bias, add = STAGED[case]
    P = 14
    K = 3 * 2 * P * P
    xs = [make(3300 + i, (1, 3, h * P, w * P), torch.bfloat16) for i, (h, w) in enumerate(items)]
    x = torch.cat([a.reshape(-1) for a in xs])
    w = make(3301, (E, 3, 2, P, P), torch.bfloat16, "uniform", 1 / math.sqrt(K))
    b = make(3302, (E,), torch.bfloat16, "uniform", 1 / math.sqrt(K)) if bias else None
    grid = [[1, h, ww] for (h, ww) in items]
    frames = [1] * len(items)
    n = sum(h * ww for (h, ww) in items)
    order = "merge" if m else "raster"
    addend = make(3303, (n, E), od) if add else None
    say("staged images %s: %d items, %d rows, m=%d, E=%d, out=%s, add=%s" % (case, len(items), n, m, E, od, add))
    mod = pe.PatchEmbed(w.to(DEV), b.to(DEV) if b is not None else None, order=order, out_dtype=od,
                        spatial_merge_size=m or 2, stage_images=True)
    plan = mod.plan(grid, frames)
    want = "images" if case == "frame_sizes_differ" else "images_lds"
    assert [L["a_mode"] for L in plan] == [want], plan
    if add:
        out = mod(x.to(DEV), grid, frames, add=addend.to(DEV))
    else:
        out = mod(x.to(DEV), grid, frames)
    torch.cuda.synchronize()
    mod.close()
    ref = oracle.forward(x, w, b, grid=grid, frames=frames, order=order, m=m or 2, addend=addend)
    check(out.double().cpu().numpy(), ref, od, "staged " + case)
    # the default path on the same request: the same sums in another k order
    mod = pe.PatchEmbed(w.to(DEV), b.to(DEV) if b is not None else None, order=order, out_dtype=od,
                        spatial_merge_size=m or 2)
    assert [L["a_mode"] for L in mod.plan(grid, frames)] == ["images"]
    out2 = mod(x.to(DEV), grid, frames, add=addend.to(DEV)) if add else mod(x.to(DEV), grid, frames)
    torch.cuda.synchronize()
    mod.close()
    check(out2.double().cpu().numpy(), ref, od, "default " + case)


def test_staged_images_integer_exact(pe):
    """Integer pixels and weights: the staged path's sums are exact, so a fragment staged to the
    wrong slot, or a grouped weight out of step with it, is an exact miss."""
    P, h, w = 14, 60, 138
    x = workloads.random_tensor((1, 3, h * P, w * P), seed=3310, dist="int", low=0, high=3).to(torch.bfloat16)
    wt = workloads.random_tensor((256, 3, 2, P, P), seed=3311, dist="int", low=-2, high=3).to(torch.bfloat16)
    say("staged images, integer inputs, %d rows" % (h * w))
    mod = pe.PatchEmbed(wt.to(DEV), None, order="merge", out_dtype=torch.float32, stage_images=True)
    assert [L["a_mode"] for L in mod.plan([[1, h, w]], [1])] == ["images_lds"]
    out = mod(x.to(DEV), [[1, h, w]], [1])
    torch.cuda.synchronize()
    mod.close()
    ref = oracle.forward(x, wt, None, grid=[[1, h, w]], frames=[1], order="merge")
    assert np.array_equal(out.double().cpu().numpy(), ref)


# ---------------------------------------------------------------------------------------------
# poisoned pixels: a NaN or an Inf makes exactly the rows of its own patch non-finite. A load that
# reached past a patch's pixels (even against a zero weight: NaN * 0 is NaN) would poison others.
# ---------------------------------------------------------------------------------------------

POISON = {
    # name: P, items (t, h, w, F), input kind, order, in/weight dtype, staged images, E
    "images_merge": (14, [(1, 12, 20, 1), (1, 8, 8, 1)], "frames", "merge", torch.bfloat16, False, 1280),
    "images_large_tiles": (14, [(1, 64, 64, 1)], "frames", "merge", torch.bfloat16, False, 1280),
    "images_staged": (14, [(1, 64, 64, 1)], "frames", "merge", torch.bfloat16, True, 1280),
    "video_raster": (14, [(4, 10, 12, 7)], "frames", "raster", torch.bfloat16, False, 640),
    "p16_images": (16, [(1, 10, 14, 1)], "frames", "raster", torch.bfloat16, False, 1152),
    "patch_rows": (14, [(1, 1, 3000)], "patches", "raster", torch.bfloat16, False, 1280),
    "fp32_frames": (14, [(1, 6, 8, 1), (2, 4, 2, 4)], "frames", "merge", torch.float32, False, 640),
}


@pytest.mark.parametrize("case", sorted(POISON))
def test_poisoned_pixels_stay_in_their_patch(pe, case):
    P, items, kind, order, dt, staged, E = POISON[case]
    K = 3 * 2 * P * P
    rng = np.random.default_rng(5100)
    w = make(5101, (E, 3, 2, P, P), dt, "uniform", 1 / math.sqrt(K))
    b = make(5102, (E,), dt, "uniform", 1 / math.sqrt(K))
    if kind == "patches":
        n = items[0][2]
        x = make(5103, (n, K), dt)
        grid, frames = [[1, 1, n]], None
        # a row's first and last elements, and one in the middle of another row
        for r, k in ((5, 0), (5, K - 1), (777, K // 2), (n - 1, K - 1)):
            x[r, k] = float("nan") if r != 777 else float("inf")
    else:
        xs = [make(5103 + i, (F, 3, h * P, ww * P), dt) for i, (t, h, ww, F) in enumerate(items)]
        # per item: a few patches, each poisoned at one pixel on its edge (px 0 or P - 1, pixel
        # row P - 1) in some channel and frame
        for (t, h, ww, F), xi in zip(items, xs):
            for _ in range(3):
                f, c = int(rng.integers(F)), int(rng.integers(3))
                hp, wp = int(rng.integers(h)), int(rng.integers(ww))
                py, px = [(0, 0), (0, P - 1), (P - 1, 0), (P - 1, P - 1)][int(rng.integers(4))]
                xi[f, c, hp * P + py, wp * P + px] = float("nan") if rng.random() < 0.5 else float("inf")
        x = torch.cat([a.reshape(-1) for a in xs])
        grid = [[t, h, ww] for (t, h, ww, F) in items]
        frames = [F for (*_, F) in items]
    say("poisoned pixels %s: %s" % (case, grid if len(grid) < 4 else "%d items" % len(grid)))
    mod = pe.PatchEmbed(w.to(DEV), b.to(DEV), order=order, stage_images=staged)
    if staged:
        assert [L["a_mode"] for L in mod.plan(grid, frames)] == ["images_lds"]
    out = mod(x.to(DEV), grid, frames, kind=kind)
    torch.cuda.synchronize()
    mod.close()
    got = out.double().cpu().numpy()
    ref = oracle.forward(x, w, b, grid=grid, frames=frames, kind=kind, order=order)
    poisoned = ~np.isfinite(ref).all(axis=1)
    assert poisoned.any() and not poisoned.all()
    # the poisoned patches' rows are non-finite wherever the oracle's are; every other row is finite
    # and within tolerance
    assert np.array_equal(~np.isfinite(got).all(axis=1), poisoned)
    check(got[~poisoned], ref[~poisoned], dt, "poisoned " + case)


# ---------------------------------------------------------------------------------------------
# empty input and error paths (validated before any launch)
# ---------------------------------------------------------------------------------------------

def test_empty_batch(pe):
    say("empty batch")
    w = make(500, (64, 3, 2, 14, 14), torch.bfloat16).to(DEV)
    mod = pe.PatchEmbed(w, order="merge")
    out = mod(torch.empty(0, dtype=torch.bfloat16, device=DEV), [])
    torch.cuda.synchronize()
    assert tuple(out.shape) == (0, 64) and mod.plan([]) == []
    # the binding returns the empty result itself; the C ABI calls 0 items (N = 0) a shape error
    assert pe.lib.pe_forward(mod._h, 1, 0x1000, 1, None, None, 0, 0x2000, None) == pe.PE_ERR_SHAPE
    assert pe.lib.pe_forward_plan(mod._h, 1, 1, None, None, 0, None, 0) == pe.PE_ERR_SHAPE
    mod.close()


def test_forward_error_paths(pe):
    import ctypes
    say("error paths")
    w = make(501, (64, 3, 2, 14, 14), torch.bfloat16).to(DEV)
    mod = pe.PatchEmbed(w, order="merge")
    h = mod._h
    g = lambda *v: (ctypes.c_int32 * len(v))(*v)
    X, O = 0x1000, 0x2000   # never dereferenced: every call below fails validation first
    # bf16 input on an fp32 weight is the unsupported dtype pair (fp32 input on a bf16 weight is
    # supported, so it must not be called with these fake pointers)
    w32 = make(503, (64, 3, 2, 14, 14), torch.float32).to(DEV)
    mod32 = pe.PatchEmbed(w32, order="merge")
    assert pe.lib.pe_forward(mod32._h, 1, X, 1, g(1, 2, 2), None, 1, O, None) == pe.PE_ERR_UNSUPPORTED
    assert "supported are" in pe.last_error()
    mod32.close()
    assert pe.lib.pe_forward(h, 1, X, 1, g(1, 2, 3), None, 1, O, None) == pe.PE_ERR_SHAPE        # odd w
    assert pe.lib.pe_forward(h, 1, X, 1, g(1, 2, 2), g(3), 1, O, None) == pe.PE_ERR_SHAPE        # F vs t
    assert pe.lib.pe_forward(h, 1, X, 1, g(1, -2, 2), None, 1, O, None) == pe.PE_ERR_SHAPE
    assert pe.lib.pe_forward(h, 7, X, 1, g(1, 2, 2), None, 1, O, None) == pe.PE_ERR_INVALID_ARG
    assert pe.lib.pe_forward(h, 1, None, 1, g(1, 2, 2), None, 1, O, None) == pe.PE_ERR_INVALID_ARG
    assert pe.lib.pe_forward(h, 1, X, 1, g(1, 2, 2), None, -1, O, None) == pe.PE_ERR_INVALID_ARG
    # one item of frames beyond the 4 GiB launch range
    assert pe.lib.pe_forward(h, 1, X, 1, g(1, 2000, 2000), g(1), 1, O, None) == pe.PE_ERR_UNSUPPORTED
    assert "4 GiB" in pe.last_error()
    # an item of 2^31 rows or more, also where t*h*w and its pixel count overflow 64 bits
    big = 2 ** 31 - 1
    for grid in ((1, 65536, 32768), (2 ** 30, big - 1, big - 1), (big, big, big)):
        assert pe.lib.pe_forward(h, 1, X, 1, g(*grid), None, 1, O, None) == pe.PE_ERR_SHAPE, grid
        assert "2^31 rows" in pe.last_error()
        assert pe.lib.pe_forward(h, 0, X, 1, g(*grid), None, 1, O, None) == pe.PE_ERR_SHAPE, grid
    # frames == NULL: a video of t = 2^30 temporal patches has 2^31 frames (counted in 64 bits)
    mod_r = pe.PatchEmbed(w, order="raster")
    assert pe.lib.pe_forward(mod_r._h, 1, X, 1, g(2 ** 30, 1, 1), None, 1, O, None) == pe.PE_ERR_UNSUPPORTED
    assert "4 GiB" in pe.last_error()
    mod_r.close()
    with pytest.raises(pe.PEError):
        mod(torch.zeros(10, dtype=torch.bfloat16, device=DEV), [[1, 2, 2]])   # wrong input size
    mod.close()


def test_graph_replays_match_eager(pe):
    """The benchmark replays captured launches: every replay must equal the eager result, with
    eager work and synchronisations between replays."""
    wl = workloads.WORKLOADS[2]
    x, w, b = workloads.generate(wl)
    say("graph replay of %s" % wl.name)
    mod = pe.PatchEmbed(w.to(DEV), None, order=wl.order)
    xd = x.to(DEV)
    eager = mod(xd, list(wl.grid), list(wl.frames))
    torch.cuda.synchronize()
    out = torch.empty_like(eager)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(3):
            mod(xd, list(wl.grid), list(wl.frames), out=out)
    for rep in range(4):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), "replay %d differs" % rep
        other = mod(xd, list(wl.grid), list(wl.frames))     # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(other, eager)
    mod.close()


def test_forward_plan_names_the_launches(pe):
    """pe_forward_plan on a live handle: the launches the benchmark reports for each workload, and
    the same request checks and codes as pe_forward."""
    say("pe_forward_plan on workloads 1-6 and on bad requests")
    expect = {1: ("pe_fwd16_kernel", 1), 2: ("pe_fwd32_sk_kernel", 1), 3: ("pe_fwd32_sk_kernel", 1),
              4: ("pe_fwd32_kernel", 1), 5: ("pe_fwd32_kernel", 1), 6: ("pe_fwd32_kernel", 1)}
    for idx, (kname, nl) in expect.items():
        wl = workloads.WORKLOADS[idx]
        _, w, b = workloads.generate(wl)
        mod = pe.PatchEmbed(w.to(DEV), b.to(DEV) if b is not None else None, order=wl.order,
                            out_dtype=workloads.DTYPES[wl.out_dtype])
        plan = mod.plan(list(wl.grid), list(wl.frames) or None, kind=wl.kind,
                        in_dtype=workloads.DTYPES[wl.in_dtype])
        assert [L["kernel"] for L in plan] == [kname] * nl, (idx, plan)
        assert sum(L["n_rows"] for L in plan) == sum(t * h * ww for (t, h, ww) in wl.grid)
        if idx == 5:
            assert plan[0]["tile"] == [256, 256] and plan[0]["workgroups"] == 6480 and plan[0]["a_mode"] == "images"
        if idx == 2:
            assert plan[0]["tile"] == [32, 160] and plan[0]["workgroups"] == 256
        if wl.order == "merge":
            with pytest.raises(pe.PEError) as e1:
                mod.plan([[1, 3, 5]], [1])           # merge order needs even h and w (frames)
            assert e1.value.code == pe.PE_ERR_SHAPE
        with pytest.raises(pe.PEError) as e2:
            mod.plan([[2, 4, 4]], [1])               # one frame cannot make two temporal patches
        assert e2.value.code == pe.PE_ERR_SHAPE
        mod.close()


def test_call_on_a_side_stream(pe):
    """stream= names a stream other than the current one: the output and the input's contiguous copy
    that the binding allocates are marked as used on that stream, and the result is right."""
    say("PatchEmbed on a side stream, non-contiguous input, binding-allocated output")
    P, E = 14, 256
    g = [[1, 6, 8]]
    x = workloads.random_tensor((3, 6 * P, 8 * P), seed=8100, dtype=torch.bfloat16)
    w = workloads.random_tensor((E, 3, 2, P, P), seed=8101, dtype=torch.bfloat16, dist="uniform", bound=0.03)
    mod = pe.PatchEmbed(w.to(DEV), None, order="merge")
    side = torch.cuda.Stream(device=DEV)
    xt = x.to(DEV).transpose(1, 2).contiguous().transpose(1, 2)   # same values, not contiguous
    assert not xt.is_contiguous()
    torch.cuda.synchronize()
    out = mod(xt, g, [1], stream=side.cuda_stream)
    side.synchronize()
    got = out.float().cpu().double().numpy()
    ref = oracle.forward(x, w, None, grid=g, frames=[1], order="merge")
    check(got, ref, torch.bfloat16, "side stream")
    mod.close()
