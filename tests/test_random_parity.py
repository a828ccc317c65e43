"""GPU parity over seeded random valid requests: patch size, embed width, bias, dtypes, row order,
items (images, videos, odd frame counts, mixed frame sizes), patch rows, the fused add and the
approximate image fold, each against the fp64 oracle with the bounds of the other parity tests.
The cases are drawn once from a fixed seed, so every run checks the same ones."""
import math
import random

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


def draw_cases(n, seed=20261203):
    rnd = random.Random(seed)
    cases = []
    for i in range(n):
        P = rnd.choice([14, 16])
        E = 16 * rnd.choice([1, 3, 8, 20, 64, 72, 80])
        wdt = rnd.choice(["bf16"] * 5 + ["f32"])
        if wdt == "f32":
            idt, odt = "f32", "f32"
        else:
            idt = rnd.choice(["bf16"] * 3 + ["f32"])
            odt = rnd.choice(["bf16"] * 3 + ["f32"])
        kind = rnd.choice(["frames"] * 4 + ["patches"])
        order = rnd.choice(["raster", "merge"])
        items = []
        if kind == "frames":
            for _ in range(rnd.randint(1, 5)):
                h, w = 2 * rnd.randint(1, 12), 2 * rnd.randint(1, 12)
                if rnd.random() < 0.6:
                    items.append((1, h, w, 1))
                else:
                    t = rnd.randint(1, 3)
                    F = rnd.choice([2 * t, 2 * t - 1]) if t > 1 else 2
                    items.append((t, h, w, F))
        rows = rnd.randint(1, 3000)
        bias = rnd.random() < 0.5
        add = rnd.random() < 0.3
        fold = wdt == "bf16" and kind == "frames" and rnd.random() < 0.3
        cases.append(dict(i=i, P=P, E=E, wdt=wdt, idt=idt, odt=odt, kind=kind, order=order, items=items,
                          rows=rows, bias=bias, add=add, fold=fold))
    return cases


CASES = draw_cases(40)
DT = {"bf16": torch.bfloat16, "f32": torch.float32}


@pytest.mark.parametrize("c", CASES, ids=["case%02d" % c["i"] for c in CASES])
def test_random_request(pe, c):
    P, E = c["P"], c["E"]
    K = 3 * 2 * P * P
    seed = 7000 + 10 * c["i"]
    wdt, idt, odt = DT[c["wdt"]], DT[c["idt"]], DT[c["odt"]]
    w = workloads.random_tensor((E, 3, 2, P, P), seed=seed, dtype=wdt, dist="uniform", bound=1 / math.sqrt(K))
    b = workloads.random_tensor((E,), seed=seed + 1, dtype=wdt, dist="uniform", bound=1 / math.sqrt(K)) if c["bias"] else None
    if c["kind"] == "patches":
        n = c["rows"]
        x = workloads.random_tensor((n, K), seed=seed + 2, dtype=idt)
        grid, frames, order = [[1, 1, n]], None, "raster"
    else:
        items = c["items"]
        x = torch.cat([workloads.random_tensor((F, 3, h * P, ww * P), seed=seed + 3 + j, dtype=idt).reshape(-1)
                       for j, (t, h, ww, F) in enumerate(items)])
        grid, frames, order = [[t, h, ww] for (t, h, ww, F) in items], [F for (*_, F) in items], c["order"]
        n = sum(t * h * ww for (t, h, ww) in grid)
    add = workloads.random_tensor((n, E), seed=seed + 9, dtype=odt, dist="uniform", bound=0.5) if c["add"] else None
    print("[case] random %02d: P%d E%d w=%s in=%s out=%s %s %s rows=%d items=%s bias=%s add=%s fold=%s" % (
        c["i"], P, E, c["wdt"], c["idt"], c["odt"], c["kind"], order, n, c["items"], c["bias"], c["add"], c["fold"]),
        flush=True)
    mod = pe.PatchEmbed(w.to(DEV), b.to(DEV) if b is not None else None, order=order, out_dtype=odt,
                        image_fold=c["fold"])
    out = mod(x.to(DEV), grid, frames, kind=c["kind"], add=add.to(DEV) if add is not None else None)
    torch.cuda.synchronize()
    mod.close()
    got = out.double().cpu().numpy()
    cast = None if idt == wdt else "bf16"
    ref = oracle.forward(x, w, b, grid=grid, frames=frames, kind=c["kind"], order=order, cast_input_to=cast,
                         addend=add)
    if odt == torch.bfloat16:
        tol = 1e-3 + 1e-2 * np.abs(ref)
    else:
        tol = np.full(ref.shape, 5e-4)
    if c["fold"]:
        # image rows: plus the folded weight's rounding, 2^-8 of sum_k |x_k| |W0_k + W1_k|
        wd = oracle._f64(w)
        wabs = np.zeros_like(wd)
        wabs[:, :, 0] = np.abs(wd[:, :, 0] + wd[:, :, 1])
        fb = oracle.forward(np.abs(oracle.round_to(x, "bf16")), wabs, None, grid=grid, frames=frames, order=order)
        pos = oracle.row_positions(grid, frames, order=order, m=2)
        img = np.array([f == 1 for f in frames])[pos[:, 0]]
        tol = tol + np.where(img[:, None], 1.01 * 2.0 ** -8 * fb, 0.0)
    assert np.all(np.isfinite(got))
    err = np.abs(got - ref)
    bad = err > tol
    assert not bad.any(), "case %d: %d of %d outside (max err %.3g, max err/bound %.3g)" % (
        c["i"], bad.sum(), bad.size, err.max(), (err / tol).max())


def draw_grouping_cases(n, seed=20261204):
    """Requests aimed at the launch grouping: long item lists (past the 64-entry item table), runs
    of identical items broken by different ones, images and videos interleaved, with and without
    the approximate image fold."""
    rnd = random.Random(seed)
    cases = []
    for i in range(n):
        P = rnd.choice([14, 16])
        E = 16 * rnd.choice([2, 5, 12])
        items = []
        while len(items) < rnd.randint(20, 150):
            h, w = 2 * rnd.randint(1, 4), 2 * rnd.randint(1, 4)
            if rnd.random() < 0.7:
                it = (1, h, w, 1)
            else:
                t = rnd.randint(1, 2)
                it = (t, h, w, rnd.choice([2 * t, 2 * t - 1]) if t > 1 else 2)
            items += [it] * rnd.choice([1, 1, 2, 5, 30, 70])
        fold = rnd.random() < 0.4
        cases.append(dict(i=i, P=P, E=E, items=items, fold=fold, order=rnd.choice(["raster", "merge"]),
                          bias=rnd.random() < 0.5))
    return cases


GROUPING = draw_grouping_cases(12)


@pytest.mark.parametrize("c", GROUPING, ids=["group%02d" % c["i"] for c in GROUPING])
def test_random_launch_grouping(pe, c):
    P, E, items = c["P"], c["E"], c["items"]
    K = 3 * 2 * P * P
    seed = 9000 + 10 * c["i"]
    w = workloads.random_tensor((E, 3, 2, P, P), seed=seed, dtype=torch.bfloat16, dist="uniform", bound=1 / math.sqrt(K))
    b = workloads.random_tensor((E,), seed=seed + 1, dtype=torch.bfloat16, dist="uniform",
                                bound=1 / math.sqrt(K)) if c["bias"] else None
    sizes = [F * 3 * (h * P) * (ww * P) for (t, h, ww, F) in items]
    x = workloads.random_tensor((sum(sizes),), seed=seed + 2, dtype=torch.bfloat16)
    grid, frames = [[t, h, ww] for (t, h, ww, F) in items], [F for (*_, F) in items]
    n = sum(t * h * ww for (t, h, ww) in grid)
    print("[case] grouping %02d: P%d E%d %d items, %d rows, order=%s fold=%s bias=%s" % (
        c["i"], P, E, len(items), n, c["order"], c["fold"], c["bias"]), flush=True)
    mod = pe.PatchEmbed(w.to(DEV), b.to(DEV) if b is not None else None, order=c["order"], image_fold=c["fold"])
    out = mod(x.to(DEV), grid, frames)
    torch.cuda.synchronize()
    mod.close()
    # every item's first and last rows, plus a seeded sample
    starts = np.cumsum([0] + [t * h * ww for (t, h, ww) in grid])
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(n, min(n, 400), replace=False).tolist())
    for s0, s1 in zip(starts[:-1], starts[1:]):
        rows.update((int(s0), int(s1) - 1))
    rows = np.array(sorted(rows), dtype=np.int64)
    got = out[torch.as_tensor(rows, device=DEV)].double().cpu().numpy()
    ref = oracle.forward(x, w, b, grid=grid, frames=frames, order=c["order"], rows=rows)
    tol = 1e-3 + 1e-2 * np.abs(ref)
    if c["fold"]:
        wd = oracle._f64(w)
        wabs = np.zeros_like(wd)
        wabs[:, :, 0] = np.abs(wd[:, :, 0] + wd[:, :, 1])
        fb = oracle.forward(np.abs(oracle.round_to(x, "bf16")), wabs, None, grid=grid, frames=frames,
                            order=c["order"], rows=rows)
        pos = oracle.row_positions(grid, frames, order=c["order"], m=2)
        img = np.array([f == 1 for f in frames])[pos[rows, 0]]
        tol = tol + np.where(img[:, None], 1.01 * 2.0 ** -8 * fb, 0.0)
    err = np.abs(got - ref)
    bad = err > tol
    assert np.all(np.isfinite(got))
    assert not bad.any(), "grouping case %d: %d of %d outside (max err/bound %.3g)" % (
        c["i"], bad.sum(), bad.size, (err / tol).max())
