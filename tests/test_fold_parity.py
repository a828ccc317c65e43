"""GPU parity of the opt-in approximate image fold (pe_config.image_fold = 1) against the fp64 oracle.

An image item's output is x . (W0 + W1) over one frame; the fold mode rounds W0 + W1 to bf16 once
and runs half the matrix work. The oracle stays the exact Conv3d. Bound, per output of an image
row, from the arithmetic: the exact path's bf16 bound (1e-3 + 1e-2 |ref|) plus the folded weight's
rounding, |RNE(W0 + W1) - (W0 + W1)| <= 2^-8 |W0 + W1| per element (bf16 keeps 8 significant bits;
the fp32 sum before the rounding is exact for bf16 operands within 2^16 of each other, else off by
at most 2^-24 of it), i.e. 1.01 * 2^-8 * sum_k |x_k| |W0_k + W1_k|. That sum is the oracle's PatchEmbed
of |x| with the weight |W0 + W1| in the first temporal slot and zero in the second. Video rows take
the exact path and the exact bound.
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


def make(seed, shape, dtype, dist="normal", bound=1.0):
    return workloads.random_tensor(shape, seed=seed, dtype=dtype, dist=dist, bound=bound)


def fold_bound(x, w, grid, frames, order, rows=None):
    """sum_k |x_k| |W0_k + W1_k| per output (fp64), through the oracle's own PatchEmbed."""
    wd = oracle._f64(w)
    wabs = np.zeros_like(wd)
    wabs[:, :, 0] = np.abs(wd[:, :, 0] + wd[:, :, 1])
    xa = np.abs(oracle.round_to(x, "bf16"))
    return oracle.forward(xa, wabs, None, grid=grid, frames=frames, order=order, rows=rows)


def image_row_mask(grid, frames, order, rows=None):
    pos = oracle.row_positions(grid, frames, order=order, m=2)
    is_img = np.array([f == 1 for f in frames])[pos[:, 0]]
    return is_img if rows is None else is_img[rows]


def run_fold(pe, name, x, w, b, grid, frames, order, out_dtype=torch.bfloat16, rows=None):
    say("fold %s: grid=%s frames=%s x=%s w=%s bias=%s out=%s rows=%s" % (
        name, grid if len(grid) <= 4 else "%d items" % len(grid), frames if len(frames) <= 4 else "...",
        tuple(x.shape), tuple(w.shape), b is not None, out_dtype, None if rows is None else len(rows)))
    wd, bd = w.to(DEV), (b.to(DEV) if b is not None else None)
    xd = x.to(DEV)
    mod = pe.PatchEmbed(wd, bd, order=order, out_dtype=out_dtype, image_fold=True)
    exact = pe.PatchEmbed(wd, bd, order=order, out_dtype=out_dtype)
    out = mod(xd, grid, frames)
    out_exact = exact(xd, grid, frames)
    torch.cuda.synchronize()
    mod.close()
    exact.close()
    sel = torch.as_tensor(rows, device=DEV) if rows is not None else None
    got = (out[sel] if sel is not None else out).double().cpu().numpy()
    got_exact = (out_exact[sel] if sel is not None else out_exact).double().cpu().numpy()
    cast = "bf16" if x.dtype != torch.bfloat16 else None
    ref = oracle.forward(x, w, b, grid=grid, frames=frames, order=order, rows=rows, cast_input_to=cast)
    img = image_row_mask(grid, frames, order, rows)
    fb = fold_bound(x, w, grid, frames, order, rows)
    return got, got_exact, ref, img, fb


def check_fold(got, got_exact, ref, img, fb, out_dtype, what):
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    err = np.abs(got - ref)
    if out_dtype == torch.bfloat16:
        base = 1e-3 + 1e-2 * np.abs(ref)
    else:
        base = np.full(ref.shape, 5e-4)
    tol = base + np.where(img[:, None], 1.01 * 2.0 ** -8 * fb, 0.0)
    bad = err > tol
    assert not bad.any(), "%s: %d of %d outside the fold bound (max err %.3g, max err/bound %.3g)" % (
        what, bad.sum(), bad.size, err.max(), (err / tol).max())
    # video rows are the exact kernel's, bit for bit
    if (~img).any():
        assert np.array_equal(got[~img], got_exact[~img]), what + ": video rows differ from the exact path"
    # image rows did take the folded weight
    if img.any():
        assert not np.array_equal(got[img], got_exact[img]), what + ": image rows equal the exact path"
    e_img = err[img].max() if img.any() else 0.0
    print("%s: max err %.3g on image rows (bound max %.3g)" % (what, e_img, tol[img].max() if img.any() else 0.0),
          flush=True)


CASES = [
    # name, P, E, items [(t, h, w, F)], order, input dtype, out dtype, bias
    ("one_image_224x896", 14, 1280, [(1, 16, 64, 1)], "merge", torch.bfloat16, torch.bfloat16, False),
    ("four_images_448", 14, 1280, [(1, 32, 32, 1)] * 4, "merge", torch.bfloat16, torch.bfloat16, True),
    ("p16_e1152_bias", 16, 1152, [(1, 28, 28, 1)], "raster", torch.bfloat16, torch.bfloat16, True),
    ("images_and_video", 14, 640, [(1, 8, 10, 1), (2, 6, 4, 4), (1, 4, 6, 1)], "merge",
     torch.bfloat16, torch.bfloat16, True),
    ("mixed_sizes", 14, 1280, [(1, 24, 40, 1), (1, 12, 16, 1), (1, 2, 2, 1), (1, 30, 18, 1)], "merge",
     torch.bfloat16, torch.bfloat16, True),
    ("f32_input", 14, 512, [(1, 10, 14, 1), (1, 6, 6, 1)], "raster", torch.float32, torch.bfloat16, False),
    ("f32_out", 14, 1280, [(1, 16, 20, 1)], "merge", torch.bfloat16, torch.float32, True),
    ("p16_mixed_sizes_video", 16, 1024, [(1, 16, 16, 1), (1, 24, 32, 1), (2, 16, 16, 4)], "merge",
     torch.bfloat16, torch.bfloat16, True),
    ("e48_ragged", 14, 48, [(1, 5, 7, 1)], "raster", torch.bfloat16, torch.bfloat16, True),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_image_fold(pe, case):
    name, P, E, items, order, dt, od, bias = case
    K = 3 * 2 * P * P
    xs = [make(4000 + i, (F, 3, h * P, w * P), dt) for i, (t, h, w, F) in enumerate(items)]
    x = torch.cat([a.reshape(-1) for a in xs])
    w = make(4100, (E, 3, 2, P, P), torch.bfloat16, "uniform", 1 / math.sqrt(K))
    b = make(4101, (E,), torch.bfloat16, "uniform", 1 / math.sqrt(K)) if bias else None
    grid = [[t, h, ww] for (t, h, ww, F) in items]
    frames = [F for (*_, F) in items]
    got, got_exact, ref, img, fb = run_fold(pe, name, x, w, b, grid, frames, order, od)
    check_fold(got, got_exact, ref, img, fb, od, name)


def test_image_fold_batch64_sampled(pe):
    """The 64 x 1008^2 batch (the large-tile kernels) in fold mode, sampled rows."""
    wl = workloads.WORKLOADS[5]
    x, w, b = workloads.generate(wl)
    rng = np.random.default_rng(55)
    n = 331776
    rows = np.array(sorted(set(rng.choice(n, 600, replace=False).tolist()) | {0, 255, 256, n - 1}), dtype=np.int64)
    grid, frames = [list(g) for g in wl.grid], list(wl.frames)
    got, got_exact, ref, img, fb = run_fold(pe, wl.name, x, w, b, grid, frames, wl.order, rows=rows)
    check_fold(got, got_exact, ref, img, fb, torch.bfloat16, wl.name)


def test_fold_off_by_default_and_video_only_unchanged(pe):
    """Without image_fold the handle is exact (the other parity tests); with it, a call of videos
    only gives exactly the exact handle's output."""
    P, E = 14, 512
    K = 3 * 2 * P * P
    items = [(2, 6, 8, 4), (1, 4, 4, 2)]
    x = torch.cat([make(4200 + i, (F, 3, h * P, w * P), torch.bfloat16).reshape(-1)
                   for i, (t, h, w, F) in enumerate(items)])
    w = make(4201, (E, 3, 2, P, P), torch.bfloat16, "uniform", 1 / math.sqrt(K))
    say("fold: videos only")
    wd = w.to(DEV)
    a = pe.PatchEmbed(wd, order="merge", image_fold=True)
    e = pe.PatchEmbed(wd, order="merge")
    grid = [[t, h, ww] for (t, h, ww, F) in items]
    frames = [F for (*_, F) in items]
    o1 = a(x.to(DEV), grid, frames)
    o2 = e(x.to(DEV), grid, frames)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    a.close()
    e.close()
