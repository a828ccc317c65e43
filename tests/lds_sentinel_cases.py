"""Parity cases on the LDS sentinel debug build (run by tests/test_lds_sentinel.py in a process of
its own, with PE_LIB_PATH naming libpe_sentinel.so).

In that build every kernel that uses LDS fills it with NaN bytes before its first use
(csrc/pe_device.h, lds_sentinel_fill), so a read of an LDS slot the workgroup has not written yet
gives a NaN in the output instead of a stale finite value. The cases below run every LDS path of
the library (the weight stages and the epilogue of the large-tile kernel, its staged A for patch
rows and for single images, the split-k kernel's partial sums, the fp32 kernel), with ragged
tails, tiles that straddle items and the fused add, and compare each output, all rows or sampled
rows, with the oracle at the parity tolerances. Exits non-zero at the first failure.
"""
import math
import os
import sys

import numpy as np
import torch

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import vlm_vision_patch_amd as pe  # noqa: E402
from test_parity import DEV, check, make, sampled_rows  # noqa: E402

import oracle  # noqa: E402


def case(name, x, w, b, grid, frames=None, kind="frames", order="merge", out_dtype=None, rows=None,
         add=None, stage=False, want_kernel=None, want_mode=None):
    out_dtype = out_dtype or w.dtype
    print("[case] %s" % name, flush=True)
    mod = pe.PatchEmbed(w.to(DEV), b.to(DEV) if b is not None else None, order=order, out_dtype=out_dtype,
                        stage_images=stage)
    plan = mod.plan(grid, frames, kind=kind)
    if want_kernel is not None:
        assert {L["kernel"] for L in plan} == {want_kernel}, (name, plan)
    if want_mode is not None:
        assert {L["a_mode"] for L in plan} == {want_mode}, (name, plan)
    xd = x.to(DEV)
    out = mod(xd, grid, frames, kind=kind, add=add.to(DEV) if add is not None else None)
    torch.cuda.synchronize()
    mod.close()
    if rows is not None:
        got = out[torch.as_tensor(rows, device=DEV)].float().cpu().double().numpy()
    else:
        got = out.float().cpu().double().numpy()
    cast = None if x.dtype == w.dtype else {torch.bfloat16: "bf16", torch.float32: "f32"}[w.dtype]
    ref = oracle.forward(x, w, b, grid=grid, frames=frames, kind=kind, order=order, rows=rows,
                         cast_input_to=cast, addend=add)
    err = check(got, ref, out_dtype, name)   # asserts every value finite and within tolerance
    print("  ok: %s, %s, max err %.3g" % (sorted({L["kernel"] for L in plan}), sorted({L["a_mode"] for L in plan}), err),
          flush=True)


def weights(seed, E, P, dt, bias=True):
    K = 3 * 2 * P * P
    w = make(seed, (E, 3, 2, P, P), dt, "uniform", 1 / math.sqrt(K))
    b = make(seed + 1, (E,), dt, "uniform", 1 / math.sqrt(K)) if bias else None
    return w, b


def frames_of(seed, items, P, dt):
    return torch.cat([make(seed + i, (F, 3, h * P, ww * P), dt).reshape(-1) for i, (t, h, ww, F) in enumerate(items)])


def main():
    assert os.path.basename(pe.LIB_PATH) == "libpe_sentinel.so", pe.LIB_PATH
    bf, f32 = torch.bfloat16, torch.float32
    P = 14

    # split-k kernel: one image (its partial tiles meet in LDS), a video with an odd frame count
    w, b = weights(4000, 1280, P, bf)
    case("splitk_image", frames_of(4010, [(1, 16, 64, 1)], P, bf), w, b, [[1, 16, 64]], [1],
         want_kernel="pe_fwd32_sk_kernel", want_mode="images")
    case("splitk_video_odd_frames", frames_of(4020, [(2, 8, 6, 3)], P, bf), w, b, [[2, 8, 6]], [3],
         want_kernel="pe_fwd32_sk_kernel", want_mode="frames")

    # large tiles: 256 x 128 (four images), 256 x 256 with a ragged tail, a video, items that
    # straddle tiles and differ in frame size, the fused add
    case("images_256x128", frames_of(4030, [(1, 32, 32, 1)] * 4, P, bf), w, b, [[1, 32, 32]] * 4, [1] * 4,
         want_kernel="pe_fwd32_kernel", want_mode="images")
    case("image_256x256_ragged", frames_of(4040, [(1, 58, 142, 1)], P, bf), w, b, [[1, 58, 142]], [1],
         want_kernel="pe_fwd32_kernel", want_mode="images")
    case("video_256x256", frames_of(4050, [(8, 32, 32, 16)], P, bf), w, b, [[8, 32, 32]], [16],
         want_kernel="pe_fwd32_kernel", want_mode="frames")
    items = [(1, 40, 60, 1), (2, 36, 72, 4), (1, 50, 50, 1), (1, 2, 2, 1)]
    case("mixed_sizes_straddling", frames_of(4060, items, P, bf), w, b, [[t, h, ww] for (t, h, ww, F) in items],
         [F for (*_, F) in items], want_kernel="pe_fwd32_kernel")
    n = 58 * 142
    case("fused_add", frames_of(4070, [(1, 58, 142, 1)], P, bf), w, b, [[1, 58, 142]], [1],
         add=make(4071, (n, 1280), bf), want_kernel="pe_fwd32_kernel")
    case("image_256x256_f32_out", frames_of(4080, [(1, 58, 142, 1)], P, bf), w, b, [[1, 58, 142]], [1],
         out_dtype=f32, want_kernel="pe_fwd32_kernel")

    # single images staged through LDS (opt-in), both large tiles
    case("staged_images_256x256", frames_of(4090, [(1, 60, 138, 1)], P, bf), w, b, [[1, 60, 138]], [1],
         stage=True, want_kernel="pe_fwd32_kernel", want_mode="images_lds")
    case("staged_images_256x128", frames_of(4100, [(1, 64, 64, 1)], P, bf), w, b, [[1, 64, 64]], [1],
         stage=True, want_kernel="pe_fwd32_kernel", want_mode="images_lds")

    # patch rows: the large-tile kernel stages A through LDS (P = 14 and 16, ragged tails)
    for P2, N, seed in ((14, 20000, 4110), (16, 9000, 4120)):
        K = 3 * 2 * P2 * P2
        w2, b2 = weights(seed, 1280, P2, bf)
        case("patch_rows_P%d_N%d" % (P2, N), make(seed + 5, (N, K), bf), w2, b2, [[1, 1, N]], kind="patches",
             order="raster", rows=sampled_rows(N, seed, 600), want_kernel="pe_fwd32_kernel", want_mode="patch_rows")

    # fp32 weight: the 16 x 16 kernel (patch rows and frames)
    w3, b3 = weights(4130, 1280, P, f32)
    case("f32_patch_rows", make(4135, (1024, 1176), f32), w3, b3, [[1, 1, 1024]], kind="patches", order="raster",
         want_kernel="pe_fwd16_kernel")
    w4, b4 = weights(4140, 640, P, f32)
    items = [(1, 6, 8, 1), (2, 4, 2, 4)]
    case("f32_frames", frames_of(4145, items, P, f32), w4, b4, [[t, h, ww] for (t, h, ww, F) in items],
         [F for (*_, F) in items], want_kernel="pe_fwd16_kernel")

    # P = 16 (Qwen3-VL shape), large tiles and split-k
    w5, b5 = weights(4150, 1024, 16, bf)
    items = [(1, 32, 32, 1), (1, 48, 64, 1), (2, 32, 32, 4)]
    case("p16_mixed_batch", frames_of(4155, items, 16, bf), w5, b5, [[t, h, ww] for (t, h, ww, F) in items],
         [F for (*_, F) in items], want_kernel="pe_fwd32_kernel")
    case("p16_splitk_image", frames_of(4160, [(1, 28, 28, 1)], 16, bf), w5, b5, [[1, 28, 28]], [1], order="raster",
         want_kernel="pe_fwd32_sk_kernel")
    print("all cases passed on %s" % pe.LIB_PATH, flush=True)


if __name__ == "__main__":
    main()
