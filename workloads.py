"""Seeded synthetic inputs for the vision PatchEmbed, shared by the tests, the smoke check
and the benchmark.

This module holds data only: the five workload descriptions (shapes, dtypes, grids) and the
random generators that fill them. It holds none of the method's arithmetic (no patch count,
no row order, no convolution), so the oracle and the HIP path can both draw from it without
sharing any computation.

Recipe (one ``torch.Generator('cpu')`` per call, seeded with the caller's seed):
  1. pixels  = randn(shape) in float32, N(0, 1), as in the Conv3d-vs-matmul check on the
     "Qwen2.5VL-Vision Encode-PatchEmbed" page;
  2. weight  = (rand(shape) * 2 - 1) / sqrt(K), i.e. U(-1/sqrt(K), +1/sqrt(K)), PyTorch's
     default Conv3d initialisation for fan_in K;
  3. bias    = the same bound, drawn after the weight (only when the workload has a bias);
then each tensor is rounded to the workload's dtype (round-to-nearest-even, torch's cast).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    """One benchmark / parity workload. ``kind`` is "patches" (pre-flattened [N, K] rows)
    or "frames" (raw [F, C, H, W] frames per item, items back to back)."""

    index: int
    name: str
    kind: str
    in_dtype: str
    w_dtype: str
    out_dtype: str
    patch: int
    embed: int
    bias: bool
    order: str                      # "raster" or "merge"
    grid: tuple                     # per item (t, h, w) in patch units
    frames: tuple                   # per item frame count (frames kind), else ()
    input_shape: tuple              # shape of the whole input buffer
    channels: int = 3
    temporal: int = 2
    merge: int = 2
    note: str = field(default="", compare=False)

    @property
    def k(self) -> int:
        return self.channels * self.temporal * self.patch * self.patch

    @property
    def weight_shape(self) -> tuple:
        return (self.embed, self.channels, self.temporal, self.patch, self.patch)


# The five workloads. Frame sizes are stated directly (H = h*P, W = w*P per item).
WORKLOADS = {
    1: Workload(1, "page1_validation_f32", "patches", "f32", "f32", "f32", 14, 1280, False,
                "raster", ((1, 32, 32),), (), (1024, 1176),
                note="pre-flattened patch rows x[1024,1176] fp32, no bias"),
    2: Workload(2, "qwen25vl_image_224x896", "frames", "bf16", "bf16", "bf16", 14, 1280, False,
                "merge", ((1, 16, 64),), (1,), (1, 3, 224, 896),
                note="single image, frame duplicated over the temporal pair"),
    3: Workload(3, "p16_448x448_bias", "frames", "bf16", "bf16", "bf16", 16, 1152, True,
                "raster", ((1, 28, 28),), (1,), (1, 3, 448, 448),
                note="patch 16, K=1536, E=1152, bias, raster rows"),
    4: Workload(4, "video_16x448x448", "frames", "bf16", "bf16", "bf16", 14, 1280, False,
                "merge", ((8, 32, 32),), (16,), (16, 3, 448, 448),
                note="16-frame clip, 8 temporal patches"),
    5: Workload(5, "batch64_1008x1008_bias", "frames", "bf16", "bf16", "bf16", 14, 1280, True,
                "merge", tuple((1, 72, 72) for _ in range(64)), tuple(1 for _ in range(64)),
                (64, 3, 1008, 1008),
                note="64 images, each frame duplicated; throughput batch"),
    # Qwen3-VL-2B-shaped vision PatchEmbed ("Optimize VLM PatchEmbed": patch 16, hidden 1024,
    # Conv3d with bias) over a batch of items of different sizes: images and one video.
    6: Workload(6, "qwen3vl2b_p16_e1024_mixed", "frames", "bf16", "bf16", "bf16", 16, 1024, True,
                "merge", ((1, 32, 32), (1, 48, 64), (2, 32, 32), (1, 24, 40), (1, 32, 32)),
                (1, 1, 4, 1, 1),
                (3 * 16 * 16 * (32 * 32 + 48 * 64 + 4 * 32 * 32 + 24 * 40 + 32 * 32),),
                note="mixed sizes: four images and a 4-frame video, items back to back"),
}


def input_elements(wl: Workload) -> int:
    """Elements of the whole input buffer."""
    n = 1
    for d in wl.input_shape:
        n *= d
    return n


def share(wl: Workload, items: int) -> Workload:
    """The first `items` items of a frames workload (one GPU's share of an item split); its
    input is the leading part of the whole input buffer."""
    if wl.kind != "frames":
        raise ValueError("item shares apply to frames workloads")
    grid, frames = wl.grid[:items], wl.frames[:items]
    elems = sum(f * wl.channels * (h * wl.patch) * (w * wl.patch) for (t, h, w), f in zip(grid, frames))
    return Workload(wl.index, "%s_share%d" % (wl.name, items), wl.kind, wl.in_dtype, wl.w_dtype,
                    wl.out_dtype, wl.patch, wl.embed, wl.bias, wl.order, grid, frames, (elems,),
                    wl.channels, wl.temporal, wl.merge, "first %d items of %s" % (items, wl.name))


def generate(wl: Workload, seed: int | None = None):
    """Return (pixels, weight, bias_or_None) as CPU tensors in the workload's dtypes.

    ``seed`` defaults to the workload's position in the list (index - 1)."""
    if seed is None:
        seed = wl.index - 1
    g = torch.Generator("cpu").manual_seed(seed)
    x = torch.randn(wl.input_shape, generator=g, dtype=torch.float32)
    bound = 1.0 / math.sqrt(wl.k)
    w = (torch.rand(wl.weight_shape, generator=g, dtype=torch.float32) * 2 - 1) * bound
    b = None
    if wl.bias:
        b = (torch.rand((wl.embed,), generator=g, dtype=torch.float32) * 2 - 1) * bound
    x = x.to(DTYPES[wl.in_dtype])
    w = w.to(DTYPES[wl.w_dtype])
    if b is not None:
        b = b.to(DTYPES[wl.w_dtype])
    return x, w, b


def random_tensor(shape, seed: int, dtype=torch.float32, dist: str = "normal", bound: float = 1.0,
                  low: int = 0, high: int = 3):
    """General seeded generator for test cases: "normal" N(0,1), "uniform" U(-bound, bound),
    or "int" integers in [low, high). Generated in float32 (int64 for "int"), then cast."""
    g = torch.Generator("cpu").manual_seed(seed)
    if dist == "normal":
        t = torch.randn(shape, generator=g, dtype=torch.float32)
    elif dist == "uniform":
        t = (torch.rand(shape, generator=g, dtype=torch.float32) * 2 - 1) * bound
    elif dist == "int":
        t = torch.randint(low, high, shape, generator=g, dtype=torch.int64).to(torch.float32)
    else:
        raise ValueError(dist)
    return t.to(dtype)
