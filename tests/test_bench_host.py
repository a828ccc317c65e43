"""CPU checks of bench.py's host-side arithmetic: the algorithmic FLOPs and bytes of each workload
(the units behind `roofline.achieved` and `hbm_frac`), the kernel it names as doing the work, and
the refusal of more than one GPU."""
import os
import subprocess
import sys

import pytest

from conftest import ROOT

sys.path.insert(0, ROOT)
import bench  # noqa: E402
import workloads  # noqa: E402

# workload: (N, FLOPs = 2 N K E, bytes = unique input once + packed weight + bias + output), each
# written out from the workload's shapes
EXPECTED = {
    # 1024 patch rows of K = 1176, fp32 in / weight / out, E = 1280, no bias
    1: (1024, 2 * 1024 * 1176 * 1280, 1024 * 1176 * 4 + 1280 * 1176 * 4 + 1024 * 1280 * 4),
    # one 224 x 896 image (one frame read once), bf16, E = 1280, no bias
    2: (1024, 2 * 1024 * 1176 * 1280, 3 * 224 * 896 * 2 + 1280 * 1176 * 2 + 1024 * 1280 * 2),
    # one 448 x 448 image, P = 16 (K = 1536), E = 1152, bf16 bias
    3: (784, 2 * 784 * 1536 * 1152, 3 * 448 * 448 * 2 + 1152 * 1536 * 2 + 1152 * 2 + 784 * 1152 * 2),
    # a 16-frame 448 x 448 video: every frame read once
    4: (8192, 2 * 8192 * 1176 * 1280, 16 * 3 * 448 * 448 * 2 + 1280 * 1176 * 2 + 8192 * 1280 * 2),
    # 64 images of 1008 x 1008 with bias
    5: (331776, 2 * 331776 * 1176 * 1280,
        64 * 3 * 1008 * 1008 * 2 + 1280 * 1176 * 2 + 1280 * 2 + 331776 * 1280 * 2),
}


@pytest.mark.parametrize("idx", sorted(EXPECTED))
def test_algorithmic_units(idx):
    n, flops, byts = bench.algorithmic(workloads.WORKLOADS[idx])
    assert (n, flops, byts) == EXPECTED[idx]


def test_algorithmic_units_of_variants():
    wl = workloads.WORKLOADS[5]
    n, flops, byts = bench.algorithmic(wl)
    # the same patches as pre-flattened rows: both temporal slots of every patch are read
    _, _, rows_bytes = bench.algorithmic(wl, rows=True)
    assert rows_bytes - byts == n * 1176 * 2 - 64 * 3 * 1008 * 1008 * 2
    # the fused add reads an [N, E] addend in the output dtype
    _, _, add_bytes = bench.algorithmic(wl, add=True)
    assert add_bytes - byts == n * 1280 * 2


@pytest.mark.parametrize("idx,kernel", [(1, "pe_fwd16_kernel"), (2, "pe_fwd32_sk_kernel"),
                                        (3, "pe_fwd32_sk_kernel"), (4, "pe_fwd32_kernel"),
                                        (5, "pe_fwd32_kernel"), (6, "pe_fwd32_kernel")])
def test_dominant_kernel(idx, kernel):
    assert bench.dominant_kernel(workloads.WORKLOADS[idx]) == kernel


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
