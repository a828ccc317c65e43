"""CPU checks of bench.py's host-side arithmetic: the algorithmic FLOPs and bytes of each workload
(the units behind `roofline.achieved` and `hbm_frac`), the row sample of the CPU baseline and its
parity check, the counter summary behind `roofline.traffic` and the machine-code hash that keys it,
and the refusal of more than one GPU.
The kernel the bench names comes from the library's own launch plan (pe_forward_plan), tested in
test_plan.py and on the GPU."""
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


def test_sample_rows_cover_edges_and_spread():
    n = 331776
    rows = bench.sample_rows(n, 5000)
    assert rows == sorted(set(rows)) and len(rows) == 5000 and rows[0] == 0 and rows[-1] == n - 1
    assert {255, 256, 511, 512} <= set(rows)
    # evenly spread: every 1/50 of the rows holds some of the sample
    assert all(any(i * n // 50 <= r < (i + 1) * n // 50 for r in rows) for i in range(50))
    assert bench.sample_rows(100, 1000) == list(range(100))


def test_cpu_info_states_model_and_share():
    info = bench.cpu_info()
    assert info["usable"] >= 1 and info["usable"] <= info["nproc"]
    assert isinstance(info["model"], str)


def test_summarize_pmc_reads_rocprof_csv(tmp_path, monkeypatch):
    """Per-dispatch sums of a counter's instance rows, averaged over dispatches, scaled by a copy;
    the record is read back for the kernel's current code only."""
    if not os.path.exists(bench.LIBPE):
        pytest.skip("libpe.so not built (the record is keyed by the kernel's machine code)")
    hdr = "Correlation_Id,Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value\n"

    def write(d, rows):
        os.makedirs(d, exist_ok=True)
        open(os.path.join(d, "pmc_counter_collection.csv"), "w").write(hdr + "".join(rows))
    k = "void pe::pe_fwd32_kernel<14>(pe::FwdArgs)"
    write(str(tmp_path / "f"), ['1,1,"%s",FETCH_SIZE,100\n' % k, '1,1,"%s",FETCH_SIZE,50\n' % k,
                                '2,2,"%s",FETCH_SIZE,150\n' % k, '3,3,other,FETCH_SIZE,999\n'])
    write(str(tmp_path / "w"), ['1,1,"%s",WRITE_SIZE,200\n' % k, '2,2,"%s",WRITE_SIZE,200\n' % k])
    write(str(tmp_path / "cf"), ['1,1,__amd_rocclr_copyBuffer,FETCH_SIZE,512\n'])
    write(str(tmp_path / "cw"), ['1,1,__amd_rocclr_copyBuffer,WRITE_SIZE,1024\n'])
    assert bench.pmc_per_dispatch(str(tmp_path / "f"), "FETCH_SIZE", "pe_fwd32_kernel") == (150.0, 2)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    os.makedirs(tmp_path / "profiles")
    rec = bench.summarize_pmc(5, "pe_fwd32_kernel", str(tmp_path / "f"), str(tmp_path / "w"),
                              str(tmp_path / "cf"), str(tmp_path / "cw"), 1024 * 1024)
    # copy of 1 MiB: fetch reads 512 KiB (factor 2), write 1024 KiB (factor 1)
    assert rec["fetch_factor"] == 2.0 and rec["write_factor"] == 1.0
    assert rec["bytes_per_launch"] == 150 * 1024 * 2 + 200 * 1024
    name = workloads.WORKLOADS[5].name
    assert bench.load_traffic("pe_fwd32_kernel", name) == rec["bytes_per_launch"]
    # counters taken on other code are not used
    monkeypatch.setattr(bench, "kernel_code_hash", lambda k, lib=None: "0" * 16)
    assert bench.load_traffic("pe_fwd32_kernel", name) is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_extra_entries_parse():
    assert bench.parse_extra("5") == (5, False, False, False, None, False)
    assert bench.parse_extra("5r") == (5, True, False, False, None, False)
    assert bench.parse_extra("5a") == (5, False, True, False, None, False)
    assert bench.parse_extra("2f") == (2, False, False, True, None, False)
    assert bench.parse_extra("5s8") == (5, False, False, False, 8, False)
    assert bench.parse_extra("5l") == (5, False, False, False, None, True)


FAMILIES = ("pe_fwd32_kernel", "pe_fwd32_sk_kernel", "pe_fwd16_kernel", "pe_layernorm_kernel")


def test_kernel_code_hash_follows_the_code(tmp_path):
    """The key of the committed traffic counters: one hash per kernel template, from its machine
    code in libpe.so. A one-byte change inside one instantiation of one kernel changes that
    kernel's hash and no other."""
    if not os.path.exists(bench.LIBPE):
        pytest.skip("libpe.so not built")
    b = open(bench.LIBPE, "rb").read()
    hs = {k: bench.kernel_code_hash(k) for k in FAMILIES}
    assert len(set(hs.values())) == len(FAMILIES)
    assert hs == {k: bench.kernel_code_hash(k) for k in FAMILIES}
    with pytest.raises(ValueError):
        bench.kernel_code_hash("pe_no_such_kernel")
    # both the entries and their descriptors are found, and the two template names do not overlap
    syms = list(bench.kernel_symbols(b, "pe_fwd16_kernel"))
    assert any(n.endswith(".kd") for n, _, _ in syms) and any(not n.endswith(".kd") for n, _, _ in syms)
    assert not any("sk_kernel" in n for n, _, _ in bench.kernel_symbols(b, "pe_fwd32_kernel"))
    name, off, size = next((n, o, z) for n, o, z in sorted(syms) if not n.endswith(".kd"))
    assert size > 64
    mutated = bytearray(b)
    mutated[off + size // 2] ^= 0x01
    lib2 = tmp_path / "libpe.so"
    lib2.write_bytes(bytes(mutated))
    after = {k: bench.kernel_code_hash(k, str(lib2)) for k in FAMILIES}
    assert after["pe_fwd16_kernel"] != hs["pe_fwd16_kernel"]
    assert {k: v for k, v in after.items() if k != "pe_fwd16_kernel"} == \
        {k: v for k, v in hs.items() if k != "pe_fwd16_kernel"}
    # a descriptor's entry offset (its distance to the code, which moves with the layout of the
    # code object) does not count; its other fields (resources) do
    kd_name, kd_off, kd_size = next((n, o, z) for n, o, z in sorted(syms) if n.endswith(".kd"))
    assert kd_size == 64
    moved = bytearray(b)
    moved[kd_off + 16] ^= 0x40
    lib3 = tmp_path / "libpe_moved.so"
    lib3.write_bytes(bytes(moved))
    assert bench.kernel_code_hash("pe_fwd16_kernel", str(lib3)) == hs["pe_fwd16_kernel"]
    moved[kd_off + 16] ^= 0x40
    moved[kd_off + 0] ^= 0x01          # group_segment_fixed_size: the LDS it asks for
    lib3.write_bytes(bytes(moved))
    assert bench.kernel_code_hash("pe_fwd16_kernel", str(lib3)) != hs["pe_fwd16_kernel"]


def test_cpu_leg_parity_of_a_secondary_line():
    """cpu_baseline_config on a small frames line whose 'timed output' is made on the host: the
    oracle's own rows rounded to bf16 pass; one element moved by 0.1 fails the tolerance; the
    approximate line reports its error with no tolerance."""
    import numpy as np
    import torch
    import oracle
    wl = workloads.Workload(0, "tiny", "frames", "bf16", "bf16", "bf16", 14, 64, True, "merge",
                            ((1, 4, 6),), (1,), (1, 3, 56, 84))
    x, w, b = workloads.generate(wl)
    grid, frames = [[1, 4, 6]], [1]
    ref = oracle.forward(x, w, b, grid=grid, frames=frames, kind="frames", order="merge")
    out = torch.from_numpy(ref).to(torch.bfloat16)
    q = dict(wl=wl, n=24, host_in=(x, w, b, None), grid=grid, frames=frames, kind="frames", out=out)
    r = bench.cpu_baseline_config(q, max_rows=10)
    assert r["rows_checked"] == 10 and r["of_rows"] == 24 and r["out_of_tolerance"] == 0
    assert r["max_abs_err"] <= np.abs(ref).max() * 2 ** -8
    bad = out.clone()
    bad[0, 3] += 0.1
    assert bench.cpu_baseline_config(dict(q, out=bad), max_rows=24)["out_of_tolerance"] == 1
    a = bench.cpu_baseline_config(dict(q, out=bad), max_rows=24, approximate=True)
    assert a["out_of_tolerance"] is None and a["max_abs_err"] >= 0.09
