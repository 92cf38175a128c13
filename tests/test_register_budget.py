"""The fused GEMM kernels run next to the side-stream copy kernel (and, with the copy-engine producer,
next to the runtime's small flag-writing kernels) on every CU, one wave of each per SIMD; in GEMM +
ReduceScatter the plain GEMM kernel runs next to the reducing kernel the same way.  That only
works if their VGPRs fit in one SIMD's 512 per lane together; if they do not, the copy cannot start
while the GEMM waits for it, and every wait runs into its time-out.  This compiles the kernel source
for gfx950 (no GPU needed) and checks the budget from the compiler's own kernel metadata."""
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "allgather_gemm_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
GRANULE = 8          # VGPR allocation granule per wave (gfx950, wave64)
VGPRS_PER_LANE = 512


def kernel_vgprs(tmp_path, src):
    out = tmp_path / (src + ".s")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
           os.path.join(CSRC, src), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    text = out.read_text()
    vg = {}
    for block in text.split("  - .agpr_count")[1:]:
        name = re.search(r"\.name:\s+(\S+)", block).group(1)
        vg[name] = int(re.search(r"\.vgpr_count:\s+(\d+)", block).group(1))
    return vg


def alloc(v):
    return (v + GRANULE - 1) // GRANULE * GRANULE


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_fused_gemm_and_concurrent_copy_kernel_fit_on_one_simd(tmp_path):
    vg = kernel_vgprs(tmp_path, "ag_gemm.hip")
    fused = {n: v for n, v in vg.items() if "gemm_fused" in n}   # bf16 and FP8 inputs, with/without trickle
    copy = [v for n, v in vg.items() if "producer_kernelILi8E" in n]
    assert len(fused) == 4 and len(copy) == 1, sorted(vg)
    for name, v in fused.items():
        assert alloc(v) + alloc(copy[0]) <= VGPRS_PER_LANE, (name, v, copy[0])


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_plain_gemm_and_reducing_kernel_fit_on_one_simd(tmp_path):
    vg = kernel_vgprs(tmp_path, "ag_gemm.hip")
    rs = kernel_vgprs(tmp_path, "rs.hip")
    plain = [v for n, v in vg.items() if "gemm_plain" in n]
    red = [v for n, v in rs.items() if "rs_reduce" in n]
    assert len(plain) == 2 and len(red) >= 1, (sorted(vg), sorted(rs))   # bf16 and FP8 inputs
    for p in plain:
        for v in red:
            assert alloc(p) + alloc(v) <= VGPRS_PER_LANE, (p, v)


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_gemm_tile_loads_use_a_uniform_buffer_resource(tmp_path):
    """The K loop's global->LDS loads take their buffer resource from scalar registers.  If the
    compiler cannot prove the resource uniform (a lane-0-only branch in the tile loop was enough to
    break its analysis once), it wraps every load in a loop over the distinct values of the lanes
    -- readfirstlane, compare, exec mask -- which cost the GEMM 8 %.  No such loop may appear."""
    out = tmp_path / "ag_gemm.s"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "--cuda-device-only", "-S",
           os.path.join(CSRC, "ag_gemm.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = out.read_text().splitlines()
    n_dma = 0
    for i, line in enumerate(lines):
        if "offen lds" in line:
            n_dma += 1
            window = lines[max(0, i - 8):i]
            assert not any("v_readfirstlane" in w for w in window), "\n".join(lines[max(0, i - 8):i + 1])
    assert n_dma > 0
