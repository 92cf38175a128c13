"""bench.py's host-side logic (no GPU): the one-GPU guard, the counter summary it takes `traffic`
from, its order statistics, and the thread count its CPU baseline reports."""
import hashlib
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def _summary(path, sha, hbm=1.5e9):
    lines = ["# test summary", "kernel: gemm_fused_kernel", "kernel_source_sha256: " + sha]
    if hbm is not None:
        lines.append("hbm_bytes_per_launch: %g" % hbm)
    path.write_text("\n".join(lines) + "\n")


def test_recorded_traffic_only_from_a_summary_of_the_current_kernel_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    sha = hashlib.sha256(open(bench.GEMM_SRC, "rb").read()).hexdigest()
    assert bench.recorded_traffic("gemm_fused_8192") is None                 # no summary
    _summary(tmp_path / "gemm_fused_8192_counters.txt", sha)
    assert bench.recorded_traffic("gemm_fused_8192") == pytest.approx(1.5e9)
    _summary(tmp_path / "gemm_fused_8192_counters.txt", "0" * 64)            # another source
    assert bench.recorded_traffic("gemm_fused_8192") is None
    _summary(tmp_path / "gemm_fused_8192_counters.txt", sha, hbm=None)      # no figure
    assert bench.recorded_traffic("gemm_fused_8192") is None


def test_order_statistics():
    xs = [5.0, 1.0, 4.0, 2.0, 3.0, 9.0, 7.0, 8.0, 6.0, 10.0, 0.0]
    assert bench.pct(xs, 0.5) == 5.0
    assert bench.pct(xs, 0.1) == 1.0 and bench.pct(xs, 0.9) == 9.0
    assert bench.pct([], 0.5) is None
    s = bench.stats([2.0, 1.0, 3.0])
    assert s == {"median_ms": 2.0, "p10_ms": 1.0, "p90_ms": 3.0}


def test_cpu_baseline_reports_the_oracle_threads():
    code = "import oracle; print(oracle.num_threads())"
    env = dict(os.environ, OMP_NUM_THREADS="3", PYTHONPATH=ROOT)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env,
                         timeout=120, cwd=ROOT)
    assert res.returncode == 0, res.stderr
    assert int(res.stdout.strip()) == 3
