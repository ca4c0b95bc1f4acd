"""Host logic of bench.py, on the CPU: the one-GPU contract and the committed
HBM-traffic summaries it reads (keyed by the grouped GEMM's source)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_traffic_summary_matches_the_kernel_source(tmp_path, monkeypatch):
    sha = bench.kernel_source_sha()
    assert len(sha) == 16
    good = tmp_path / "l1_gemm_prefill_traffic.txt"
    good.write_text(f"# test\nkernel_source_sha = {sha}\nhbm_bytes_per_launch = 1234.0\n")
    stale = tmp_path / "l1_gemm_decode_traffic.txt"
    stale.write_text("kernel_source_sha = 0000000000000000\nhbm_bytes_per_launch = 99.0\n")
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    assert bench.read_traffic("prefill") == 1234.0
    assert bench.read_traffic("decode") is None       # taken on another source: not reported
    assert bench.read_traffic("skewed") is None       # no summary

