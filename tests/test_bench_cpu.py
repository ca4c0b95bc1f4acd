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
    good = tmp_path / "gemm_prefill_traffic.txt"
    good.write_text(f"# test\nkernel_source_sha = {sha}\nl1_hbm_bytes_per_launch = 1234\n"
                    f"l2_hbm_bytes_per_launch = 567   # comment\n")
    stale = tmp_path / "gemm_decode_traffic.txt"
    stale.write_text("kernel_source_sha = 0000000000000000\nl1_hbm_bytes_per_launch = 99.0\n")
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    assert bench.read_traffic("prefill") == 1234.0
    assert bench.read_traffic("prefill", "l2") == 567.0
    assert bench.read_traffic("decode") is None       # taken on another source: not reported
    assert bench.read_traffic("skewed") is None       # no summary


def test_counter_summaries_name_kernels():
    assert bench._gemm_epi("void nvfp4::grouped_gemm_kernel<3, 2, 8, 2, 1>(unsigned char const*)") == 1
    assert bench._kernel_label("nvfp4::grouped_gemm_kernel<3, 2, 8, 2, 0>(x)") == "l2_gemm"
    assert bench._kernel_label("nvfp4::grouped_gemm_kernel<3, 2, 8, 2, 3>(x)") == "l1_gemm_nvfp4"
    assert bench._gemm_epi("nvfp4::quantize_kernel<false>(x)") is None


def test_stats():
    s = bench.stats([1.0, 2.0, 3.0, 4.0, 5.0])
    assert s["median"] == 3.0 and s["n"] == 5 and s["p10"] < s["median"] < s["p90"]
