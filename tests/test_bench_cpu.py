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


def _counter_csv(path, rows):
    """A rocprofv3 --pmc csv file with the columns the summaries read."""
    path.mkdir(parents=True, exist_ok=True)
    with open(path / "run_counter_collection.csv", "w") as f:
        f.write('"Kernel_Name","Counter_Name","Counter_Value"\n')
        for k, c, v in rows:
            f.write(f'"{k}","{c}",{v}\n')


L1 = "void nvfp4::grouped_gemm_kernel<3, 2, 8, 2, 1>(unsigned char const*)"
L2 = "void nvfp4::grouped_gemm_kernel<3, 2, 8, 2, 0>(unsigned char const*)"
NEG = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>(int)"


def test_traffic_summary_scales_by_the_copy(tmp_path, monkeypatch):
    # the copy reads and writes 1 GiB; the counters report half the read and all of the write (KiB)
    cal = bench.COPY_CAL_BYTES / 1024
    _counter_csv(tmp_path / "f", [(NEG, "FETCH_SIZE", cal / 2)] * 3 + [(L1, "FETCH_SIZE", 100.0),
                                                                     (L1, "FETCH_SIZE", 300.0),
                                                                     (L2, "FETCH_SIZE", 50.0)])
    _counter_csv(tmp_path / "w", [(NEG, "WRITE_SIZE", cal)] * 3 + [(L1, "WRITE_SIZE", 10.0),
                                                                 (L1, "WRITE_SIZE", 10.0),
                                                                 (L2, "WRITE_SIZE", 40.0)])
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    bench.summarize_traffic("prefill", str(tmp_path / "f"), str(tmp_path / "w"))
    kv = bench._kv(str(tmp_path / "gemm_prefill_traffic.txt"))
    assert float(kv["fetch_copy_factor"]) == 2.0 and float(kv["write_copy_factor"]) == 1.0
    assert float(kv["l1_fetch_bytes_per_launch"]) == 200.0 * 1024 * 2
    assert float(kv["l1_hbm_bytes_per_launch"]) == 200.0 * 1024 * 2 + 10.0 * 1024
    assert float(kv["l2_hbm_bytes_per_launch"]) == 50.0 * 1024 * 2 + 40.0 * 1024
    assert bench.read_traffic("prefill", "l2") == 50.0 * 1024 * 2 + 40.0 * 1024


def test_mfma_busy_share_counts_every_xcd(tmp_path, monkeypatch):
    # GRBM_GUI_ACTIVE is summed over the 8 XCDs: 8000 counted cycles are 1000 cycles of the GPU; 1024 SIMDs
    # busy for 500 of them give a share of one half
    rows = [(L1, "GRBM_GUI_ACTIVE", 8000.0), (L1, "SQ_VALU_MFMA_BUSY_CYCLES", 500.0 * 1024),
            (L1, "SQ_INSTS_MFMA", 500.0 * 1024 / 32)]
    rows += [(L1, c, 1.0) for c in bench.MFMA_COUNTERS if c not in {r[1] for r in rows}]
    _counter_csv(tmp_path / "m", rows)
    monkeypatch.setattr(bench, "PROFILE_DIR", str(tmp_path))
    bench.summarize_mfma("prefill", str(tmp_path / "m"))
    kv = bench._kv(str(tmp_path / "gemm_prefill_mfma.txt"))
    assert float(kv["l1_mfma_busy_share"]) == 0.5
    assert float(kv["l1_executed_mfma_flop_per_launch"]) == 500.0 * 1024 / 32 * 32768
