"""The quantizer's exact roundings (quant_block.h), compiled for the host and
run on the CPU: the E2M1 index (two elements per 32-bit add, a three-test
binary search, byte-permute packing) against plain counting of the thresholds
passed, every BF16 value in every position of eight against random
non-decreasing threshold sets, including thresholds at and past the largest
finite magnitude and the nothing-passes table of scale code 0; the block
maximum; the block scale code (a float32 estimate settled by two table tests)
against counts of exact float64 midpoint comparisons for every finite block
maximum at fixed, random and tie-making global scales; the threshold table's
16-bit entries; and the threshold round-down against the float64 route. No
GPU is needed and no kernel is launched."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "quant_block_host_check.hip")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not (os.path.exists(HIPCC) or shutil.which("hipcc")), reason="hipcc not available")
def test_two_per_word_rounding_matches_counting(tmp_path):
    exe = str(tmp_path / "quant_block_host_check")
    build = subprocess.run([HIPCC, "-O2", "-std=c++17", "--offload-arch=gfx950", "-I", os.path.join(ROOT, "include"),
                            SRC, "-o", exe], capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-2000:]
    run = subprocess.run([exe, "200"], capture_output=True, text=True, timeout=300)
    assert run.returncode == 0, run.stdout[-2000:]
    assert "mismatches 0" in run.stdout
