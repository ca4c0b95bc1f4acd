"""The quantizer's exact E2M1 rounding (two elements per 32-bit add, index
read from the thermometer code of the seven midpoint tests) against plain
counting of the thresholds passed, compiled for the host and run on the CPU:
every low-half BF16 value against random non-decreasing threshold sets,
including thresholds at and past the largest finite magnitude and the
nothing-passes table of scale code 0; also the block maximum and the byte
packing. No GPU is needed and no kernel is launched."""
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
