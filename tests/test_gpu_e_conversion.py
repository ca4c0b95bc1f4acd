"""The float32 -> BF16 conversion instruction the kernels round with (gfx950
v_cvt_pk_bf16_f32) against round-to-nearest-even on the bits, over every
finite float32 pattern (both signs). Runs the check kernel of the probe
library on the GPU."""
import ctypes
import os

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_bf16_conversion_is_rne_on_every_finite_float32():
    lib = ctypes.CDLL(os.path.join(ROOT, "nvfp4_quantized_moe_amd", "libnvfp4probe.so"))
    lib.nvfp4probe_bf16_check.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    res = torch.zeros(2, dtype=torch.int32, device="cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    assert lib.nvfp4probe_bf16_check(ctypes.c_void_p(res.data_ptr()), stream) == 0
    torch.cuda.synchronize()
    bad, first = (int(v) & 0xFFFFFFFF for v in res.cpu().tolist())
    assert bad == 0, f"{bad} patterns differ, first 0x{first:08x}"
