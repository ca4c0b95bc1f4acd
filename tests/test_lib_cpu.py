"""The C-ABI library loads and exports every entry point of include/nvfp4moe.h
(CPU only: no kernel is launched). Argument validation happens on the host
before any launch, so invalid calls return their status here too."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "nvfp4_quantized_moe_amd", "libnvfp4moe.so")
HEADER = os.path.join(ROOT, "include", "nvfp4moe.h")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="library not built (run build())")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "sizeof")))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("nvfp4_quantize", "moe_route_slots", "nvfp4_grouped_gemm", "nvfp4_moe_forward",
              "moe_weighted_scatter", "nvfp4_fold_scales", "nvfp4_pack_weights", "nvfp4_packed_bytes",
              "nvfp4_quantize_static", "nvfp4_grouped_gemm_silu_nvfp4", "nvfp4_moe_forward_static"):
        assert n in names


def test_every_declared_symbol_is_exported():
    lib = ctypes.CDLL(LIB)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing


def _lib():
    import nvfp4_quantized_moe_amd as nv
    return nv


def test_status_strings_and_sizes():
    nv = _lib()
    assert nv._status_string(0) == b"ok"
    assert b"workspace" in nv._status_string(4)
    assert nv.version() == 300
    assert nv.nvfp4_tile_table_len(512, 48, 32) == 1 + 2 * (16 + 48)
    lay = nv.nvfp4_moe_ws_layout(64, 8, 7168, 3072, 48)
    offs = [lay[r] for r in nv.WS_REGIONS]
    assert offs == sorted(offs) and all(o % 256 == 0 for o in offs)
    assert lay["end"] == nv.nvfp4_moe_ws_bytes(64, 8, 7168, 3072, 48)
    assert lay["y"] - lay["h_sf"] >= 512 * 3072 // 16
    assert nv.nvfp4_moe_tile_m(64, 8, 48) == 32 and nv.nvfp4_moe_tile_m(8192, 8, 48) == 96


def test_invalid_arguments_are_rejected_before_launch():
    nv = _lib()
    buf = ctypes.c_void_p(4096)       # never dereferenced: validation fails first
    odd = ctypes.c_void_p(4097)
    null = None
    s = None
    # quantize: bad K, NULL outputs, misalignment, small workspace
    assert nv._quantize(buf, 1, 4, 48, null, buf, buf, buf, buf, 1 << 20, s) == 2
    assert nv._quantize(buf, 1, 4, 64, null, null, buf, buf, buf, 1 << 20, s) == 1
    assert nv._quantize(odd, 1, 4, 64, null, buf, buf, buf, buf, 1 << 20, s) == 3
    assert nv._quantize(buf, 1, 4, 64, null, buf, buf, buf, buf, 8, s) == 4
    assert nv._quantize(buf, 0, 4, 64, null, buf, buf, buf, buf, 1 << 20, s) == 2
    # route: k out of range, tile_m unsupported, NULL outputs
    args = [buf] * 7
    assert nv._route(buf, buf, 4, 0, 0, 8, 32, *args, buf, 1 << 20, s) == 2
    assert nv._route(buf, buf, 4, 2, 0, 8, 40, *args, buf, 1 << 20, s) == 2
    assert nv._route(buf, buf, 4, 2, 0, 8, 272, *args, buf, 1 << 20, s) == 2
    assert nv._route(buf, buf, 4, 2, 0, 8, 32, null, *args[1:], buf, 1 << 20, s) == 1
    # grouped GEMM: K not a multiple of 128, unknown epilogue, odd tile height
    g = [buf] * 8
    assert nv._gemm(*g, 8, 64, 256, 96, 32, 0, buf, null, s) == 2
    assert nv._gemm(*g, 8, 64, 256, 256, 32, 7, buf, null, s) == 6
    assert nv._gemm(*g, 8, 64, 256, 256, 32, 2, buf, null, s) == 1   # dual-scale SiLU also needs amax_out
    assert nv._gemm(*g, 8, 64, 256, 256, 48, 0, buf, null, s) == 2
    assert nv._gemm(*g, 8, 64, 256, 256, 32, 1, buf, null, s) == 1   # SiLU epilogue needs amax_out
    assert nv._gemm(*g, 8, 64, 1 << 23, 128, 96, 0, buf, null, s) == 2  # a 128-row output tile past 2^31 bytes
    # packed size / pack: N not a multiple of 32, K not a multiple of 128, NULL input, misaligned output
    assert nv.nvfp4_packed_bytes(2, 64, 256) == 2 * 64 * 256 * 9 // 16
    assert nv.nvfp4_packed_bytes(1, 48, 256) == -1 and nv.nvfp4_packed_bytes(1, 64, 192) == -1
    assert nv._pack(buf, buf, 1, 48, 256, buf, s) == 2
    assert nv._pack(buf, buf, 1, 64, 192, buf, s) == 2
    assert nv._pack(null, buf, 1, 64, 256, buf, s) == 1
    assert nv._pack(buf, buf, 1, 64, 256, odd, s) == 3
    # scatter / fold
    assert nv._scatter(buf, buf, buf, 4, 2, 12, buf, s) == 2
    assert nv._fold(null, buf, buf, buf, 4, 64, 256, s) == 1
    # forward: NULL weights struct, bad hidden
    assert nv._forward(None, buf, 4, buf, buf, 2, 0, buf, buf, 1 << 30, s) == 1
    w = nv._Weights(8, 200, 128, 4096, 4096, 4096, 4096)
    assert nv._forward(ctypes.byref(w), buf, 4, buf, buf, 2, 0, buf, buf, 1 << 30, s) == 2
    w = nv._Weights(8, 256, 128, 4096, 4096, 4096, 4096)
    assert nv._forward(ctypes.byref(w), buf, 4, buf, buf, 2, 0, buf, buf, 16, s) == 4
    w = nv._Weights(8, 256, 128, 4096, 4096, None, 4096)
    assert nv._forward(ctypes.byref(w), buf, 4, buf, buf, 2, 0, buf, buf, 1 << 30, s) == 1
    w = nv._Weights(8, 256, 128, 4097, 4096, 4096, 4096)
    assert nv._forward(ctypes.byref(w), buf, 4, buf, buf, 2, 0, buf, buf, 1 << 30, s) == 3
    # 32-bit offsets: T*H/2, T*k*I/2 and 2I*H*9/16 must stay below 2^31; T*k below 2^30
    big = nv._Weights(8, 7168, 3072, 4096, 4096, 4096, 4096)
    # (every call here fails validation: the pointers are fake and must never reach a launch)
    assert nv._forward(ctypes.byref(big), buf, (1 << 31) // 3584 + 1, buf, buf, 1, 96, buf, buf, 1 << 62, s) == 2
    assert nv._forward(ctypes.byref(big), buf, 175000, buf, buf, 8, 96, buf, buf, 1 << 62, s) == 2  # T*k*I/2
    assert nv._forward(ctypes.byref(big), buf, 1 << 27, buf, buf, 8, 96, buf, buf, 1 << 62, s) == 2   # T*k = 2^30
    huge = nv._Weights(8, 65536, 32768, 4096, 4096, 4096, 4096)                                  # 2I*H*9/16 >= 2^31
    assert nv._forward(ctypes.byref(huge), buf, 4, buf, buf, 2, 0, buf, buf, 1 << 62, s) == 2
    wide = nv._Weights(8, 1 << 23, 128, 4096, 4096, 4096, 4096)                                  # 256*H = 2^31
    assert nv._forward(ctypes.byref(wide), buf, 1, buf, buf, 1, 0, buf, buf, 1 << 62, s) == 2
    w = nv._Weights(8, 256, 128, 4096, 4096, 4096, 4096, 2)     # unknown gate/up scale mode
    assert nv._forward(ctypes.byref(w), buf, 4, buf, buf, 2, 0, buf, buf, 1 << 30, s) == 6
    # quantize without a workspace: more tensors than its array holds, bad K, NULL gs
    assert nv._quantize_noalloc(buf, 129, 4, 64, null, buf, buf, buf, s) == 4
    assert nv._quantize_noalloc(buf, 1, 4, 48, null, buf, buf, buf, s) == 2
    assert nv._quantize_noalloc(buf, 1, 4, 64, null, buf, buf, null, s) == 1
    assert nv._quantize_noalloc(odd, 1, 4, 64, null, buf, buf, buf, s) == 3
    # fixed-scale entry points: NULL scales, bad shapes, unknown gate/up scale mode
    assert nv._quantize_static(buf, 1, 4, 64, null, buf, buf, s) == 1
    assert nv._quantize_static(buf, 1, 4, 48, buf, buf, buf, s) == 2
    assert nv._quantize_static(buf, 65536, 4, 64, buf, buf, buf, s) == 2
    assert nv._quantize_static(odd, 1, 4, 64, buf, buf, buf, s) == 3
    gq = [buf] * 6
    assert nv._gemm_nvfp4(*gq, 2, buf, buf, 8, 64, 256, 256, 32, buf, buf, buf, s) == 6
    assert nv._gemm_nvfp4(*gq, 0, buf, buf, 8, 64, 192, 256, 32, buf, buf, buf, s) == 2   # N % 128
    assert nv._gemm_nvfp4(*gq, 0, buf, buf, 8, 64, 256, 256, 48, buf, buf, buf, s) == 2   # tile_m
    assert nv._gemm_nvfp4(*gq, 0, buf, buf, 8, 64, 256, 256, 32, null, buf, buf, s) == 1  # out_gs
    w = nv._Weights(8, 256, 128, 4096, 4096, 4096, 4096)
    assert nv._forward_static(ctypes.byref(w), buf, 4, buf, buf, 2, 0, null, buf, buf, 1 << 30, s) == 1
    assert nv._forward_static(ctypes.byref(w), buf, 4, buf, buf, 2, 0, buf, buf, buf, 16, s) == 4
