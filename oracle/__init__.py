"""CPU oracle for the NVFP4 MoE expert-FFN path — TEST INFRASTRUCTURE ONLY.

Plain, slow, NumPy-only reference of what the path computes. Only the tests,
the smoke check and the benchmark's CPU-baseline leg may import it; the
product library never does, and this package imports nothing from it.

Sources (commit-log pages of the nvfp4-megamoe-kernel project):
  * nvfp4_mega_moe.py history — global scale as GEMM alpha, the fix for
    UE4M3 overflow (global scale = amax / (6*448)), global -> local expert
    ids, the three quantizer bugs (sign-magnitude nibbles, stored scale =
    block_max/6, nearest E2M1 magnitude), the float8 bit-view pack/unpack.
  * src history — one 1-D slot order for both GEMMs, gather only for L1.
  * nvfp4_cutedsl.py history — GPU-side routing (bincount/cumsum/argsort),
    intermediate split at intermediate_size, gate/up global-scale ratio fold.
  * tests history — packing along K, the six-step pipeline, the layer test
    against a BF16 reference.

Quantization, routing and the scale fold have exactly one correct result and
are computed exactly here. GEMMs, SiLU and the weighted scatter accumulate in
float32 with BF16 roundings at the points the pipeline names.

Parity status: every function is pinned by `tests/test_oracle_*.py` except the
float32 summation order of the GEMMs and SiLU's exp, which are parity
unpinned beyond tolerance.
"""
from .formats import (E2M1_MAGNITUDES, E4M3_MAX_CODE, bf16_to_f32, bf16_to_f64, f32_to_bf16,
                      e4m3_decode, e4m3_encode, e2m1_decode, pack_nibbles, unpack_nibbles)
from .quantize import quantize, quantize_batched, dequantize, global_scale
from .route import route, tile_schedule
from .fold import fold_gate_up, prepare_weights
from .layer import (grouped_gemm, silu_mul, scatter, moe_forward, bf16_reference_layer,
                    cosine, OracleTrace)

__all__ = [
    "E2M1_MAGNITUDES", "E4M3_MAX_CODE", "bf16_to_f32", "bf16_to_f64", "f32_to_bf16",
    "e4m3_decode", "e4m3_encode", "e2m1_decode", "pack_nibbles", "unpack_nibbles",
    "quantize", "quantize_batched", "dequantize", "global_scale", "route", "tile_schedule",
    "fold_gate_up", "prepare_weights", "grouped_gemm", "silu_mul", "scatter", "moe_forward",
    "bf16_reference_layer", "cosine", "OracleTrace",
]
