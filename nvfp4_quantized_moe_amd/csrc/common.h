// Shared device helpers for the NVFP4 MoE kernels (gfx950 only).
//
// Number formats (nvfp4_mega_moe.py history, three-quantizer-bugs and float8
// bit-view commits; tests history, packing-along-K commit):
//   E2M1 nibble  bit 3 sign, bits 2:0 index {0, .5, 1, 1.5, 2, 3, 4, 6}
//   E4M3 byte    float8_e4m3fn, bias 7, max 0x7E = 448, 0x7F NaN
//   BF16         raw 16-bit patterns
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "nvfp4moe.h"

namespace nvfp4 {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef float float4_t __attribute__((ext_vector_type(4)));

constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, one L2 each

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float32 -> BF16 bits, nearest with ties to even (inputs are finite): the
// gfx950 conversion v_cvt_pk_bf16_f32, which equals the bit construction
// (u + 0x7FFF + bit 16 of u) >> 16 on every finite float32 (all 2^32
// patterns compared on MI355X)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// two float32 -> a BF16 pair (a in the low half), one instruction
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  const float2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Exact value of an E4M3 code (non-NaN) as float32.
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  return __builtin_amdgcn_cvt_f32_fp8(code & 0xFFu, 0);
}

// Nearest E4M3 code to a non-negative double, ties to the even code,
// saturating at 448 (0x7E). Subnormal codes are multiples of 2^-9.
__host__ __device__ __forceinline__ uint32_t e4m3_encode_rne_sat(double v) {
  if (!(v < 448.0)) return 0x7Eu;                      // also catches +inf
  if (v < 0.015625) {                                   // below 2^-6: step 2^-9
    return (uint32_t)__builtin_rint(v * 512.0);        // 8 -> 0x08 = 2^-6, still exact
  }
  int e;
  double f = __builtin_frexp(v, &e);                    // v = f * 2^e, f in [0.5, 1)
  // v = 2^(e-1) * (1 + m/8): m = rint(16 f) - 8 (may round to 8: carries into the exponent)
  uint32_t m = (uint32_t)__builtin_rint(f * 16.0) - 8u;
  uint32_t code = ((uint32_t)(e - 1 + 7) << 3) + m;
  return code > 0x7Eu ? 0x7Eu : code;
}

// Largest BF16 value <= t (t > 0, double), as its bit pattern, and whether it equals t.
__host__ __device__ __forceinline__ uint32_t bf16_round_down_bits(double t, bool* exact) {
  int e;
  (void)__builtin_frexp(t, &e);                         // t in [2^(e-1), 2^e)
  int ulp_exp = e - 8;                                  // BF16: 8 significant bits
  if (ulp_exp < -133) ulp_exp = -133;                   // BF16 subnormal spacing 2^-133
  double n = __builtin_floor(__builtin_ldexp(t, -ulp_exp));
  double rd = __builtin_ldexp(n, ulp_exp);              // exactly representable in BF16
  *exact = (rd == t);
  return __builtin_bit_cast(uint32_t, (float)rd) >> 16;
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  for (int o = 32; o > 0; o >>= 1) {
    uint32_t w = (uint32_t)__shfl_xor((int)v, o, 64);
    v = v > w ? v : w;
  }
  return v;
}

}  // namespace nvfp4

// Host-side helpers shared by the entry points.
#define NVFP4_CHECK_LAUNCH()                                  \
  do {                                                        \
    if (hipGetLastError() != hipSuccess) return NVFP4_ERR_HIP; \
  } while (0)

static inline bool nvfp4_aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
static inline size_t nvfp4_align256(size_t n) { return (n + 255) & ~(size_t)255; }
