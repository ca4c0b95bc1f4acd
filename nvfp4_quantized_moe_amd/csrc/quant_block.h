// Exact NVFP4 rounding of 16-element BF16 blocks against a global scale gs,
// shared by the quantizer kernels and the GEMM epilogue that writes NVFP4.
//
// nvfp4_mega_moe.py history, three-quantizer-bugs commit: stored scale =
// block_max / 6 (after normalization by gs), nearest E2M1 magnitude, sign in
// bit 3 of the nibble; overflow-fix commit: scales saturate at 448.
//
// Both roundings are decided exactly, as on the real quotients:
//   sf = nearest E4M3 (ties even, saturating) to bmax / (6 gs)
//   m  = nearest E2M1 index (ties even) to |x| / (E4M3(sf) gs)
// The scale comes from a float64 quotient (an E4M3 value or midpoint has at
// most 5 significant bits, so the quotient of a BF16 by 6*gs that is not one
// of them lies >= 2^-32 away relative; float64 rounding cannot move it across).
// The magnitude is a count of E2M1 midpoints c*E4M3(sf)*gs passed; each
// midpoint (3 x 4 x 24 significant bits) is turned exactly, from a float32
// product and its fma residual, into a BF16 bit-pattern threshold U such that
// |x| passes it iff bits(|x|) > U.
//
// Two elements per 32-bit word: a BF16 magnitude a has bits <= 0x7FFF, so
// with C = 0x7FFF - U (<= 0x7FFF) the sum a + C stays below 2^16 and has bit
// 15 set iff a > U. One 32-bit add of (C | C << 16) to the word holding two
// magnitudes therefore tests both against one threshold, with no carry
// between the halves. The thresholds increase with the midpoint, so the seven
// tests of an element form a thermometer code, and the 3-bit index is read
// from it with bit selects (a binary search over the results).
#pragma once
#include "common.h"

namespace nvfp4 {

// 128 scale codes x 8 words (word 7 unused)
constexpr int kLutWords = 128 * 8;
constexpr int kLutBytes = kLutWords * 4;

// Offset word for threshold U (0xFFFF or any U >= 0x7FFF: nothing passes).
__host__ __device__ __forceinline__ uint32_t threshold_offset_pair(uint32_t u) {
  const uint32_t c = u >= 0x7FFFu ? 0u : 0x7FFFu - u;
  return c | (c << 16);
}

// Largest BF16 value <= m * gs (m a float32 with at most 7 significant bits,
// gs > 0 finite, both positive), as its bit pattern, and whether it equals
// m * gs. The float32 product hi and its exact residual fma(m, gs, -hi) give
// the real product; hi with its low 16 bits cleared is a BF16 value <= hi,
// and below the real product unless it equals hi and the residual is
// negative. Products under 2^-100 (where the residual may not be exact) or
// past the float32 range take the float64 route.
__host__ __device__ __forceinline__ uint32_t bf16_round_down_product(float m, float gs, bool* exact) {
  const float hi = m * gs;
  if (!(hi >= 0x1p-100f && hi <= 0x1.fffffep127f))
    return bf16_round_down_bits((double)m * (double)gs, exact);  // exact in float64
  const float lo = __builtin_fmaf(m, gs, -hi);
  const uint32_t hb = __builtin_bit_cast(uint32_t, hi);
  const bool on_bf16 = (hb & 0xFFFFu) == 0u;
  *exact = on_bf16 && lo == 0.0f;
  return (hb >> 16) - (on_bf16 && lo < 0.0f ? 1u : 0u);
}

// Threshold table for global scale gs: entry `code`, word j < 7, holds the
// offset pair of E2M1 midpoint j of that scale code (all zero, so that
// nothing passes, for code 0 and for gs <= 0 or NaN). Threads tid = 0 ..
// nthreads-1 fill it together; the caller synchronises.
__device__ __forceinline__ void build_threshold_lut(float gs, uint32_t* lut, int tid, int nthreads) {
  for (int i = tid; i < kLutWords; i += nthreads) {
    const int code = i >> 3, j = i & 7;
    uint32_t u = 0xFFFFu;
    if (j < 7 && code > 0 && code <= 0x7E && gs > 0.0f) {
      // E2M1 midpoint j (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5); an exact tie
      // rounds up at the odd j (0.75, 1.75, 3.5: the upper code is even)
      const float mid = j < 4 ? 0.25f + 0.5f * j : (j == 6 ? 5.0f : j - 1.5f);
      const bool tie_up = (j & 1) != 0;
      // midpoint times the scale value: 3 x 4 significant bits, exact in float32
      const float ms = mid * e4m3_to_f32((uint32_t)code);
      bool exact;
      const uint32_t rd = bf16_round_down_product(ms, gs, &exact);
      // strict midpoint: |x| > thr  <=>  bits > bits(RD(thr))
      // tie-up midpoint: |x| >= thr <=>  bits > bits(RU(thr)) - 1
      u = (tie_up && exact) ? rd - 1u : rd;
    }
    lut[i] = threshold_offset_pair(u);
  }
}

// (m & a) | (~m & b), one v_bfi_b32
__host__ __device__ __forceinline__ uint32_t bit_select(uint32_t m, uint32_t a, uint32_t b) {
  return (m & a) | (~m & b);
}

// Nibbles of the two elements of word w (element 2i in the low half) from the
// offset pairs cc[0..6] of their block's scale code. Returns a word whose
// byte 1 is (nibble of element 2i+1) << 4 | nibble of element 2i.
__host__ __device__ __forceinline__ uint32_t nibble_pair(uint32_t w, const uint32_t cc[7]) {
  const uint32_t a = w & 0x7FFF7FFFu;
  uint32_t p[7];  // bit 15 / 31: the low / high element passes midpoint j
#pragma unroll
  for (int j = 0; j < 7; ++j) p[j] = a + cc[j];
  // index m = number of midpoints passed, from the thermometer code:
  //   bit 2 = p3;  bit 1 = p3 ? p5 : p1;  bit 0 = p3 ? (p5 ? p6 : p4) : (p1 ? p2 : p0)
  const uint32_t m1 = bit_select(p[3], p[5], p[1]);
  const uint32_t m0 = bit_select(p[3], bit_select(p[5], p[6], p[4]), bit_select(p[1], p[2], p[0]));
  // sign, m2, m1, m0 at bits 15..12 (low element) and 31..28 (high element)
  constexpr uint32_t kTop = 0x80008000u;
  uint32_t z = bit_select(kTop, m1, m0 >> 1);
  z = bit_select(kTop, p[3], z >> 1);
  z = bit_select(kTop, w, z >> 1);
  return bit_select(0xF000u, z >> 16, z >> 4);
}

// Largest BF16 magnitude of a block, as bits: w[j] holds elements 2j (low
// half) and 2j+1 (high half). Maxima of both halves at once (v_pk_max_u16).
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__host__ __device__ __forceinline__ uint32_t block_max_bits(const uint32_t w[8]) {
  u16x2_t m = __builtin_bit_cast(u16x2_t, w[0] & 0x7FFF7FFFu);
#pragma unroll
  for (int j = 1; j < 8; ++j) m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, w[j] & 0x7FFF7FFFu));
  return m[0] > m[1] ? m[0] : m[1];
}

// Packs byte 1 of four nibble_pair results into one word (bytes in order).
__host__ __device__ __forceinline__ uint32_t pack_pairs(uint32_t r0, uint32_t r1, uint32_t r2, uint32_t r3) {
  return ((r0 >> 8) & 0xFFu) | (r1 & 0xFF00u) | ((r2 << 8) & 0xFF0000u) | ((r3 << 16) & 0xFF000000u);
}

// One block: w[j] holds elements 2j (low half) and 2j+1 (high half) as BF16.
// Writes the 16 nibbles (element 2j in the low nibble of byte j) to *out and
// returns the scale code. six_gs = 6 * (double)gs; lut is the table of gs.
__device__ __forceinline__ uint32_t quantize_block16(const uint32_t w[8], float gs, double six_gs, const uint4* lut,
                                                     uint2* out) {
  const uint32_t bmax = block_max_bits(w);
  uint32_t code = 0;
  if (gs > 0.0f) code = e4m3_encode_rne_sat((double)bf16_to_f32(bmax) / six_gs);
  const uint4 t0 = lut[2 * code], t1 = lut[2 * code + 1];
  const uint32_t cc[7] = {t0.x, t0.y, t0.z, t0.w, t1.x, t1.y, t1.z};
  uint32_t r[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = nibble_pair(w[j], cc);
  *out = make_uint2(pack_pairs(r[0], r[1], r[2], r[3]), pack_pairs(r[4], r[5], r[6], r[7]));
  return code;
}

}  // namespace nvfp4
