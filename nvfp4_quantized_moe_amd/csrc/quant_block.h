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
// Each is a count of rounding midpoints passed. A midpoint times gs (at most
// 7 x 24 significant bits) is turned exactly, from a float32 product and its
// fma residual, into a BF16 bit-pattern threshold U such that a BF16
// magnitude passes it iff its bits are > U.
//
// Two magnitudes per 32-bit word: a BF16 magnitude a has bits <= 0x7FFF, so
// with C = 0x7FFF - U (<= 0x7FFF) the sum a + C stays below 2^16 and has bit
// 15 set iff a > U. One 32-bit add of a per-half pair of such offsets to the
// word holding two magnitudes tests both, with no carry between the halves.
//
// Scale code: a float32 estimate of bmax / (6 gs) rounded to a code c is
// within one code of the exact one (its relative error is ~2^-23, and the
// E4M3 midpoints are 2^-4 apart relative), so the exact code is
// c - 1 + [bmax passes the midpoint below c] + [bmax passes the one above],
// both tested with one add against a table word.
//
// E2M1 index: the midpoint thresholds increase with the index, so the index
// is found by a binary search of three tests (midpoint 3, then 5 or 1, then
// 6, 4, 2 or 0), each an add of thresholds picked per half with byte masks.
// v_perm_b32's sign-byte selects turn the test bits of two words into one
// byte per element, and three bit selects and two byte permutes build the
// packed nibbles.
#pragma once
#include "common.h"

namespace nvfp4 {

// Threshold table in LDS: words [0, 512) hold 16-bit E2M1 midpoint offsets,
// four words (seven offsets and a spare) per scale code; word kScaleWords + c
// (c <= 126) holds the two E4M3 midpoint offsets that settle a scale-code
// estimate c. 16-bit entries keep the per-block reads to 20 bytes.
constexpr int kScaleWords = 512;
constexpr int kLutWords = kScaleWords + 128;
constexpr int kLutBytes = kLutWords * 4;

// Offset of threshold U in one 16-bit half (0 for U >= 0x7FFF: nothing passes).
__host__ __device__ __forceinline__ uint32_t threshold_offset(uint32_t u) {
  return u >= 0x7FFFu ? 0u : 0x7FFFu - u;
}
// The same offset in both halves.
__host__ __device__ __forceinline__ uint32_t threshold_offset_pair(uint32_t u) {
  const uint32_t c = threshold_offset(u);
  return c | (c << 16);
}
// An offset that every magnitude (0 included) passes: a + 0x8000 has bit 15
// set and, as a <= 0x7FFF, stays below 2^16.
constexpr uint32_t kAlwaysPasses = 0x8000u;

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

// Threshold U (BF16 bits) of midpoint value m * gs (m > 0 with at most 7
// significant bits): a magnitude a passes iff bits(a) > U, where passing
// means a > m * gs, or a >= m * gs when an exact tie rounds up.
__host__ __device__ __forceinline__ uint32_t midpoint_threshold(float m, float gs, bool tie_up) {
  bool exact;
  const uint32_t rd = bf16_round_down_product(m, gs, &exact);
  // strict midpoint: |x| > thr  <=>  bits > bits(RD(thr))
  // tie-up midpoint: |x| >= thr <=>  bits > bits(RU(thr)) - 1
  return (tie_up && exact) ? rd - 1u : rd;
}

// Exact value of E4M3 code c (0 <= c <= 0x7E) as float32.
__host__ __device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, f = c & 7u;
  return e == 0 ? (float)f * 0x1p-9f : __builtin_ldexpf(1.0f + 0.125f * (float)f, (int)e - 7);
}

// Offset of the E4M3 rounding midpoint between scale codes c and c + 1
// (0 <= c <= 125), at 6 * gs: a block maximum passes it iff its nearest code
// is above c. An exact tie rounds to the even code, i.e. up when c is odd.
// 6 * (E4M3(c) + E4M3(c + 1)) / 2 has at most 7 significant bits.
__host__ __device__ __forceinline__ uint32_t scale_midpoint_offset(int c, float gs) {
  if (!(gs > 0.0f)) return 0u;
  const float m = 3.0f * (e4m3_value((uint32_t)c) + e4m3_value((uint32_t)c + 1u));
  return threshold_offset(midpoint_threshold(m, gs, (c & 1) != 0));
}

// E2M1 midpoint j (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5) of scale code `code`
// as a 16-bit offset (0, so that nothing passes, for code 0 and for gs <= 0
// or NaN); an exact tie rounds up at the odd j (0.75, 1.75, 3.5: the upper
// E2M1 code is even). The midpoint times the scale value has 3 x 4
// significant bits, exact in float32.
__host__ __device__ __forceinline__ uint32_t e2m1_midpoint_offset(int code, int j, float gs) {
  if (!(code > 0 && code <= 0x7E && gs > 0.0f)) return 0u;
  const float mid = j < 4 ? 0.25f + 0.5f * j : (j == 6 ? 5.0f : j - 1.5f);
  return threshold_offset(midpoint_threshold(mid * e4m3_value((uint32_t)code), gs, (j & 1) != 0));
}

// Word i of the threshold table for global scale gs: for i < kScaleWords,
// offsets of midpoints 2(i%4) (low half) and 2(i%4)+1 (high half) of scale
// code i/4 (the high half of the fourth word is unused); word kScaleWords + c:
// the offset of the scale midpoint below c in the low half (one that always
// passes for c = 0) and of the one above c in the high half (none for
// c >= 126). Threads tid = 0 .. nthreads-1 fill it together; the caller
// synchronises.
__host__ __device__ __forceinline__ uint32_t threshold_lut_word(float gs, int i) {
  if (i >= kScaleWords) {
    const int c = i - kScaleWords;
    const uint32_t lo = c == 0 ? kAlwaysPasses : scale_midpoint_offset(c - 1, gs);
    const uint32_t hi = c >= 126 ? 0u : scale_midpoint_offset(c, gs);
    return lo | (hi << 16);
  }
  const int code = i >> 2, j = 2 * (i & 3);
  return e2m1_midpoint_offset(code, j, gs) | (j + 1 < 7 ? e2m1_midpoint_offset(code, j + 1, gs) << 16 : 0u);
}
__device__ __forceinline__ void build_threshold_lut(float gs, uint32_t* lut, int tid, int nthreads) {
  for (int i = tid; i < kLutWords; i += nthreads) lut[i] = threshold_lut_word(gs, i);
}

// Per-tensor constants of the scale-code estimate: bmax / (6 gs) is taken as
// (bmax * rcp) * 2^nexp with gs = g * 2^-nexp, g in [0.5, 1) and rcp =
// RN(1 / (6 g)). For gs in [2^-60, 2^60] a product that loses precision
// below the float32 normal range stands for a quotient below 2^-66, whose
// code is 0 either way; other positive gs take the float64 quotient and the
// exact encoder. gs <= 0 gives the estimate 0 (and code 0 with its table).
struct QuantScale {
  float rcp;
  int nexp;
  bool fast;
  double six_gs;
};
__host__ __device__ __forceinline__ QuantScale quant_scale(float gs) {
  QuantScale s;
  s.six_gs = 6.0 * (double)gs;  // exact
  int e = 0;
  const float g = gs > 0.0f ? __builtin_frexpf(gs, &e) : 0.0f;
  s.rcp = gs > 0.0f ? (float)(1.0 / (6.0 * (double)g)) : 0.0f;
  s.nexp = -e;
  s.fast = !(gs > 0.0f) || (gs >= 0x1p-60f && gs <= 0x1p60f);
  return s;
}

// An E4M3 code within one of the nearest code to q >= 0 (saturating at
// 0x7E): below 2^-6 the truncated multiple of 2^-9; above, the float32 bits
// rounded (half up) to 3 mantissa bits, minus the exponent bias difference
// (120 << 3).
__host__ __device__ __forceinline__ uint32_t e4m3_code_near(float q) {
  const uint32_t nrm = ((__builtin_bit_cast(uint32_t, q) + 0x80000u) >> 20) - 960u;
  const uint32_t c = q < 0x1p-6f ? (uint32_t)(q * 512.0f) : nrm;
  return c < 0x7Eu ? c : 0x7Eu;
}

// Exact nearest E4M3 code to bmax / (6 gs) (bmax: BF16 bits of a finite
// block maximum, < 0x7F80): the estimate c, then c - 1 plus the two midpoint
// tests of table word kScaleWords + c.
__host__ __device__ __forceinline__ uint32_t block_scale_code(uint32_t bmax, const QuantScale& qs,
                                                             const uint32_t* lut) {
  const float b = __builtin_bit_cast(float, bmax << 16);
  uint32_t c;
  if (qs.fast)
    c = e4m3_code_near(__builtin_ldexpf(b * qs.rcp, qs.nexp));
  else
    c = e4m3_encode_rne_sat((double)b / qs.six_gs);
  const uint32_t s = (bmax | (bmax << 16)) + lut[kScaleWords + c];
  return c - 1u + ((s >> 15) & 1u) + (s >> 31);
}

// v_perm_b32: byte i of the result is selected by byte i of sel from the
// eight bytes of {s0 (high), s1 (low)}: 0..7 a byte, 8 / 9 / 10 / 11 the sign
// of bit 15 / 31 / 47 / 63 spread over the byte, 12 zero, 13 and above 0xFF.
// The host build (for the CPU check of these helpers) spells the same rule
// out.
__host__ __device__ __forceinline__ uint32_t byte_perm(uint32_t s0, uint32_t s1, uint32_t sel) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_perm(s0, s1, sel);
#else
  const uint64_t in = ((uint64_t)s0 << 32) | s1;
  uint32_t r = 0;
  for (int i = 0; i < 4; ++i) {
    const uint32_t k = (sel >> (8 * i)) & 0xFFu;
    uint32_t b;
    if (k >= 13) b = 0xFFu;
    else if (k == 12) b = 0u;
    else if (k >= 8) b = ((in >> (16 * (k - 8) + 15)) & 1u) ? 0xFFu : 0u;
    else b = (uint32_t)(in >> (8 * k)) & 0xFFu;
    r |= b << (8 * i);
  }
  return r;
#endif
}

// (m & a) | (~m & b): one v_bitop3_b32 with truth table 0xCA (the result
// bit for inputs (m, a, b) is bit 4m + 2a + b of the table), written as the
// builtin so that nested selects stay one instruction each
__host__ __device__ __forceinline__ uint32_t bit_select(uint32_t m, uint32_t a, uint32_t b) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_bitop3_b32(m, a, b, 0xCA);
#else
  return (m & a) | (~m & b);
#endif
}

// Binary search of the E2M1 index of the two magnitudes of a (bits <= 0x7FFF
// per half) over the offset pairs cc[0..6]: index bit 2 is bit 15 / 31 of
// b2 (midpoint 3 passed), bit 1 that of b1 (midpoint 5 or 1), bit 0 that of
// b0 (midpoint 6, 4, 2 or 0).
struct IndexBits {
  uint32_t b2, b1, b0;
};
__host__ __device__ __forceinline__ IndexBits index_search(uint32_t a, const uint32_t cc[7]) {
  constexpr uint32_t kHalfSigns = 0x09090808u;  // each half filled with its bit 15
  const uint32_t b2 = a + cc[3];
  const uint32_t m2 = byte_perm(b2, b2, kHalfSigns);
  const uint32_t b1 = a + bit_select(m2, cc[5], cc[1]);
  const uint32_t m1 = byte_perm(b1, b1, kHalfSigns);
  const uint32_t b0 = a + bit_select(m1, bit_select(m2, cc[6], cc[2]), bit_select(m2, cc[4], cc[0]));
  return {b2, b1, b0};
}

// Nibbles of words wa, wb (wa: elements 0, 1; wb: elements 2, 3 of a group of
// four) as one byte per element in the order (0, 2, 1, 3): the even elements'
// nibbles in the low half of bytes 0 and 1, the odd elements' in the high
// half of bytes 2 and 3 (the other halves are don't-care).
__host__ __device__ __forceinline__ uint32_t nibble_quad(uint32_t wa, uint32_t wb, const uint32_t cc[7]) {
  const IndexBits pa = index_search(wa & 0x7FFF7FFFu, cc);
  const IndexBits pb = index_search(wb & 0x7FFF7FFFu, cc);
  constexpr uint32_t kSigns = 0x0B090A08u;  // bytes: sign of wa lo, wb lo, wa hi, wb hi
  uint32_t x = bit_select(0x20200202u, byte_perm(pb.b1, pa.b1, kSigns), byte_perm(pb.b0, pa.b0, kSigns));
  x = bit_select(0x40400404u, byte_perm(pb.b2, pa.b2, kSigns), x);
  return bit_select(0x80800808u, byte_perm(wb, wa, kSigns), x);
}

// Eight packed nibbles (element 2i low, 2i+1 high in byte i) from the
// nibble_quad results of elements 0..3 (x) and 4..7 (y).
__host__ __device__ __forceinline__ uint32_t pack_quads(uint32_t x, uint32_t y) {
  const uint32_t even = byte_perm(y, x, 0x05040100u);  // elements 0, 2, 4, 6
  const uint32_t odd = byte_perm(y, x, 0x07060302u);   // elements 1, 3, 5, 7
  return bit_select(0x0F0F0F0Fu, even, odd);
}

// Largest BF16 magnitude of a block, as bits: w[j] holds elements 2j (low
// half) and 2j+1 (high half). Maxima of both halves at once (v_pk_max_u16),
// as a tree.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__host__ __device__ __forceinline__ uint32_t block_max_bits(const uint32_t w[8]) {
  u16x2_t m[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) m[j] = __builtin_bit_cast(u16x2_t, w[j] & 0x7FFF7FFFu);
#pragma unroll
  for (int s = 1; s < 8; s *= 2)
#pragma unroll
    for (int j = 0; j < 8; j += 2 * s) m[j] = __builtin_elementwise_max(m[j], m[j + s]);
  return m[0][0] > m[0][1] ? m[0][0] : m[0][1];
}

// The seven E2M1 offset pairs of scale code `code` from its four table words
// (each 16-bit offset copied into both halves by a byte permute).
__host__ __device__ __forceinline__ void e2m1_offsets(const uint4& t, uint32_t cc[7]) {
  constexpr uint32_t kLo = 0x01000100u, kHi = 0x03020302u;
  cc[0] = byte_perm(t.x, t.x, kLo);
  cc[1] = byte_perm(t.x, t.x, kHi);
  cc[2] = byte_perm(t.y, t.y, kLo);
  cc[3] = byte_perm(t.y, t.y, kHi);
  cc[4] = byte_perm(t.z, t.z, kLo);
  cc[5] = byte_perm(t.z, t.z, kHi);
  cc[6] = byte_perm(t.w, t.w, kLo);
}

// One block: w[j] holds elements 2j (low half) and 2j+1 (high half) as BF16.
// Writes the 16 nibbles (element 2j in the low nibble of byte j) to *out and
// returns the scale code. qs = quant_scale(gs); lut is the table of gs.
__device__ __forceinline__ uint32_t quantize_block16(const uint32_t w[8], const QuantScale& qs, const uint4* lut,
                                                     uint2* out) {
  const uint32_t code = block_scale_code(block_max_bits(w), qs, reinterpret_cast<const uint32_t*>(lut));
  uint32_t cc[7];
  e2m1_offsets(lut[code], cc);
  *out = make_uint2(pack_quads(nibble_quad(w[0], w[1], cc), nibble_quad(w[2], w[3], cc)),
                    pack_quads(nibble_quad(w[4], w[5], cc), nibble_quad(w[6], w[7], cc)));
  return code;
}

}  // namespace nvfp4
