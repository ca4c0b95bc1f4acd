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
// midpoint is exact in float64 (3 x 4 x 24 significant bits) and is turned
// into a BF16 bit-pattern threshold U such that |x| passes it iff
// bits(|x|) > U; a table of 7 thresholds per scale code (127 codes) lives in
// LDS, so the per-element work is seven integer compares.
#pragma once
#include "common.h"

namespace nvfp4 {

// Threshold table for global scale gs, as 128 entries of 8 BF16 bit patterns
// (entry `code`, slot j < 7: |x| passes E2M1 midpoint j of that scale code iff
// bits(|x|) > U; 0xFFFF where nothing passes, also for gs <= 0 or NaN).
// Threads tid = 0 .. nthreads-1 fill it together; the caller synchronises.
__device__ __forceinline__ void build_threshold_lut(float gs, uint16_t* lut, int tid, int nthreads) {
  for (int i = tid; i < 128 * 8; i += nthreads) {
    const int code = i >> 3, j = i & 7;
    uint32_t u = 0xFFFFu;
    if (j < 7 && code > 0 && code <= 0x7E && gs > 0.0f) {
      // E2M1 midpoint j (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5); an exact tie
      // rounds up at the odd j (0.75, 1.75, 3.5: the upper code is even)
      const double mid = j < 4 ? 0.25 + 0.5 * j : (j == 6 ? 5.0 : j - 1.5);
      const bool tie_up = (j & 1) != 0;
      const double step = (double)e4m3_to_f32((uint32_t)code) * (double)gs;  // exact
      const double thr = mid * step;                                          // exact
      bool exact;
      const uint32_t rd = bf16_round_down_bits(thr, &exact);
      // strict midpoint: |x| > thr  <=>  bits > bits(RD(thr))
      // tie-up midpoint: |x| >= thr <=>  bits > bits(RU(thr)) - 1
      u = (tie_up && exact) ? rd - 1u : rd;
    }
    lut[i] = (uint16_t)u;
  }
}

// One block: w[j] holds elements 2j (low half) and 2j+1 (high half) as BF16.
// Writes the 16 nibbles (element 2j in the low nibble of byte j) to *out and
// returns the scale code. six_gs = 6 * (double)gs.

__device__ __forceinline__ uint32_t quantize_block16(const uint32_t w[8], float gs, double six_gs, const uint4* lut,
                                                     uint2* out) {
  uint32_t bmax = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) bmax = max(bmax, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
  uint32_t code = 0;
  if (gs > 0.0f) code = e4m3_encode_rne_sat((double)bf16_to_f32(bmax) / six_gs);
  const uint4 tv = lut[code];
  const uint32_t U[7] = {tv.x & 0xFFFFu, tv.x >> 16, tv.y & 0xFFFFu, tv.y >> 16,
                         tv.z & 0xFFFFu, tv.z >> 16, tv.w & 0xFFFFu};
  uint32_t packed[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const uint32_t bits = (e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu);
    const uint32_t a = bits & 0x7FFFu;
    uint32_t m = 0;
#pragma unroll
    for (int j = 0; j < 7; ++j) m += (a > U[j]) ? 1u : 0u;
    const uint32_t nib = ((bits >> 12) & 8u) | m;
    packed[e >> 3] |= nib << (4 * (e & 7));
  }
  *out = make_uint2(packed[0], packed[1]);
  return code;
}

}  // namespace nvfp4
