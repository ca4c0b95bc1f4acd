// Host-side check of the quantizer's exact rounding helpers (quant_block.h),
// built and run by test_quant_block_host.py on the CPU. No kernel is launched.
// * E2M1 index by binary search, two elements per word, packed with byte
//   permutes. Reference: the index of a BF16 magnitude a is the number of E2M1
//   midpoint thresholds U_j (BF16 bit patterns, non-decreasing in j) with
//   a > U_j; the nibble is (sign << 3) | index.
// * The block scale code from a float32 estimate and two table tests.
//   Reference: the number of E4M3 midpoints 3 * (E(c) + E(c + 1)) * gs that
//   the block maximum B passes (B > it, or B equal to it with c odd), each
//   product exact in float64; also the float64 quotient route.
// * The float32 round-down of threshold products to BF16. Reference: the
//   float64 route (the product is exact in float64).
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <random>
#include <vector>

#include "../nvfp4_quantized_moe_amd/csrc/quant_block.h"

using namespace nvfp4;

static uint32_t count_nibble(uint32_t bits, const uint32_t U[7]) {
  const uint32_t a = bits & 0x7FFFu;
  uint32_t m = 0;
  for (int j = 0; j < 7; ++j) m += a > U[j] ? 1u : 0u;
  return ((bits >> 12) & 8u) | m;
}

// E4M3 code c as a float64, from its fields
static double e4m3_ref(int c) {
  const int e = (c >> 3) & 15, f = c & 7;
  return e == 0 ? f * std::ldexp(1.0, -9) : std::ldexp(1.0 + f / 8.0, e - 7);
}

// every finite block maximum 0 .. 0x7F7F against the scale code reference at gs
static long check_scale_codes(float gs, long* n) {
  uint32_t lut[kLutWords];
  for (int i = 0; i < kLutWords; ++i) lut[i] = threshold_lut_word(gs, i);
  const QuantScale qs = quant_scale(gs);
  long bad = 0;
  int ref = 0;  // nondecreasing in the block maximum
  for (uint32_t bm = 0; bm < 0x7F80u; ++bm) {
    const double B = (double)__builtin_bit_cast(float, bm << 16);
    if (gs > 0.0f) {
      while (ref < 126) {
        const double t = 3.0 * (e4m3_ref(ref) + e4m3_ref(ref + 1)) * (double)gs;  // exact
        if (B > t || (B == t && (ref & 1))) ++ref;
        else break;
      }
    }
    const uint32_t got = block_scale_code(bm, qs, lut);
    const uint32_t quot = gs > 0.0f ? e4m3_encode_rne_sat(B / (6.0 * (double)gs)) : 0u;
    ++*n;
    if ((got != (uint32_t)ref || quot != (uint32_t)ref) && ++bad <= 5)
      printf("scale code mismatch: gs %a bmax %04x -> %u, expected %d (quotient route %u)\n", gs, bm, got, ref, quot);
  }
  return bad;
}

int main(int argc, char** argv) {
  const int sets = argc > 1 ? atoi(argv[1]) : 200;
  std::mt19937_64 rng(20261203);
  long n = 0, bad = 0;
  for (int t = 0; t < sets; ++t) {
    uint32_t U[7];
    for (int j = 0; j < 7; ++j) {
      switch (t % 5) {
        case 0: U[j] = rng() % 0x8000; break;                          // anywhere
        case 1: U[j] = 0x7F00 + rng() % 0x100; break;                  // near and past 0x7FFF
        case 2: U[j] = rng() % 64; break;                              // tiny, with repeats
        case 3: U[j] = (rng() % 3 == 0) ? 0xFFFFu : rng() % 0x8000; break;  // some never passed
        default: U[j] = 0xFFFFu; break;                                // scale code 0: nothing passes
      }
    }
    std::sort(U, U + 7);
    uint32_t cc[7];
    for (int j = 0; j < 7; ++j) cc[j] = threshold_offset_pair(U[j]);
    // element k of eight takes every BF16 pattern in turn, the others random
    for (uint32_t v = 0; v < 0x10000u; ++v) {
      if ((v & 0x7FFFu) > 0x7F80u) continue;  // finite BF16 only
      uint32_t e[8];
      for (int k = 0; k < 8; ++k) {
        do e[k] = (uint32_t)(rng() & 0xFFFFu); while ((e[k] & 0x7FFFu) > 0x7F80u);
      }
      e[v % 8] = v;
      uint32_t w[4];
      for (int k = 0; k < 4; ++k) w[k] = e[2 * k] | (e[2 * k + 1] << 16);
      const uint32_t got = pack_quads(nibble_quad(w[0], w[1], cc), nibble_quad(w[2], w[3], cc));
      uint32_t want = 0;
      for (int k = 0; k < 8; ++k) want |= count_nibble(e[k], U) << (4 * k);
      ++n;
      if (got != want && ++bad <= 5) printf("nibble mismatch: %08x %08x %08x %08x -> %08x, expected %08x\n",
                                            w[0], w[1], w[2], w[3], got, want);
    }
  }
  for (int t = 0; t < 100000; ++t) {
    uint32_t w[8], want = 0;
    for (int j = 0; j < 8; ++j) {
      w[j] = (uint32_t)rng();
      want = std::max(want, std::max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
    }
    if (block_max_bits(w) != want && ++bad <= 5) printf("block max mismatch\n");
  }
  // block scale codes: fixed, random and tie-making global scales, also
  // outside [2^-60, 2^60] (the float64 route) and gs = 0
  {
    std::vector<float> gss = {0.0f, 1.0f, 0.5f, 2000.0f / 2688.0f, 0x1p-60f, 0x1p60f, 0x1.fffffep-61f, 0x1p-126f,
                              1e-40f, 0x1p100f, 3.0e38f / 2688.0f};
    for (int i = 0; i < 120; ++i) gss.push_back(__builtin_bit_cast(float, 0x00800000u + (uint32_t)(rng() % 0x7E800000u)));
    for (int i = 0; i < 120; ++i) {
      // block maximum B exactly on the midpoint of codes c, c+1 at gs = B / (3 (E(c) + E(c+1)))
      const int c = (int)(rng() % 126);
      const float m = (float)(3.0 * (e4m3_ref(c) + e4m3_ref(c + 1)));
      const float B = __builtin_bit_cast(float, (0x2000u + (uint32_t)(rng() % 0x3000u)) << 16);
      const uint32_t gb = __builtin_bit_cast(uint32_t, B / m);
      for (int d = -1; d <= 1; ++d) gss.push_back(__builtin_bit_cast(float, gb + d));
    }
    for (float g : gss) bad += check_scale_codes(g, &n);
  }
  // threshold table entries: the float32 product-and-residual round-down to
  // BF16 against the float64 route, for every E2M1 midpoint x E4M3 scale value
  // and global scales over the float32 range, also ones that put the product
  // on a BF16 value or one float32 step from it (the ties)
  {
    const float mids[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
    std::vector<float> ms, gss = {1.0f, 0.5f, 2000.0f / 2688.0f, 1e-30f, 1e-38f, 0x1p-100f, 0x1p-99f, 1e35f};
    for (int c = 1; c <= 0x7E; ++c) {
      const int e = (c >> 3) & 15, f = c & 7;
      const double v = e == 0 ? f * std::ldexp(1.0, -9) : std::ldexp(1.0 + f / 8.0, e - 7);
      for (float md : mids) ms.push_back((float)(md * v));
    }
    for (int i = 0; i < 300; ++i) gss.push_back(__builtin_bit_cast(float, 0x00800000u + (uint32_t)(rng() % 0x7C000000u)));
    for (int i = 0; i < 300; ++i) {
      const float m = ms[rng() % ms.size()];
      const float target = __builtin_bit_cast(float, (0x3000u + (uint32_t)(rng() % 0x1800u)) << 16);
      const uint32_t gb = __builtin_bit_cast(uint32_t, target / m);
      for (int d = -2; d <= 2; ++d) gss.push_back(__builtin_bit_cast(float, gb + d));
    }
    for (float g : gss)
      for (float m : ms) {
        bool e1, e2;
        const uint32_t a = bf16_round_down_product(m, g, &e1);
        const uint32_t b = bf16_round_down_bits((double)m * (double)g, &e2);
        ++n;
        if ((a != b || e1 != e2) && ++bad <= 5) printf("round-down mismatch: %a * %a\n", m, g);
      }
  }
  // the E2M1 part of the table: every scale code's four words expand to the
  // seven offset pairs of its midpoints
  {
    const float mids[7] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f};
    const float gss[] = {0.0f, 1.0f, 2000.0f / 2688.0f, 0x1p-60f, 1e-40f, 3.0e38f / 2688.0f, 0.3f, 7.1e-3f};
    for (float g : gss) {
      uint32_t lut[kLutWords];
      for (int i = 0; i < kLutWords; ++i) lut[i] = threshold_lut_word(g, i);
      for (int code = 0; code < 128; ++code) {
        uint32_t cc[7];
        const uint4 t = make_uint4(lut[4 * code], lut[4 * code + 1], lut[4 * code + 2], lut[4 * code + 3]);
        e2m1_offsets(t, cc);
        for (int j = 0; j < 7; ++j) {
          uint32_t want = 0;
          if (code > 0 && code <= 0x7E && g > 0.0f)
            want = threshold_offset_pair(midpoint_threshold((float)(mids[j] * e4m3_ref(code)), g, (j & 1) != 0));
          ++n;
          if (cc[j] != want && ++bad <= 5) printf("table mismatch: gs %a code %d midpoint %d\n", g, code, j);
        }
      }
    }
  }
  printf("pairs %ld mismatches %ld\n", n, bad);
  return bad != 0;
}
