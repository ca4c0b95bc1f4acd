// Host-side check of the quantizer's exact rounding helpers (quant_block.h),
// built and run by test_quant_block_host.py on the CPU. No kernel is launched.
// * Two-elements-per-word E2M1 index selection. Reference: the index of a
//   BF16 magnitude a is the number of E2M1 midpoint thresholds U_j (BF16 bit
//   patterns, non-decreasing in j) with a > U_j; the nibble is
//   (sign << 3) | index.
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
    for (uint32_t lo = 0; lo < 0x10000u; ++lo) {
      const uint32_t hi = (uint32_t)(rng() & 0xFFFFu);
      if ((lo & 0x7FFFu) > 0x7F80u || (hi & 0x7FFFu) > 0x7F80u) continue;  // finite BF16 only
      for (int swap = 0; swap < 2; ++swap) {
        const uint32_t l = swap ? hi : lo, h = swap ? lo : hi;
        const uint32_t got = (nibble_pair(l | (h << 16), cc) >> 8) & 0xFFu;
        const uint32_t want = count_nibble(l, U) | (count_nibble(h, U) << 4);
        ++n;
        if (got != want && ++bad <= 5) printf("mismatch: word %08x -> %02x, expected %02x\n", l | (h << 16), got, want);
      }
    }
  }
  for (int t = 0; t < 100000; ++t) {
    uint32_t w[8], want = 0;
    for (int j = 0; j < 8; ++j) {
      w[j] = (uint32_t)rng();
      want = std::max(want, std::max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
    }
    if (block_max_bits(w) != want && ++bad <= 5) printf("block max mismatch\n");
    uint32_t r[4];
    for (int j = 0; j < 4; ++j) r[j] = (uint32_t)rng();
    const uint32_t p = pack_pairs(r[0], r[1], r[2], r[3]);
    for (int j = 0; j < 4; ++j)
      if (((p >> (8 * j)) & 0xFFu) != ((r[j] >> 8) & 0xFFu) && ++bad <= 5) printf("pack mismatch\n");
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
  printf("pairs %ld mismatches %ld\n", n, bad);
  return bad != 0;
}
