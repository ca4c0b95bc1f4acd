// Host-side check of the quantizer's two-elements-per-word E2M1 index
// selection (quant_block.h), built and run by test_quant_block_host.py on the
// CPU. Reference: the index of a BF16 magnitude a is the number of E2M1
// midpoint thresholds U_j (BF16 bit patterns, non-decreasing in j) with
// a > U_j, and the nibble is (sign << 3) | index. No kernel is launched.
#include <algorithm>
#include <cstdio>
#include <random>

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
  printf("pairs %ld mismatches %ld\n", n, bad);
  return bad != 0;
}
