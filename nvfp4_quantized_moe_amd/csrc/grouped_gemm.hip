// NVFP4 x NVFP4 grouped GEMM over slot rows (steps a4/a5 and a7 of the layer).
//
// nvfp4_mega_moe.py history, alpha commit: D = alpha * A @ B with alpha the
//   product of the two global scales, applied in the epilogue.
// src history, 1-D slot-id and gather commits: one 1-D slot order; L1 reads
//   activation rows through slot_token (a gather folded into the tile load),
//   L2 reads its rows in slot order.
// tests history, NVFP4-native layer-test commit: tokens of one expert form a
//   contiguous block of rows; each expert's block is a separate GEMM.
// nvfp4_cutedsl.py history, intermediate-split commit: gate = columns [0, I),
//   up = columns [I, 2I) of the L1 output; the fused epilogue pairs them.
//
// Why fp16 MFMA: a block-16 E4M3 scale does not map onto gfx950's block-32
// E8M0 scaled MFMA, and E2M1 x E4M3 products need up to 6 significant bits
// (more than FP8 holds). Every product lies in [2^-10, 2688], so it is exact
// in fp16; the GEMM therefore decodes both operands to fp16 exactly and uses
// v_mfma_f32_32x32x16_f16 with float32 accumulation. Decoding one byte (two
// values) is v_cvt_scalef32_pk_f16_fp4 with scale 1 (that instruction applies
// only the exponent of its scale operand) and one v_pk_mul_f16 by the E4M3
// scale converted to fp16 (exact).
//
// Structure: a persistent grid walks work items (row tile from the device
// tile table x column tile); block ids are remapped so that each XCD (own L2)
// takes a contiguous run of items, whose row tiles share the expert's weight
// tile. Each item streams K in stages of 128, and the loads run ahead across
// the items of a workgroup. The row tile's activations (row-major
// NVFP4, gathered through the slot's token) go global -> registers -> LDS as
// fp16, double buffered; every wave reads its A fragments from LDS. Weights
// are stored pre-packed in MFMA fragment order (nvfp4_pack_weights), so each
// wave streams its own 32-row subtiles global -> registers with every load
// instruction reading 1 KB (or 256 B of scales) contiguously, P stages ahead.
// Within a 128-wide stage, lane half g of a wave takes the contiguous K range
// [64g, 64g + 64) across the 8 MFMA steps; A and B use the same assignment,
// so each MFMA step still sums matching K indices.
#include "common.h"
#include "internal.h"
#include "quant_block.h"

namespace nvfp4 {

constexpr int kBK = 128;        // K elements per stage
constexpr int kAPitch = 272;    // LDS bytes per fp16 A row of a stage (256 + 16 padding)
// Packed weights: one chunk per (matrix, 32-row subtile, 128-wide K stage):
// [h = 0, 1][lane 0..63][16 B] FP4 bytes, then [lane 0..63][4 B] scales, where
// lane l holds row 32*sub + l%32, FP4 bytes [32*(l/32) + 16*h, +16) of the
// stage's 64 bytes and scale bytes [4*(l/32), +4) of the stage's 8.
constexpr int kPackChunk = 2304;
constexpr int kPackScaleOff = 2048;

// Internal epilogue: the SiLU*up epilogue writing h as NVFP4 with a fixed
// global scale (h_q, h_sf) instead of BF16 h and its amax.
constexpr int kEpiSiluNvfp4 = 3;

template <int SUB_M, int SUB_N, int WAVES, int P>
struct GemmCfg {
  static constexpr int BM = 32 * SUB_M;            // rows of the row tile
  static constexpr int BN = 32 * SUB_N * WAVES;    // weight rows of the column tile
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int A_TASKS = BM * 4;           // (row, 32-element chunk) per stage
  static constexpr int A_PER_T = (A_TASKS + THREADS - 1) / THREADS;
  static constexpr int LDS = 2 * BM * kAPitch;   // two A buffers (a spare 1 KB follows them)
  static constexpr int LDS_SPARE = 1024;
};

// Buffer resources (gfx9 descriptor): loads at offsets >= num_records return
// zero, so rows past a group's end and column tiles past N need no branches.
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr uint32_t kOutOfRange = 0x80000000u;  // offset that is never in range

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t num_records) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_records, (int)kRsrcWord3);
}
// Address = per-lane voffset + wave-uniform soffset (an SGPR: per-stage and
// per-subtile offsets cost no vector instructions). An out-of-range voffset
// or soffset is >= 2^31, and the other term is below 2^31 whenever it is in
// range, so their 32-bit sum stays out of range (or, when both are out of
// range, wraps to a small in-range offset of a lane whose result is discarded).
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ uint32_t buf_load4(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ uint32_t buf_load2(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
}
// The same loads with the non-temporal cache policy (for data read once).
constexpr int kCachePolicyNT = 2;
__device__ __forceinline__ uint4 buf_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kCachePolicyNT));
}
__device__ __forceinline__ uint32_t buf_load4_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, kCachePolicyNT);
}

__device__ __forceinline__ uint32_t pick_u32(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Four E4M3 scale bytes of a word -> four fp16 values, two per instruction
// (v_cvt_scalef32_pk_f16_fp8 with scale 1: exact for every E4M3 value).
struct Scales4 {
  half2_t lo, hi;  // (s0, s1), (s2, s3)
};
__device__ __forceinline__ Scales4 scales4(uint32_t sw) {
  return {__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, false),
          __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw, 1.0f, true)};
}
// scale i of the four, in both halves of a pair (the multiply broadcasts it)
__device__ __forceinline__ half2_t scale_pair(const Scales4& s, int i) {
  const _Float16 v = i == 0 ? s.lo[0] : i == 1 ? s.lo[1] : i == 2 ? s.hi[0] : s.hi[1];
  half2_t r;
  r[0] = v;
  r[1] = v;
  return r;
}

// 8 E2M1 values (one dword, element 8d..8d+7 in nibble order) times a scale pair
__device__ __forceinline__ half8_t decode8(uint32_t w, half2_t s2) {
  half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
  half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
  half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2);
  half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3);
  p0 *= s2;
  p1 *= s2;
  p2 *= s2;
  p3 *= s2;
  half8_t r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ float silu_f32(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// h = BF16(SiLU(g) * u) with g = BF16(acc_gate * alpha) and u = BF16(acc_up * alpha_up), as BF16 bits
__device__ __forceinline__ uint32_t silu_mul_bf16(float acc_gate, float acc_up, float alpha, float alpha_up) {
  const uint32_t gu = f32x2_to_bf16x2(acc_gate * alpha, acc_up * alpha_up);
  const float g = __uint_as_float(gu << 16), u = __uint_as_float(gu & 0xFFFF0000u);
  return f32_to_bf16(silu_f32(g) * u);
}

// Work item = (row tile from the tile table, column tile). The row tile's
// activations are decoded once per stage into LDS as fp16 and shared by the
// waves; each wave streams its own 32*SUB_N weight rows from global memory
// into registers, P stages ahead, and decodes them just before its MFMAs.
template <int SUB_M, int SUB_N, int WAVES, int P, int EPI>
__global__ __launch_bounds__(64 * WAVES) void grouped_gemm_kernel(
    const uint8_t* __restrict__ a_q, const uint8_t* __restrict__ a_sf, const int32_t* __restrict__ a_row_index,
    const float* __restrict__ a_gs, const uint8_t* __restrict__ b_packed, const float* __restrict__ b_gs,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tile_table, int max_tiles, int N, int K,
    int n_out, int n_ntiles, int col_fastest, int dual_gs, uint16_t* __restrict__ d, float* __restrict__ amax_out,
    uint8_t* __restrict__ d_sf, const float* __restrict__ out_gs) {
  constexpr bool kSilu = EPI != NVFP4_EPI_BF16;  // gate/up pairs, n_out = N / 2
  using C = GemmCfg<SUB_M, SUB_N, WAVES, P>;
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int lr = lane & 31, lg = lane >> 5;

  int ntiles = tile_table[0];
  ntiles = ntiles < max_tiles ? ntiles : max_tiles;
  const int items = ntiles * n_ntiles;
  const int G = gridDim.x;
  // consecutive slots on one XCD: blocks are dispatched round-robin over the XCDs
  const int slot = (G % kXcds == 0) ? (blockIdx.x % kXcds) * (G / kXcds) + blockIdx.x / kXcds : blockIdx.x;
  const int64_t pitch = K / 2, spitch = K / 16;
  const int nstages = K / kBK;
  const uint32_t b_bytes = (uint32_t)((int64_t)N * K / 32 * 18);  // one expert's packed weights
  // activation rows: every valid row offset is below 2^31 (checked on the host)
  const __amdgpu_buffer_rsrc_t ra_q = make_rsrc(a_q, 0x7FFFFFFFu);
  const __amdgpu_buffer_rsrc_t ra_s = make_rsrc(a_sf, 0x7FFFFFFFu);
  const int half_n = N / 2;
  const int S = (nstages + P - 1) / P * P;  // loop stages per item (see below)
  float amax_local = 0.0f;

  // Sources of one work item's stage loads: its expert's weight resource, this
  // thread's activation row offsets and the byte offsets of the wave's weight
  // subtiles at stage 0. A slot past the last item gets sources that read zeros.
  struct Src {
    __amdgpu_buffer_rsrc_t rbw;
    uint32_t a_off[C::A_PER_T], as_off[C::A_PER_T];
    uint32_t b_off[SUB_N];  // byte offset of weight subtile j's stage-0 chunk, or out of range
  };
  // row-tile order: the row tiles of one column tile are adjacent, so the
  // row tiles of one expert share its weight tile in L2 at the same time;
  // column order: adjacent items walk one expert's weights contiguously
  auto tile_of = [&](int item, int& mt, int& nt) {
    mt = col_fastest ? item / n_ntiles : item % ntiles;
    nt = col_fastest ? item % n_ntiles : item / ntiles;
  };
  auto make_src = [&](int item, Src& src) {
    src.rbw = make_rsrc(b_packed, 0u);
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
      src.a_off[i] = kOutOfRange;
      src.as_off[i] = kOutOfRange;
    }
#pragma unroll
    for (int j = 0; j < SUB_N; ++j) src.b_off[j] = kOutOfRange;
    if (item >= items) return;
    int mt, nt;
    tile_of(item, mt, nt);
    const int e = tile_table[1 + 2 * mt];
    const int r0 = tile_table[2 + 2 * mt];
    const int r_end = min(r0 + C::BM, offsets[e + 1]);
    src.rbw = make_rsrc(b_packed + (size_t)e * b_bytes, b_bytes);
    // activation staging task i of this thread: 16 FP4 bytes + 2 scale bytes of
    // row rw + lane/4 per stage. The 64 lanes of a wave cover the 16 rows from
    // rw on; their gather indices are read with scalar loads (clamped to the
    // group), so the wait for them does not also wait for the stage loads in
    // flight, which retire in order on the vector memory counter.
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
      const int rw = (i * C::THREADS + 64 * wave) >> 2;  // wave-uniform
      if (rw >= C::BM) continue;
      const int row = rw + (lane >> 2);
      uint32_t ar = (uint32_t)(r0 + row);
      if (a_row_index && r0 + row < r_end) ar = (uint32_t)a_row_index[r0 + row];
      if (row < C::BM && r0 + row < r_end) {
        src.a_off[i] = ar * (uint32_t)pitch + 16u * (lane & 3);
        src.as_off[i] = ar * (uint32_t)spitch + 2u * (lane & 3);
      }
    }
    // weight rows: subtile j of this wave covers 32 consecutive rows starting at
    // the wave-uniform row0 (none past the end); lane lr takes row0 + lr and lane
    // half lg holds bytes [32 lg, 32 lg + 32) of each 64-byte stage
#pragma unroll
    for (int j = 0; j < SUB_N; ++j) {
      const int ch = wave * SUB_N + j;
      int row0;
      if (kSilu) {
        const int col0 = nt * (C::BN / 2) + (ch >> 1) * 32;
        row0 = col0 < half_n ? ((ch & 1) ? half_n + col0 : col0) : -1;
      } else {
        const int col0 = nt * C::BN + ch * 32;
        row0 = col0 < N ? col0 : -1;
      }
      // the stage-0 chunk offset is kept, so that a stage's loads need one add
      // and no multiply (which the compiler would branch around in the loop)
      src.b_off[j] = row0 >= 0 ? (uint32_t)(row0 >> 5) * (uint32_t)nstages * kPackChunk : kOutOfRange;
    }
  };
  const uint32_t b_lane = 16u * (uint32_t)lane;
  const uint32_t bs_lane = kPackScaleOff + 4u * (uint32_t)lane;

  // Register rings of P stages for both operands. Global loads complete in
  // issue order, so stage s's activation and weight loads are issued
  // together, P - 1 stages ahead; waiting for one stage never waits for a
  // later stage's loads.
  uint4 ra[P][C::A_PER_T];
  uint32_t rsa[P][C::A_PER_T];
  uint4 rb[P][SUB_N][2];
  uint32_t rsb[P][SUB_N];
  // stages past the end read zeros (out-of-range offsets), so the loop body
  // needs no branches around its loads
  auto store_a = [&](int buf, int slot_) {
    uint8_t* base = lds + buf * (C::BM * kAPitch);
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
      const int task = tid + i * C::THREADS;
      if (task < C::A_TASKS) {
        uint8_t* dst = base + (task >> 2) * kAPitch + (task & 3) * 64;
        const Scales4 sa = scales4(rsa[slot_][i]);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          half8_t v = decode8(pick_u32(ra[slot_][i], q), scale_pair(sa, q >> 1));
          *reinterpret_cast<half8_t*>(dst + 16 * q) = v;
        }
      }
    }
  };
  // Loads of loop stage t into ring slot slot_: stage t of the current item
  // for t < nstages, stage t - S of the next item for t >= S, zeros between
  // (padding stages). The choice is wave-uniform and made with selects.
  // Activations are loaded one stage earlier than weights (their LDS copy is
  // written during the stage before the one that reads it).
  auto load_a = [&](const Src& cur, const Src& nxt, int t, int slot_) {
    const bool in_cur = t < nstages, in_nxt = t >= S;
    const int st = in_cur ? t : t - S;
    const bool in = in_cur || (in_nxt && st < nstages);
    const uint32_t so = in ? (uint32_t)(st * 64) : kOutOfRange, sso = in ? (uint32_t)(st * 8) : kOutOfRange;
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
      ra[slot_][i] = buf_load16(ra_q, in_cur ? cur.a_off[i] : nxt.a_off[i], so);
      rsa[slot_][i] = buf_load2(ra_s, in_cur ? cur.as_off[i] : nxt.as_off[i], sso);
    }
  };
  auto load_b = [&](const Src& cur, const Src& nxt, int t, int slot_) {
    const bool in_cur = t < nstages, in_nxt = t >= S;
    const int st = in_cur ? t : t - S;
    const bool in = in_cur || (in_nxt && st < nstages);
    const __amdgpu_buffer_rsrc_t rbw = in_cur ? cur.rbw : nxt.rbw;
#pragma unroll
    for (int j = 0; j < SUB_N; ++j) {
      // wave-uniform: a scalar offset. A subtile past N has an out-of-range base
      // (>= 2^31), which stays out of range after adding st * kPackChunk (< 2^31).
      const uint32_t base = in_cur ? cur.b_off[j] : nxt.b_off[j];
      const uint32_t chunk = in ? base + (uint32_t)st * kPackChunk : kOutOfRange;
      // decode-height tiles stream every weight byte once (one row tile per
      // expert): non-temporal loads, measured 6-11% faster there; taller tiles
      // re-read an expert's weights for its next row tile and keep them cached
      if (SUB_M == 1) {
        rb[slot_][j][0] = buf_load16_nt(rbw, b_lane, chunk);
        rb[slot_][j][1] = buf_load16_nt(rbw, b_lane + 1024u, chunk);
        rsb[slot_][j] = buf_load4_nt(rbw, bs_lane, chunk);
      } else {
        rb[slot_][j][0] = buf_load16(rbw, b_lane, chunk);
        rb[slot_][j][1] = buf_load16(rbw, b_lane + 1024u, chunk);
        rsb[slot_][j] = buf_load4(rbw, bs_lane, chunk);
      }
    }
  };
  float16_t acc[SUB_M][SUB_N];
  // MFMAs of one stage from ring slot u and LDS buffer buf; meanwhile the
  // activations of the next stage (ring slot su) are decoded into LDS buffer
  // sbuf, one 8-value piece per MFMA step, so that the stage ends with no
  // decode work left before its barrier
  // Prefill-height tiles (64 rows and more) load activations a stage earlier
  // and decode them into LDS during the previous stage's MFMAs; decode-height
  // tiles (32 rows, weight-streaming) keep the decode after the MFMAs, which
  // holds fewer registers (more resident workgroups per CU).
  constexpr bool kEarlyA = C::BM >= 64;
  // BF16 output of prefill-height tiles: two rows per 4-byte store (below)
  constexpr bool kPairStores = C::BM >= 64;
  auto mma_stage = [&](int buf, int u, int sbuf, int su) {
    const uint8_t* abuf = lds + buf * (C::BM * kAPitch) + lr * kAPitch + 128 * lg;
    uint8_t* sdst = lds + sbuf * (C::BM * kAPitch);
    // software pipeline over the 8 MFMA steps of the stage: the operands of
    // step t + 1 are read and decoded while the MFMAs of step t execute
    half8_t av[2][SUB_M], bv[2][SUB_N];
    Scales4 sb[SUB_N], sa[C::A_PER_T];
#pragma unroll
    for (int j = 0; j < SUB_N; ++j) sb[j] = scales4(rsb[u][j]);
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) sa[i] = scales4(rsa[su][i]);
#pragma unroll
    for (int i = 0; i < SUB_M; ++i) av[0][i] = *reinterpret_cast<const half8_t*>(abuf + 32 * i * kAPitch);
#pragma unroll
    for (int j = 0; j < SUB_N; ++j) bv[0][j] = decode8(rb[u][j][0].x, scale_pair(sb[j], 0));
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int cur = t & 1, nxt = cur ^ 1;
      if (t + 1 < 8) {
#pragma unroll
        for (int i = 0; i < SUB_M; ++i)
          av[nxt][i] = *reinterpret_cast<const half8_t*>(abuf + 32 * i * kAPitch + 16 * (t + 1));
#pragma unroll
        for (int j = 0; j < SUB_N; ++j)
          bv[nxt][j] = decode8(pick_u32(rb[u][j][(t + 1) >> 2], (t + 1) & 3), scale_pair(sb[j], (t + 1) >> 1));
      }
      // piece q of staging task i of the next stage's activations (A_PER_T <= 2)
      const int si = (t >> 2) < C::A_PER_T ? (t >> 2) : 0, q = t & 3;
      // threads past the tile's tasks decode the zeros their out-of-range loads
      // returned into a spare 1 KB of LDS: with no branch around the decode,
      // the compiler keeps every activation load where it is issued instead of
      // sinking it next to its only use
      if (kEarlyA && (t >> 2) < C::A_PER_T) {
        const int task = tid + si * C::THREADS;
        uint8_t* dst = task < C::A_TASKS ? sdst + (task >> 2) * kAPitch + (task & 3) * 64 + 16 * q
                                         : lds + C::LDS + 16 * lane;
        *reinterpret_cast<half8_t*>(dst) = decode8(pick_u32(ra[su][si], q), scale_pair(sa[si], q >> 1));
      }
#pragma unroll
      for (int i = 0; i < SUB_M; ++i)
#pragma unroll
        for (int j = 0; j < SUB_N; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[cur][i], bv[cur][j], acc[i][j], 0, 0, 0);
      // issue order: the next step's LDS reads first, then one MFMA followed by
      // a share of the step's VALU work (next step's weight decode, this
      // step's activation piece), repeated; the LDS write last
      constexpr int kValu = 10 * SUB_N + (kEarlyA ? 9 : 0);
      __builtin_amdgcn_sched_group_barrier(0x100, SUB_M, 0);
#pragma unroll
      for (int m = 0; m < SUB_M * SUB_N; ++m) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, (kValu + SUB_M * SUB_N - 1) / (SUB_M * SUB_N), 0);
      }
      if (kEarlyA) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    }
  };

  // Each item runs S stages (K's stage count rounded up to a multiple of P; the
  // extra stages multiply zeros). The loads run ahead across item boundaries
  // (activations P stages, weights P - 1): the last stages of an item load the
  // first stages of the workgroup's next item (load_a/load_b select the source
  // per stage), and the item's last stage decodes the next item's stage 0 into
  // LDS, so the next item starts without waiting for memory. Stage s of an
  // item uses LDS buffer (s + par) & 1, where par flips with every item when S
  // is odd.
  int par = 0;
  Src cur;
  make_src(slot, cur);
  // prologue: activations of stages 0 .. P-1 and weights of stages 0 .. P-2
  // (stage t in ring slot t % P); stage 0's activations decoded into LDS
#pragma unroll
  for (int p = 0; p < P; ++p) {
    if (kEarlyA || p < P - 1) load_a(cur, cur, p, p);
    if (p < P - 1) load_b(cur, cur, p, p);
  }
  store_a(0, 0);
  // NVFP4 output: the threshold table of the fixed global scale of h
  uint8_t* const epi_lds = lds + C::LDS + C::LDS_SPARE;
  uint16_t* h_tile = reinterpret_cast<uint16_t*>(epi_lds);  // [BM][BN/2] BF16 h of one item
  const uint4* h_lut = reinterpret_cast<const uint4*>(epi_lds + C::BM * C::BN);
  if (EPI == kEpiSiluNvfp4) build_threshold_lut(out_gs[0], reinterpret_cast<uint32_t*>(epi_lds + C::BM * C::BN),
                                                tid, C::THREADS);
  __syncthreads();

  for (int item = slot; item < items; item += G) {
    Src nxt;
    make_src(item + G, nxt);
#pragma unroll
    for (int i = 0; i < SUB_M; ++i)
#pragma unroll
      for (int j = 0; j < SUB_N; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    for (int s0 = 0; s0 < S; s0 += P) {
#pragma unroll
      for (int u = 0; u < P; ++u) {
        const int s = s0 + u;
        // early activations: stage s + P into slot u (stage s's were decoded
        // during stage s - 1), weights of stage s + P - 1; then stage s's MFMAs,
        // during which stage s + 1's activations go from slot (u + 1) % P into
        // LDS. Otherwise both P - 1 stages ahead and the decode after the MFMAs.
        if (kEarlyA) {
          load_a(cur, nxt, s + P, u);
          load_b(cur, nxt, s + P - 1, (u + P - 1) % P);
          // the stage's global loads stay ahead of all of its MFMA work, so
          // that their latency runs under the whole stage
          __builtin_amdgcn_sched_barrier(0);
          mma_stage((s + par) & 1, u, (s + 1 + par) & 1, (u + 1) % P);
        } else {
          load_a(cur, nxt, s + P - 1, (u + P - 1) % P);
          load_b(cur, nxt, s + P - 1, (u + P - 1) % P);
          mma_stage((s + par) & 1, u, 0, 0);
          store_a((s + 1 + par) & 1, (u + 1) % P);
        }
        __syncthreads();
      }
    }

    // one global scale per expert, or (gate, up) pairs for an unfolded L1 weight
    int mt, nt;
    tile_of(item, mt, nt);
    const int e = tile_table[1 + 2 * mt];
    const int r0 = tile_table[2 + 2 * mt];
    const int r_end = min(r0 + C::BM, offsets[e + 1]);
    const float alpha = a_gs[0] * b_gs[dual_gs ? 2 * e : e];
    const float alpha_up = dual_gs ? a_gs[0] * b_gs[2 * e + 1] : alpha;
    // epilogue: lane holds column lr and rows 8*(v/4) + 4*lg + (v%4) of each 32x32 tile
    if (EPI == kEpiSiluNvfp4 || !kPairStores) {
      // one value per store (NVFP4 output: into the LDS tile); decode-height
      // tiles keep this form, whose registers fit 4 resident workgroups per CU
#pragma unroll
      for (int i = 0; i < SUB_M; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int row = r0 + i * 32 + 8 * (v >> 2) + 4 * lg + (v & 3);
          if (row >= r_end) continue;
          if (kSilu) {
#pragma unroll
            for (int j = 0; j < SUB_N; j += 2) {
              const int ch = wave * SUB_N + j;  // even chunk: gate, next chunk: up
              const int lc = (ch >> 1) * 32 + lr, col = nt * (C::BN / 2) + lc;
              if (col >= n_out) continue;
              const uint32_t h = silu_mul_bf16(acc[i][j][v], acc[i][j + 1][v], alpha, alpha_up);
              if (EPI == kEpiSiluNvfp4) {
                h_tile[(row - r0) * (C::BN / 2) + lc] = (uint16_t)h;
              } else {
                d[(size_t)row * n_out + col] = (uint16_t)h;
                amax_local = fmaxf(amax_local, fabsf(bf16_to_f32(h)));
              }
            }
          } else {
#pragma unroll
            for (int j = 0; j < SUB_N; ++j) {
              const int col = nt * C::BN + (wave * SUB_N + j) * 32 + lr;
              if (col >= n_out) continue;
              d[(size_t)row * n_out + col] = (uint16_t)f32_to_bf16(acc[i][j][v] * alpha);
            }
          }
        }
      }
    } else {
      // BF16 output, two rows at a time: rows (v, v + 1) of a lane's column
      // become one BF16 pair, swapped with lane lr ^ 1 so that an even lane
      // holds row v, columns (lr, lr + 1) and an odd lane row v + 1, columns
      // (lr - 1, lr): one 4-byte store each. The store resource starts at
      // the row tile's first row and ends at the group's last row, so rows
      // past the group's end are dropped by the range check.
      const int odd = lr & 1;
      const uint32_t pair_sel = odd ? 0x03020706u : 0x05040100u;
      const uint32_t row_bytes = (uint32_t)n_out * 2u;
      const __amdgpu_buffer_rsrc_t rd =
          make_rsrc(d + (size_t)r0 * n_out, (uint32_t)(r_end - r0) * row_bytes);
#pragma unroll
      for (int j = 0; j < SUB_N; j += (kSilu ? 2 : 1)) {
        const int ch = wave * SUB_N + j;  // with SiLU: even chunk gate, next chunk up
        const int col0 = kSilu ? nt * (C::BN / 2) + (ch >> 1) * 32 : nt * C::BN + ch * 32;
        if (col0 >= n_out) continue;  // the whole 32-column subtile is past N
        const uint32_t lane_off = ((uint32_t)(4 * lg + odd) * (uint32_t)n_out + (uint32_t)(col0 + (lr & ~1))) * 2u;
#pragma unroll
        for (int i = 0; i < SUB_M; ++i) {
#pragma unroll
          for (int v = 0; v < 16; v += 2) {
            uint32_t p;
            if (kSilu) {
              const uint32_t ha = silu_mul_bf16(acc[i][j][v], acc[i][j + 1][v], alpha, alpha_up);
              const uint32_t hb = silu_mul_bf16(acc[i][j][v + 1], acc[i][j + 1][v + 1], alpha, alpha_up);
              // rows past the group hold zeros (their activations read as zero)
              amax_local = fmaxf(amax_local, fmaxf(fabsf(bf16_to_f32(ha)), fabsf(bf16_to_f32(hb))));
              p = ha | (hb << 16);
            } else {
              p = f32x2_to_bf16x2(acc[i][j][v] * alpha, acc[i][j][v + 1] * alpha);
            }
            const uint32_t q = (uint32_t)__builtin_amdgcn_mov_dpp((int)p, 0xB1, 0xF, 0xF, false);  // lane lr ^ 1
            const uint32_t row = (uint32_t)(i * 32 + 8 * (v >> 2) + (v & 3));
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_amdgcn_perm(q, p, pair_sel), rd, (int)lane_off,
                                                  (int)(row * row_bytes), 0);
          }
        }
      }
    }
    if (EPI == kEpiSiluNvfp4) {
      // h of the item is in LDS: each thread quantizes whole 16-column blocks
      // (exact roundings, the quantizer's own code) and writes them as NVFP4
      __syncthreads();
      const QuantScale qs_o = quant_scale(out_gs[0]);
      uint8_t* d_q = reinterpret_cast<uint8_t*>(d);
      for (int blk = tid; blk < C::BM * (C::BN / 32); blk += C::THREADS) {
        const int lrow = blk / (C::BN / 32), lb = blk % (C::BN / 32);
        const int row = r0 + lrow, col0 = nt * (C::BN / 2) + 16 * lb;
        if (row >= r_end || col0 >= n_out) continue;
        const uint4* src = reinterpret_cast<const uint4*>(h_tile + lrow * (C::BN / 2) + 16 * lb);
        const uint4 v0 = src[0], v1 = src[1];
        const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        uint2 packed;
        const uint32_t code = quantize_block16(w, qs_o, h_lut, &packed);
        *reinterpret_cast<uint2*>(d_q + (size_t)row * (n_out / 2) + col0 / 2) = packed;
        d_sf[(size_t)row * (n_out / 16) + col0 / 16] = (uint8_t)code;
      }
    }
    cur = nxt;
    par = (par + S) & 1;
  }
  if (EPI == NVFP4_EPI_SILU_MUL) {
    const float m = wave_max(amax_local);
    if (lane == 0 && m > 0.0f) atomicMax(reinterpret_cast<unsigned int*>(amax_out), __float_as_uint(m));
  }
}

template <int SUB_M, int SUB_N, int WAVES, int P, int EPI>
static int launch_cfg(const uint8_t* a_q, const uint8_t* a_sf, const int32_t* a_row_index, const float* a_gs,
                      const uint8_t* b_packed, const float* b_gs, const int32_t* offsets,
                      const int32_t* tile_table, int32_t num_local, int32_t rows_cap, int32_t N, int32_t K,
                      void* d, float* amax_out, hipStream_t stream, int dual_gs = 0, int col_fastest = 0,
                      uint8_t* d_sf = nullptr, const float* out_gs = nullptr) {
  using C = GemmCfg<SUB_M, SUB_N, WAVES, P>;
  static_assert(EPI == NVFP4_EPI_BF16 || SUB_N % 2 == 0, "gate/up pairs live in one wave");
  const int n_out = EPI != NVFP4_EPI_BF16 ? N / 2 : N;
  const int bn_out = EPI != NVFP4_EPI_BF16 ? C::BN / 2 : C::BN;
  // NVFP4 output adds the BF16 h tile of one item and the threshold table
  constexpr int lds_bytes = C::LDS + C::LDS_SPARE + (EPI == kEpiSiluNvfp4 ? C::BM * C::BN + kLutBytes : 0);
  const int n_ntiles = (n_out + bn_out - 1) / bn_out;
  const int max_tiles = rows_cap / C::BM + num_local;
  const int64_t max_items = (int64_t)max_tiles * n_ntiles;
  auto kern = grouped_gemm_kernel<SUB_M, SUB_N, WAVES, P, EPI>;
  // resident workgroups on the device: CU count x workgroups per CU (host
  // queries, once per device and configuration)
  static std::atomic<int> resident_wgs[kMaxDevices];
  const int dev = nvfp4_current_device();
  if (dev < 0) return NVFP4_ERR_HIP;
  int resident = resident_wgs[dev].load(std::memory_order_relaxed);
  if (resident == 0) {
    int n_cu = 0;
    if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu < 1)
      return NVFP4_ERR_HIP;
    if (lds_bytes > 64 * 1024 &&
        hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                            lds_bytes) != hipSuccess)
      return NVFP4_ERR_HIP;
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void*>(kern), C::THREADS,
                                                     lds_bytes) != hipSuccess || nb < 1)
      nb = 1;
    resident = n_cu * nb;
    resident_wgs[dev].store(resident, std::memory_order_relaxed);
  }
  int64_t grid = resident;
  if (grid > max_items) grid = max_items;
  if (grid >= kXcds) grid -= grid % kXcds;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::THREADS), lds_bytes, stream, a_q, a_sf, a_row_index, a_gs,
                     b_packed, b_gs, offsets, tile_table, max_tiles, N, K, n_out, n_ntiles, col_fastest, dual_gs,
                     reinterpret_cast<uint16_t*>(d), amax_out, d_sf, out_gs);
  NVFP4_CHECK_LAUNCH();
  return NVFP4_OK;
}

}  // namespace nvfp4

using namespace nvfp4;

// Row-tile heights with a kernel configuration (measured on MI355X over
// decode- and prefill-shaped problems):
//   32  decode-shaped batches: 4 waves, each 32 x 64, 3 stages in flight
//   64  8 waves, each 64 x 64, 4 stages in flight
//   96  prefill-shaped: 8 waves, each 96 x 64, 2 stages in flight (a third
//       less weight decode per MFMA than 64 rows; with experts of ~170 or
//       ~256 rows it pads no more than 64-row tiles do)
//   128 large groups: 4 waves, each 128 x 64, 3 stages in flight
int nvfp4_launch_grouped_gemm(const uint8_t* a_q, const uint8_t* a_sf, const int32_t* a_row_index,
                              const float* a_gs, const uint8_t* b_packed, const float* b_gs,
                              const int32_t* offsets, const int32_t* tile_table, int32_t num_local,
                              int32_t rows_cap, int32_t N, int32_t K, int32_t tile_m, int32_t epilogue, void* d,
                              float* amax_out, hipStream_t stream) {
#define NVFP4_GEMM_ARGS a_q, a_sf, a_row_index, a_gs, b_packed, b_gs, offsets, tile_table, num_local, rows_cap, \
                        N, K, d, amax_out, stream, epilogue == NVFP4_EPI_SILU_MUL_DUAL ? 1 : 0
#define NVFP4_GEMM_CFG(SM, SN, W, PF)                                                          \
  return epilogue != NVFP4_EPI_BF16 ? launch_cfg<SM, SN, W, PF, NVFP4_EPI_SILU_MUL>(NVFP4_GEMM_ARGS) \
                                    : launch_cfg<SM, SN, W, PF, NVFP4_EPI_BF16>(NVFP4_GEMM_ARGS)
  switch (tile_m) {
    case 32: NVFP4_GEMM_CFG(1, 2, 4, 3);
    case 64: NVFP4_GEMM_CFG(2, 2, 8, 4);
    case 96: NVFP4_GEMM_CFG(3, 2, 8, 2);
    case 128: NVFP4_GEMM_CFG(4, 2, 4, 3);
    default: return NVFP4_ERR_SHAPE;
  }
#undef NVFP4_GEMM_CFG
#undef NVFP4_GEMM_ARGS
}

// The L1 GEMM whose SiLU*up epilogue writes h as NVFP4 with the fixed global
// scale out_gs[0] (d_q [rows_cap, N/4], d_sf [rows_cap, N/32]); same tile
// configurations as nvfp4_launch_grouped_gemm.
int nvfp4_launch_grouped_gemm_nvfp4(const uint8_t* a_q, const uint8_t* a_sf, const int32_t* a_row_index,
                                    const float* a_gs, const uint8_t* b_packed, const float* b_gs, int32_t dual_gs,
                                    const int32_t* offsets, const int32_t* tile_table, int32_t num_local,
                                    int32_t rows_cap, int32_t N, int32_t K, int32_t tile_m, const float* out_gs,
                                    uint8_t* d_q, uint8_t* d_sf, hipStream_t stream) {
#define NVFP4_GEMM_CFG(SM, SN, W, PF)                                                                             \
  return launch_cfg<SM, SN, W, PF, kEpiSiluNvfp4>(a_q, a_sf, a_row_index, a_gs, b_packed, b_gs, offsets,        \
                                                 tile_table, num_local, rows_cap, N, K, d_q, nullptr, stream,  \
                                                 dual_gs, 0, d_sf, out_gs)
  switch (tile_m) {
    case 32: NVFP4_GEMM_CFG(1, 2, 4, 3);
    case 64: NVFP4_GEMM_CFG(2, 2, 8, 4);
    case 96: NVFP4_GEMM_CFG(3, 2, 8, 2);
    case 128: NVFP4_GEMM_CFG(4, 2, 4, 3);
    default: return NVFP4_ERR_SHAPE;
  }
#undef NVFP4_GEMM_CFG
}

extern "C" int nvfp4_grouped_gemm_silu_nvfp4(const uint8_t* a_q, const uint8_t* a_sf, const int32_t* a_row_index,
                                             const float* a_gs, const uint8_t* b_packed, const float* b_gs,
                                             int32_t dual_gs, const int32_t* offsets, const int32_t* tile_table,
                                             int32_t num_local, int32_t rows_cap, int32_t N, int32_t K,
                                             int32_t tile_m, const float* out_gs, uint8_t* d_q, uint8_t* d_sf,
                                             void* stream) {
  if (dual_gs != 0 && dual_gs != 1) return NVFP4_ERR_ARG;
  if (num_local < 1 || rows_cap < 0 || N <= 0 || K <= 0 || K % kBK != 0 || N % 128 != 0) return NVFP4_ERR_SHAPE;
  if (tile_m != 32 && tile_m != 64 && tile_m != 96 && tile_m != 128) return NVFP4_ERR_SHAPE;
  if (!a_q || !a_sf || !a_gs || !b_packed || !b_gs || !offsets || !tile_table || !out_gs || !d_q || !d_sf)
    return NVFP4_ERR_NULL;
  if (!nvfp4_aligned16(a_q) || !nvfp4_aligned16(a_sf) || !nvfp4_aligned16(b_packed) || !nvfp4_aligned16(d_q))
    return NVFP4_ERR_ALIGN;
  if ((int64_t)rows_cap * (K / 2) >= (1ll << 31) || (int64_t)N * K / 32 * 18 >= (1ll << 31)) return NVFP4_ERR_SHAPE;
  if (rows_cap == 0) return NVFP4_OK;
  return nvfp4_launch_grouped_gemm_nvfp4(a_q, a_sf, a_row_index, a_gs, b_packed, b_gs, dual_gs, offsets, tile_table,
                                         num_local, rows_cap, N, K, tile_m, out_gs, d_q, d_sf, (hipStream_t)stream);
}

extern "C" int nvfp4_grouped_gemm(const uint8_t* a_q, const uint8_t* a_sf, const int32_t* a_row_index,
                                  const float* a_gs, const uint8_t* b_packed, const float* b_gs,
                                  const int32_t* offsets, const int32_t* tile_table, int32_t num_local,
                                  int32_t rows_cap, int32_t N, int32_t K, int32_t tile_m, int32_t epilogue, void* d,
                                  float* amax_out, void* stream) {
  if (epilogue != NVFP4_EPI_BF16 && epilogue != NVFP4_EPI_SILU_MUL && epilogue != NVFP4_EPI_SILU_MUL_DUAL)
    return NVFP4_ERR_ARG;
  const bool silu = epilogue != NVFP4_EPI_BF16;
  if (num_local < 1 || rows_cap < 0 || N <= 0 || K <= 0 || K % kBK != 0 || N % 64 != 0) return NVFP4_ERR_SHAPE;
  if (silu && N % 128 != 0) return NVFP4_ERR_SHAPE;
  if (tile_m != 32 && tile_m != 64 && tile_m != 96 && tile_m != 128) return NVFP4_ERR_SHAPE;
  if (!a_q || !a_sf || !a_gs || !b_packed || !b_gs || !offsets || !tile_table || !d) return NVFP4_ERR_NULL;
  if (silu && !amax_out) return NVFP4_ERR_NULL;
  if (!nvfp4_aligned16(a_q) || !nvfp4_aligned16(a_sf) || !nvfp4_aligned16(b_packed) || !nvfp4_aligned16(d))
    return NVFP4_ERR_ALIGN;
  // buffer offsets are 32-bit: activation row offsets, one expert's packed weights and one row tile of the
  // output (at most 128 rows) stay below 2^31
  if ((int64_t)rows_cap * (K / 2) >= (1ll << 31) || (int64_t)N * K / 32 * 18 >= (1ll << 31)) return NVFP4_ERR_SHAPE;
  if ((int64_t)N * 2 * 128 >= (1ll << 31)) return NVFP4_ERR_SHAPE;
  if (rows_cap == 0) return NVFP4_OK;
  return nvfp4_launch_grouped_gemm(a_q, a_sf, a_row_index, a_gs, b_packed, b_gs, offsets, tile_table, num_local,
                                   rows_cap, N, K, tile_m, epilogue, d, amax_out, (hipStream_t)stream);
}

// ------------------------------------------------------------ weight packing

// One thread per (matrix, subtile, stage, lane): moves the lane's 32 FP4 bytes
// and 4 scale bytes from the row-major tensors into the packed chunk.
__global__ __launch_bounds__(256) void pack_kernel(const uint8_t* __restrict__ q, const uint8_t* __restrict__ sf,
                                                   int64_t total, int N, int K, uint8_t* __restrict__ out) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int nst = K / kBK, nsub = N / 32;
  const int l = (int)(idx & 63);
  int64_t rest = idx >> 6;
  const int c = (int)(rest % nst);
  rest /= nst;
  const int sub = (int)(rest % nsub);
  const int64_t b = rest / nsub;
  const int64_t row = b * N + sub * 32 + (l & 31);
  const int g = l >> 5;
  const uint4* src = reinterpret_cast<const uint4*>(q + row * (K / 2) + 64 * c + 32 * g);
  const uint32_t s = *reinterpret_cast<const uint32_t*>(sf + row * (K / 16) + 8 * c + 4 * g);
  uint8_t* dst = out + ((b * nsub + sub) * nst + c) * kPackChunk;
  *reinterpret_cast<uint4*>(dst + 16 * l) = src[0];
  *reinterpret_cast<uint4*>(dst + 1024 + 16 * l) = src[1];
  *reinterpret_cast<uint32_t*>(dst + kPackScaleOff + 4 * l) = s;
}

extern "C" int64_t nvfp4_packed_bytes(int64_t B, int64_t N, int64_t K) {
  if (B < 0 || N <= 0 || K <= 0 || N % 32 != 0 || K % kBK != 0) return -1;
  return B * N * K / 32 * 18;
}

extern "C" int nvfp4_pack_weights(const uint8_t* q, const uint8_t* sf, int64_t B, int64_t N, int64_t K,
                                  uint8_t* packed, void* stream) {
  if (B < 0 || N <= 0 || K <= 0 || N % 32 != 0 || K % kBK != 0 || N >= (1ll << 30) || K >= (1ll << 30))
    return NVFP4_ERR_SHAPE;
  if (!q || !sf || !packed) return NVFP4_ERR_NULL;
  if (!nvfp4_aligned16(q) || !nvfp4_aligned16(sf) || !nvfp4_aligned16(packed)) return NVFP4_ERR_ALIGN;
  const int64_t total = B * (N / 32) * (K / kBK) * 64;
  if (total == 0) return NVFP4_OK;
  const int64_t blocks = (total + 255) / 256;
  if (blocks >= (1ll << 31)) return NVFP4_ERR_SHAPE;
  hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, q, sf, total, (int)N,
                     (int)K, packed);
  NVFP4_CHECK_LAUNCH();
  return NVFP4_OK;
}
