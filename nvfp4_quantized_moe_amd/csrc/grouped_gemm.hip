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
// takes a contiguous run of items, which share the row tile's activations.
// Each item streams K in stages of 128: FP4 bytes and scale bytes of the row
// and column tiles go global -> registers -> LDS (double buffered, next stage
// loaded while the current one is multiplied); every wave decodes its own
// fragments from LDS. Within a 128-wide stage, lane half g of a wave takes
// the contiguous K range [64g, 64g + 64) across the 8 MFMA steps; A and B use
// the same assignment, so each MFMA step still sums matching K indices.
#include "common.h"
#include "internal.h"

namespace nvfp4 {

constexpr int kBK = 128;           // K elements per stage
constexpr int kRowBytes = kBK / 2; // 64 FP4 bytes per row per stage
constexpr int kRowPitch = 80;      // LDS pitch of a row (16 bytes padding)
constexpr int kSfBytes = kBK / 16; // 8 scale bytes per row per stage

template <int SUB_M, int SUB_N, int WAVES_M, int WAVES_N>
struct GemmCfg {
  static constexpr int BM = 32 * SUB_M * WAVES_M;
  static constexpr int BN = 32 * SUB_N * WAVES_N;
  static constexpr int THREADS = 64 * WAVES_M * WAVES_N;
  static constexpr int A_BYTES = BM * kRowPitch;
  static constexpr int B_BYTES = BN * kRowPitch;
  static constexpr int STAGE = A_BYTES + B_BYTES + (BM + BN) * kSfBytes;
  static constexpr int LDS = 2 * STAGE;
  // 16-byte data chunks and 8-byte scale chunks per stage
  static constexpr int A_CHUNKS = BM * (kRowBytes / 16);
  static constexpr int B_CHUNKS = BN * (kRowBytes / 16);
  static constexpr int A_PER_T = (A_CHUNKS + THREADS - 1) / THREADS;
  static constexpr int B_PER_T = (B_CHUNKS + THREADS - 1) / THREADS;
  static constexpr int SA_PER_T = (BM + THREADS - 1) / THREADS;
  static constexpr int SB_PER_T = (BN + THREADS - 1) / THREADS;
};

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

__device__ __forceinline__ uint32_t pick_u32(const uint4& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

template <int SEL>
__device__ __forceinline__ half2_t scale_pair(uint32_t sw) {
  _Float16 s = (_Float16)__builtin_amdgcn_cvt_f32_fp8(sw, SEL);  // E4M3 -> f32 -> f16, both exact
  half2_t r;
  r[0] = s;
  r[1] = s;
  return r;
}

__device__ __forceinline__ float silu_f32(float g) { return g / (1.0f + __expf(-g)); }

template <int SUB_M, int SUB_N, int WAVES_M, int WAVES_N, int EPI>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N) void grouped_gemm_kernel(
    const uint8_t* __restrict__ a_q, const uint8_t* __restrict__ a_sf, const int32_t* __restrict__ a_row_index,
    const float* __restrict__ a_gs, const uint8_t* __restrict__ b_q, const uint8_t* __restrict__ b_sf,
    const float* __restrict__ b_gs, const int32_t* __restrict__ offsets, const int32_t* __restrict__ tile_table,
    int max_tiles, int N, int K, int n_out, int n_ntiles, uint16_t* __restrict__ d, float* __restrict__ amax_out) {
  using C = GemmCfg<SUB_M, SUB_N, WAVES_M, WAVES_N>;
  extern __shared__ __align__(16) uint8_t lds[];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int lr = lane & 31, lg = lane >> 5;

  int ntiles = tile_table[0];
  ntiles = ntiles < max_tiles ? ntiles : max_tiles;
  const int items = ntiles * n_ntiles;
  const int G = gridDim.x;
  const int slot = (G % kXcds == 0) ? (blockIdx.x % kXcds) * (G / kXcds) + blockIdx.x / kXcds : blockIdx.x;
  const int64_t a_pitch = K / 2, a_spitch = K / 16;
  const int nstages = K / kBK;
  float amax_local = 0.0f;

  for (int item = slot; item < items; item += G) {
    const int mt = item / n_ntiles, nt = item % n_ntiles;
    const int e = tile_table[1 + 2 * mt];
    const int r0 = tile_table[2 + 2 * mt];
    const int r_end = min(r0 + C::BM, offsets[e + 1]);
    const float alpha = a_gs[0] * b_gs[e];
    const uint8_t* bq = b_q + (size_t)e * N * a_pitch;
    const uint8_t* bs = b_sf + (size_t)e * N * a_spitch;

    // per-thread source rows for this item (fixed across stages)
    const uint8_t* a_src[C::A_PER_T];
    const uint8_t* b_src[C::B_PER_T];
    const uint8_t* sa_src[C::SA_PER_T];
    const uint8_t* sb_src[C::SB_PER_T];
#pragma unroll
    for (int i = 0; i < C::A_PER_T; ++i) {
      int c = tid + i * C::THREADS, row = c >> 2;
      const uint8_t* p = nullptr;
      if (c < C::A_CHUNKS && r0 + row < r_end) {
        int ar = a_row_index ? a_row_index[r0 + row] : r0 + row;
        p = a_q + (size_t)ar * a_pitch + (c & 3) * 16;
      }
      a_src[i] = p;
    }
#pragma unroll
    for (int i = 0; i < C::SA_PER_T; ++i) {
      int row = tid + i * C::THREADS;
      const uint8_t* p = nullptr;
      if (row < C::BM && r0 + row < r_end) {
        int ar = a_row_index ? a_row_index[r0 + row] : r0 + row;
        p = a_sf + (size_t)ar * a_spitch;
      }
      sa_src[i] = p;
    }
    auto brow = [&](int r) -> int {  // LDS row of the column tile -> weight row (or -1)
      if (EPI == NVFP4_EPI_SILU_MUL) {
        int c = r >> 5, half_n = N / 2;
        int col = nt * (C::BN / 2) + (c >> 1) * 32 + (r & 31);
        if (col >= half_n) return -1;
        return (c & 1) ? half_n + col : col;
      } else {
        int col = nt * C::BN + r;
        return col < N ? col : -1;
      }
    };
#pragma unroll
    for (int i = 0; i < C::B_PER_T; ++i) {
      int c = tid + i * C::THREADS, row = c >> 2;
      const uint8_t* p = nullptr;
      if (c < C::B_CHUNKS) {
        int wr = brow(row);
        if (wr >= 0) p = bq + (size_t)wr * a_pitch + (c & 3) * 16;
      }
      b_src[i] = p;
    }
#pragma unroll
    for (int i = 0; i < C::SB_PER_T; ++i) {
      int row = tid + i * C::THREADS;
      const uint8_t* p = nullptr;
      if (row < C::BN) {
        int wr = brow(row);
        if (wr >= 0) p = bs + (size_t)wr * a_spitch;
      }
      sb_src[i] = p;
    }

    uint4 ra[C::A_PER_T], rb[C::B_PER_T];
    uint2 rsa[C::SA_PER_T], rsb[C::SB_PER_T];
    auto gload = [&](int s) {
      const int kb = s * kRowBytes, ks = s * kSfBytes;
#pragma unroll
      for (int i = 0; i < C::A_PER_T; ++i)
        ra[i] = a_src[i] ? *reinterpret_cast<const uint4*>(a_src[i] + kb) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < C::B_PER_T; ++i)
        rb[i] = b_src[i] ? *reinterpret_cast<const uint4*>(b_src[i] + kb) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < C::SA_PER_T; ++i)
        rsa[i] = sa_src[i] ? *reinterpret_cast<const uint2*>(sa_src[i] + ks) : make_uint2(0, 0);
#pragma unroll
      for (int i = 0; i < C::SB_PER_T; ++i)
        rsb[i] = sb_src[i] ? *reinterpret_cast<const uint2*>(sb_src[i] + ks) : make_uint2(0, 0);
    };
    auto lstore = [&](int buf) {
      uint8_t* st = lds + buf * C::STAGE;
      uint8_t* sA = st;
      uint8_t* sB = st + C::A_BYTES;
      uint8_t* sSA = st + C::A_BYTES + C::B_BYTES;
      uint8_t* sSB = sSA + C::BM * kSfBytes;
#pragma unroll
      for (int i = 0; i < C::A_PER_T; ++i) {
        int c = tid + i * C::THREADS;
        if (c < C::A_CHUNKS) *reinterpret_cast<uint4*>(sA + (c >> 2) * kRowPitch + (c & 3) * 16) = ra[i];
      }
#pragma unroll
      for (int i = 0; i < C::B_PER_T; ++i) {
        int c = tid + i * C::THREADS;
        if (c < C::B_CHUNKS) *reinterpret_cast<uint4*>(sB + (c >> 2) * kRowPitch + (c & 3) * 16) = rb[i];
      }
#pragma unroll
      for (int i = 0; i < C::SA_PER_T; ++i) {
        int row = tid + i * C::THREADS;
        if (row < C::BM) *reinterpret_cast<uint2*>(sSA + row * kSfBytes) = rsa[i];
      }
#pragma unroll
      for (int i = 0; i < C::SB_PER_T; ++i) {
        int row = tid + i * C::THREADS;
        if (row < C::BN) *reinterpret_cast<uint2*>(sSB + row * kSfBytes) = rsb[i];
      }
    };

    float16_t acc[SUB_M][SUB_N];
#pragma unroll
    for (int i = 0; i < SUB_M; ++i)
#pragma unroll
      for (int j = 0; j < SUB_N; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    __syncthreads();  // previous item's readers are done with both buffers
    gload(0);
    lstore(0);
    __syncthreads();
    for (int s = 0; s < nstages; ++s) {
      const int buf = s & 1;
      if (s + 1 < nstages) gload(s + 1);
      const uint8_t* st = lds + buf * C::STAGE;
      const uint8_t* sA = st;
      const uint8_t* sB = st + C::A_BYTES;
      const uint8_t* sSA = st + C::A_BYTES + C::B_BYTES;
      const uint8_t* sSB = sSA + C::BM * kSfBytes;
      // raw FP4 of this lane: 32 bytes (64 K values) per subtile, and 4 scale bytes
      uint4 fa[SUB_M][2], fb[SUB_N][2];
      uint32_t sa[SUB_M], sb[SUB_N];
#pragma unroll
      for (int i = 0; i < SUB_M; ++i) {
        int row = wm * 32 * SUB_M + i * 32 + lr;
        const uint8_t* p = sA + row * kRowPitch + lg * 32;
        fa[i][0] = *reinterpret_cast<const uint4*>(p);
        fa[i][1] = *reinterpret_cast<const uint4*>(p + 16);
        sa[i] = *reinterpret_cast<const uint32_t*>(sSA + row * kSfBytes + lg * 4);
      }
#pragma unroll
      for (int j = 0; j < SUB_N; ++j) {
        int row = wn * 32 * SUB_N + j * 32 + lr;
        const uint8_t* p = sB + row * kRowPitch + lg * 32;
        fb[j][0] = *reinterpret_cast<const uint4*>(p);
        fb[j][1] = *reinterpret_cast<const uint4*>(p + 16);
        sb[j] = *reinterpret_cast<const uint32_t*>(sSB + row * kSfBytes + lg * 4);
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        half8_t av[SUB_M], bv[SUB_N];
#pragma unroll
        for (int i = 0; i < SUB_M; ++i) {
          uint32_t w = pick_u32(fa[i][t >> 2], t & 3);
          half2_t s2 = (t >> 1) == 0 ? scale_pair<0>(sa[i])
                     : (t >> 1) == 1 ? scale_pair<1>(sa[i])
                     : (t >> 1) == 2 ? scale_pair<2>(sa[i]) : scale_pair<3>(sa[i]);
          av[i] = decode8(w, s2);
        }
#pragma unroll
        for (int j = 0; j < SUB_N; ++j) {
          uint32_t w = pick_u32(fb[j][t >> 2], t & 3);
          half2_t s2 = (t >> 1) == 0 ? scale_pair<0>(sb[j])
                     : (t >> 1) == 1 ? scale_pair<1>(sb[j])
                     : (t >> 1) == 2 ? scale_pair<2>(sb[j]) : scale_pair<3>(sb[j]);
          bv[j] = decode8(w, s2);
        }
#pragma unroll
        for (int i = 0; i < SUB_M; ++i)
#pragma unroll
          for (int j = 0; j < SUB_N; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
      }
      if (s + 1 < nstages) {
        lstore(buf ^ 1);
        __syncthreads();
      }
    }

    // epilogue: lane holds column (lane & 31) and rows 8*(v/4) + 4*lg + (v%4) of each 32x32 tile
#pragma unroll
    for (int i = 0; i < SUB_M; ++i) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = r0 + wm * 32 * SUB_M + i * 32 + 8 * (v >> 2) + 4 * lg + (v & 3);
        if (row >= r_end) continue;
        if (EPI == NVFP4_EPI_SILU_MUL) {
#pragma unroll
          for (int j = 0; j < SUB_N; j += 2) {
            const int c = wn * SUB_N + j;  // 32-row chunk of the column tile (even: gate)
            const int col = nt * (C::BN / 2) + (c >> 1) * 32 + lr;
            if (col >= n_out) continue;
            float g = bf16_to_f32(f32_to_bf16(acc[i][j][v] * alpha));
            float u = bf16_to_f32(f32_to_bf16(acc[i][j + 1][v] * alpha));
            uint32_t h = f32_to_bf16(silu_f32(g) * u);
            d[(size_t)row * n_out + col] = (uint16_t)h;
            amax_local = fmaxf(amax_local, fabsf(bf16_to_f32(h)));
          }
        } else {
#pragma unroll
          for (int j = 0; j < SUB_N; ++j) {
            const int col = nt * C::BN + wn * 32 * SUB_N + j * 32 + lr;
            if (col >= n_out) continue;
            d[(size_t)row * n_out + col] = (uint16_t)f32_to_bf16(acc[i][j][v] * alpha);
          }
        }
      }
    }
  }
  if (EPI == NVFP4_EPI_SILU_MUL) {
    float m = wave_max(amax_local);
    if (lane == 0 && m > 0.0f) atomicMax(reinterpret_cast<unsigned int*>(amax_out), __float_as_uint(m));
  }
}

template <int SUB_M, int SUB_N, int WAVES_M, int WAVES_N, int EPI>
static int launch_cfg(const uint8_t* a_q, const uint8_t* a_sf, const int32_t* a_row_index, const float* a_gs,
                      const uint8_t* b_q, const uint8_t* b_sf, const float* b_gs, const int32_t* offsets,
                      const int32_t* tile_table, int32_t num_local, int32_t rows_cap, int32_t N, int32_t K,
                      void* d, float* amax_out, hipStream_t stream) {
  using C = GemmCfg<SUB_M, SUB_N, WAVES_M, WAVES_N>;
  const int n_out = EPI == NVFP4_EPI_SILU_MUL ? N / 2 : N;
  const int bn_out = EPI == NVFP4_EPI_SILU_MUL ? C::BN / 2 : C::BN;
  const int n_ntiles = (n_out + bn_out - 1) / bn_out;
  const int max_tiles = rows_cap / C::BM + num_local;
  int64_t max_items = (int64_t)max_tiles * n_ntiles;
  int occupancy = (160 * 1024) / C::LDS;
  if (occupancy > 4) occupancy = 4;
  if (occupancy < 1) occupancy = 1;
  int64_t grid = 256 * occupancy;
  if (grid > max_items) grid = max_items;
  if (grid >= kXcds) grid -= grid % kXcds;
  if (grid < 1) grid = 1;
  auto kern = grouped_gemm_kernel<SUB_M, SUB_N, WAVES_M, WAVES_N, EPI>;
  static bool attr_set = false;  // raising the dynamic LDS limit is idempotent
  if (!attr_set) {
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, C::LDS);
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(C::THREADS), C::LDS, stream, a_q, a_sf, a_row_index, a_gs,
                     b_q, b_sf, b_gs, offsets, tile_table, max_tiles, N, K, n_out, n_ntiles,
                     reinterpret_cast<uint16_t*>(d), amax_out);
  NVFP4_CHECK_LAUNCH();
  return NVFP4_OK;
}

}  // namespace nvfp4

using namespace nvfp4;

// Tile heights with a kernel configuration: 32 (decode-shaped batches: one
// MFMA row tile, four waves across N) and 128 (prefill-shaped: 2 x 2 waves of
// 64 x 64).
int nvfp4_launch_grouped_gemm(const uint8_t* a_q, const uint8_t* a_sf, const int32_t* a_row_index,
                              const float* a_gs, const uint8_t* b_q, const uint8_t* b_sf, const float* b_gs,
                              const int32_t* offsets, const int32_t* tile_table, int32_t num_local,
                              int32_t rows_cap, int32_t N, int32_t K, int32_t tile_m, int32_t epilogue, void* d,
                              float* amax_out, hipStream_t stream) {
#define NVFP4_GEMM_ARGS a_q, a_sf, a_row_index, a_gs, b_q, b_sf, b_gs, offsets, tile_table, num_local, rows_cap, \
                        N, K, d, amax_out, stream
  if (tile_m == 32) {
    if (epilogue == NVFP4_EPI_SILU_MUL) return launch_cfg<1, 2, 1, 4, NVFP4_EPI_SILU_MUL>(NVFP4_GEMM_ARGS);
    return launch_cfg<1, 2, 1, 4, NVFP4_EPI_BF16>(NVFP4_GEMM_ARGS);
  }
  if (tile_m == 128) {
    if (epilogue == NVFP4_EPI_SILU_MUL) return launch_cfg<2, 2, 2, 2, NVFP4_EPI_SILU_MUL>(NVFP4_GEMM_ARGS);
    return launch_cfg<2, 2, 2, 2, NVFP4_EPI_BF16>(NVFP4_GEMM_ARGS);
  }
#undef NVFP4_GEMM_ARGS
  return NVFP4_ERR_SHAPE;
}

extern "C" int nvfp4_grouped_gemm(const uint8_t* a_q, const uint8_t* a_sf, const int32_t* a_row_index,
                                  const float* a_gs, const uint8_t* b_q, const uint8_t* b_sf, const float* b_gs,
                                  const int32_t* offsets, const int32_t* tile_table, int32_t num_local,
                                  int32_t rows_cap, int32_t N, int32_t K, int32_t tile_m, int32_t epilogue, void* d,
                                  float* amax_out, void* stream) {
  if (epilogue != NVFP4_EPI_BF16 && epilogue != NVFP4_EPI_SILU_MUL) return NVFP4_ERR_ARG;
  if (num_local < 1 || rows_cap < 0 || N <= 0 || K <= 0 || K % kBK != 0 || N % 64 != 0) return NVFP4_ERR_SHAPE;
  if (epilogue == NVFP4_EPI_SILU_MUL && N % 128 != 0) return NVFP4_ERR_SHAPE;
  if (tile_m != 32 && tile_m != 128) return NVFP4_ERR_SHAPE;
  if (!a_q || !a_sf || !a_gs || !b_q || !b_sf || !b_gs || !offsets || !tile_table || !d) return NVFP4_ERR_NULL;
  if (epilogue == NVFP4_EPI_SILU_MUL && !amax_out) return NVFP4_ERR_NULL;
  if (!nvfp4_aligned16(a_q) || !nvfp4_aligned16(a_sf) || !nvfp4_aligned16(b_q) || !nvfp4_aligned16(b_sf) ||
      !nvfp4_aligned16(d))
    return NVFP4_ERR_ALIGN;
  if (rows_cap == 0) return NVFP4_OK;
  return nvfp4_launch_grouped_gemm(a_q, a_sf, a_row_index, a_gs, b_q, b_sf, b_gs, offsets, tile_table, num_local,
                                   rows_cap, N, K, tile_m, epilogue, d, amax_out, (hipStream_t)stream);
}
