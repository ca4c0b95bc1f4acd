// Weighted scatter back to token rows (step a8) and the offline gate/up
// scale fold (weight preparation).
//
// Scatter — nvfp4_cutedsl.py history, GPU-native routing commit: each slot's
// output row is added into its token's row times the routing weight; the
// pages use an atomic scatter-add, here each token gathers its own k slots
// in increasing j with float32 multiply then add (no fused multiply-add) and
// rounds once to BF16, so the result is deterministic. Tokens with no local
// slot get zeros (nvfp4_mega_moe.py history, expert-parallel note: the rank
// writes a local partial output that the caller reduces).
//
// Fold — nvfp4_cutedsl.py history, finalize_weights commit: gate and up are
// brought to one global scale max(gs_gate, gs_up) by one float32 multiply of
// the smaller half's block scales by the ratio and a round trip to E4M3.
#include "common.h"
#include "internal.h"

namespace nvfp4 {

constexpr int kScatterChunks = 4;  // 8-element chunks per thread and round, their loads in flight together
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void scatter_kernel(const uint16_t* __restrict__ y,
                                                      const int32_t* __restrict__ token_slot,
                                                      const float* __restrict__ topk_w, int T, int k, int H,
                                                      uint16_t* __restrict__ out) {
#pragma clang fp contract(off)  // separate multiply and add roundings, in j order
  __shared__ int s_slot[64];
  __shared__ float s_w[64];
  __shared__ int s_n;
  const int t = blockIdx.x;
  // the token's local slots, compacted in increasing j (lane j of wave 0
  // takes entry j; its place is the number of local entries before it)
  if (threadIdx.x < 64) {
    const int j = threadIdx.x;
    const int slot = j < k ? token_slot[(size_t)t * k + j] : -1;
    const float w = j < k ? topk_w[(size_t)t * k + j] : 0.0f;
    const uint64_t local = __ballot(slot >= 0);
    if (slot >= 0) {
      const int at = __popcll(local & ((1ull << j) - 1ull));
      s_slot[at] = slot;
      s_w[at] = w;
    }
    if (j == 0) s_n = __popcll(local);
  }
  __syncthreads();
  const int n = s_n;
  // workgroup (t, y) takes every gridDim.y-th run of 256 8-element chunks of
  // row t; a thread's kScatterChunks chunks of a round lie one such step apart
  const int nchunk = H / 8;
  const int step = gridDim.y * blockDim.x;
  for (int c0 = blockIdx.y * blockDim.x + threadIdx.x; c0 < nchunk; c0 += kScatterChunks * step) {
    float acc[kScatterChunks][8];
#pragma unroll
    for (int g = 0; g < kScatterChunks; ++g)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[g][e] = 0.0f;
    for (int jj = 0; jj < n; ++jj) {
      const uint16_t* row = y + (size_t)s_slot[jj] * H;
      const float w = s_w[jj];
      uint4 v[kScatterChunks];
#pragma unroll
      for (int g = 0; g < kScatterChunks; ++g) {
        const int c = c0 + g * step;
        v[g] = c < nchunk ? *reinterpret_cast<const uint4*>(row + c * 8) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int g = 0; g < kScatterChunks; ++g) {
        const uint32_t u[4] = {v[g].x, v[g].y, v[g].z, v[g].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float p0 = w * bf16_to_f32(u[q] & 0xFFFFu);
          const float p1 = w * bf16_to_f32(u[q] >> 16);
          acc[g][2 * q] = acc[g][2 * q] + p0;
          acc[g][2 * q + 1] = acc[g][2 * q + 1] + p1;
        }
      }
    }
#pragma unroll
    for (int g = 0; g < kScatterChunks; ++g) {
      const int c = c0 + g * step;
      if (c >= nchunk) continue;
      const u32x4_t ov = {f32x2_to_bf16x2(acc[g][0], acc[g][1]), f32x2_to_bf16x2(acc[g][2], acc[g][3]),
                          f32x2_to_bf16x2(acc[g][4], acc[g][5]), f32x2_to_bf16x2(acc[g][6], acc[g][7])};
      // non-temporal: the output is not read again in the layer, and its
      // lines would otherwise be written back from the caches during the next
      // launches (the next layer step's amax pass ran 7 us longer for it)
      __builtin_nontemporal_store(ov, reinterpret_cast<u32x4_t*>(out + (size_t)t * H + c * 8));
    }
  }
}

__global__ __launch_bounds__(256) void fold_kernel(uint8_t* __restrict__ w1_sf, const float* __restrict__ gs_gate,
                                                   const float* __restrict__ gs_up, float* __restrict__ gs1,
                                                   int L, int inter, int k16) {
  const int64_t per_e = (int64_t)2 * inter * k16;
  const int64_t n = per_e * L;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int e = (int)(idx / per_e);
    const int64_t rem = idx - (int64_t)e * per_e;
    const int row = (int)(rem / k16);
    const float g = gs_gate[e], u = gs_up[e];
    const float m = fmaxf(g, u);
    if (rem == 0) gs1[e] = m;
    const float p = row < inter ? g : u;
    if (p < m) {
      const float ratio = (float)((double)p / (double)m);  // = RN_f32(p / m): 53 >= 2*24 + 2
      const float prod = __fmul_rn(e4m3_to_f32(w1_sf[idx]), ratio);
      w1_sf[idx] = (uint8_t)e4m3_encode_rne_sat((double)prod);
    }
  }
}

}  // namespace nvfp4

using namespace nvfp4;

int nvfp4_launch_scatter(const void* y_bf16, const int32_t* token_slot, const float* topk_w, int32_t T, int32_t k,
                         int32_t H, void* out_bf16, hipStream_t stream) {
  if (T == 0) return NVFP4_OK;
  // small batches split each row over up to one chunk per thread, so that
  // about 1024 workgroups run; large batches keep one workgroup per row
  const int64_t gy_max = ((int64_t)H / 8 + 255) / 256;
  int64_t gy = (1024 + T - 1) / T;
  if (gy > gy_max) gy = gy_max;
  if (gy > 65535) return NVFP4_ERR_SHAPE;
  hipLaunchKernelGGL(scatter_kernel, dim3(T, (unsigned)gy), dim3(256), 0, stream, reinterpret_cast<const uint16_t*>(y_bf16),
                     token_slot, topk_w, T, k, H, reinterpret_cast<uint16_t*>(out_bf16));
  NVFP4_CHECK_LAUNCH();
  return NVFP4_OK;
}

extern "C" int moe_weighted_scatter(const void* y_bf16, const int32_t* token_slot, const float* topk_w, int32_t T,
                                    int32_t k, int32_t H, void* out_bf16, void* stream) {
  if (T < 0 || k < 1 || k > 64 || H <= 0 || H % 8 != 0) return NVFP4_ERR_SHAPE;
  if (T > 0 && (!y_bf16 || !token_slot || !topk_w || !out_bf16)) return NVFP4_ERR_NULL;
  if (T > 0 && (!nvfp4_aligned16(y_bf16) || !nvfp4_aligned16(out_bf16))) return NVFP4_ERR_ALIGN;
  return nvfp4_launch_scatter(y_bf16, token_slot, topk_w, T, k, H, out_bf16, (hipStream_t)stream);
}

extern "C" int nvfp4_fold_scales(uint8_t* w1_sf, const float* gs_gate, const float* gs_up, float* gs1,
                                 int32_t num_local, int32_t inter, int32_t K, void* stream) {
  if (num_local < 1 || inter < 1 || K <= 0 || K % 16 != 0) return NVFP4_ERR_SHAPE;
  if (!w1_sf || !gs_gate || !gs_up || !gs1) return NVFP4_ERR_NULL;
  const int64_t n = (int64_t)num_local * 2 * inter * (K / 16);
  int64_t grid = (n + 255) / 256;
  if (grid > 4096) grid = 4096;
  hipLaunchKernelGGL(fold_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, w1_sf, gs_gate, gs_up,
                     gs1, num_local, inter, K / 16);
  NVFP4_CHECK_LAUNCH();
  return NVFP4_OK;
}
