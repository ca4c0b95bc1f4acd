// BF16 -> NVFP4 quantizer (steps a1/a2/a6 of the layer).
//
// nvfp4_mega_moe.py history:
//   overflow-fix commit   gs = amax / (6 * 448) keeps every block scale <= 448
//   alpha commit          gs is returned next to (x_fp4, x_sf), not folded
//   three-bugs commit     stored scale = block_max / 6, nearest E2M1 magnitude,
//                         sign kept in bit 3 of the nibble
// tests history, packing-along-K commit: two nibbles per byte along K.
//
// The exact per-block rounding (threshold table in LDS) is in quant_block.h.
//
// Kernels: amax (wave reductions, one partial maximum per workgroup on the
// float bits, order-free) and quantize (each workgroup reduces the partials,
// derives gs and builds the threshold table in LDS, then quantizes 16-element
// blocks, two per thread and round, grid-stride over the tensor). With amax given (the
// h path) or with a fixed global scale (nvfp4_cutedsl.py history, static-scale
// commit: gs measured once at warmup, then no max reduction) only the
// quantize kernel runs.
#include "common.h"
#include "internal.h"
#include "amax.h"
#include "quant_block.h"
#include "route_body.h"

namespace nvfp4 {

__global__ void fill_u32_kernel(uint32_t* p, int n, uint32_t v) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

constexpr int kQuantPerCu = 8;      // quantize workgroups per CU (at most the resident count)
constexpr int kQuantBlocks = 2;     // 16-element blocks per thread and round

__global__ __launch_bounds__(kAmaxThreads) void amax_kernel(const uint16_t* __restrict__ x, int64_t per_batch,
                                                   const int32_t* __restrict__ rows_dev, int64_t K,
                                                   uint32_t* __restrict__ partial, uint32_t* __restrict__ clear,
                                                   int n_clear) {
  amax_block(x, per_batch, rows_dev, K, partial, clear, n_clear, blockIdx.y, blockIdx.x, gridDim.x);
}

// gs of tensor b (the fixed gs_in[b], or RN_f32(amax / 2688) with amax from
// amax_in or the partials) and its threshold table in LDS.
__device__ __forceinline__ float block_gs_and_lut(const float* __restrict__ gs_in, const float* __restrict__ amax_in,
                                                  const uint32_t* __restrict__ partial, int n_partial, int b,
                                                  uint32_t* lut /* [128][8] in LDS */) {
  __shared__ uint32_t red[4];
  float gs;
  if (gs_in) {
    gs = gs_in[b];
  } else {
    uint32_t m = 0;
    if (amax_in) {
      m = __float_as_uint(amax_in[b]);
    } else {
      for (int i = threadIdx.x; i < n_partial; i += blockDim.x) m = max(m, partial[(size_t)b * n_partial + i]);
      m = wave_max_u32(m);
      if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
      __syncthreads();
      m = max(max(red[0], red[1]), max(red[2], red[3]));
    }
    const float amax = __uint_as_float(m);
    // float64 quotient rounded to float32: 53 >= 2*24 + 2, so this equals one
    // correctly rounded float32 division
    gs = (float)((double)amax / 2688.0);
  }
  build_threshold_lut(gs, lut, threadIdx.x, blockDim.x);
  __syncthreads();
  return gs;
}

// Workgroup bid of nbid quantizing tensor b: gs and threshold table, then a
// grid-stride loop over the 16-element blocks.
template <bool kRowsDev>
__device__ __forceinline__ void quantize_body(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                              const int32_t* __restrict__ rows_dev, const float* __restrict__ gs_in,
                                              const float* __restrict__ amax_in,
                                              const uint32_t* __restrict__ partial, int n_partial,
                                              float* __restrict__ gs_out, uint8_t* __restrict__ q,
                                              uint8_t* __restrict__ sf, int b, int bid, int nbid) {
  __shared__ uint4 lut[kLutWords / 4];
  const float gs = block_gs_and_lut(gs_in, amax_in, partial, n_partial, b, reinterpret_cast<uint32_t*>(lut));
  if (gs_out && bid == 0 && threadIdx.x == 0) gs_out[b] = gs;
  const QuantScale qs = quant_scale(gs);
  int64_t rows = M;
  if (kRowsDev) rows = min(rows, (int64_t)rows_dev[0]);
  const int64_t nblk = rows * (K / 16);
  const uint16_t* xb = x + (size_t)b * M * K;
  uint8_t* qb = q + (size_t)b * M * (K / 2);
  uint8_t* sfb = sf + (size_t)b * M * (K / 16);
  auto one = [&](int64_t blk, const uint4& v0, const uint4& v1) {
    const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    uint2 packed;
    const uint32_t code = quantize_block16(w, qs, lut, &packed);
    *reinterpret_cast<uint2*>(qb + blk * 8) = packed;
    sfb[blk] = (uint8_t)code;
  };
  const uint4* src = reinterpret_cast<const uint4*>(xb);
  const int64_t stride = (int64_t)nbid * blockDim.x;
  int64_t blk = (int64_t)bid * blockDim.x + threadIdx.x;
  // kQuantBlocks blocks per thread and round, all loads issued before the
  // first block is quantized (blocks past the end re-read the last block and
  // store nothing)
  for (; blk < nblk; blk += kQuantBlocks * stride) {
    uint4 v[kQuantBlocks][2];
#pragma unroll
    for (int u = 0; u < kQuantBlocks; ++u) {
      const int64_t bu = min(blk + u * stride, nblk - 1);
      v[u][0] = src[2 * bu];
      v[u][1] = src[2 * bu + 1];
    }
#pragma unroll
    for (int u = 0; u < kQuantBlocks; ++u)
      if (blk + u * stride < nblk) one(blk + u * stride, v[u][0], v[u][1]);
  }
}

template <bool kRowsDev>
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ x, int64_t M, int64_t K,
                                                       const int32_t* __restrict__ rows_dev,
                                                       const float* __restrict__ gs_in,
                                                       const float* __restrict__ amax_in,
                                                       const uint32_t* __restrict__ partial, int n_partial,
                                                       float* __restrict__ gs_out, uint8_t* __restrict__ q,
                                                       uint8_t* __restrict__ sf) {
  quantize_body<kRowsDev>(x, M, K, rows_dev, gs_in, amax_in, partial, n_partial, gs_out, q, sf, blockIdx.y,
                          blockIdx.x, gridDim.x);
}

// The static layer's quantization of x with a fixed global scale for
// prefill-sized batches, with the route's per-chunk histograms in the same
// launch: workgroups [0, nchunks) count one chunk each (dispatched first, so
// that they run beside the quantization), the others quantize x with gs_in[0].
__global__ __launch_bounds__(256) void quantize_static_count_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, const float* __restrict__ gs_in, uint8_t* __restrict__ q,
    uint8_t* __restrict__ sf, const int32_t* __restrict__ ids, int32_t n, int32_t start, int32_t L,
    int32_t* __restrict__ chunk_counts, int nchunks) {
  const int bid = (int)blockIdx.x;
  if (bid < nchunks) {
    route_count_body(ids, n, start, L, chunk_counts, bid);
    return;
  }
  quantize_body<false>(x, M, K, nullptr, gs_in, nullptr, nullptr, 0, nullptr, q, sf, 0, bid - nchunks,
                       (int)gridDim.x - nchunks);
}

// The layer's quantization of x for prefill-sized batches with the route's
// scan and scatter in the same launch (both need only the per-chunk
// histograms of the previous launch, and the quantization needs neither):
// workgroups [0, nchunks) scatter one chunk each, computing their chunk's
// first slot per expert from the histograms; workgroup nchunks writes counts,
// offsets and the tile table; the others quantize x. Two launches of a few
// microseconds each (scan, scatter) no longer run between quantize x and the
// L1 GEMM.
__global__ __launch_bounds__(256) void quantize_route_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, const uint32_t* __restrict__ partial, int n_partial,
    float* __restrict__ gs_out, uint8_t* __restrict__ q, uint8_t* __restrict__ sf, const int32_t* __restrict__ ids,
    const float* __restrict__ w, int32_t n, int32_t k, int32_t start, int32_t L, int tile_m, int nbits,
    const int32_t* __restrict__ chunk_counts, int nchunks, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ slot_token, int32_t* __restrict__ slot_expert,
    float* __restrict__ slot_weight, int32_t* __restrict__ token_slot, int32_t* __restrict__ tile_table) {
  const int bid = (int)blockIdx.x;
  if (bid < nchunks) {
    extern __shared__ int32_t route_lds[];  // running [L], totals [L]
    const int S = route_chunk_bases(chunk_counts, nchunks, L, bid, route_lds, route_lds + L);
    route_scatter_chunk(ids, w, n, k, start, L, nbits, S, bid, route_lds, slot_token, slot_expert, slot_weight,
                        token_slot);
    return;
  }
  if (bid == nchunks) {
    route_tiles_wg(chunk_counts, nchunks, L, tile_m, counts, offsets, tile_table);
    return;
  }
  quantize_body<false>(x, M, K, nullptr, nullptr, nullptr, partial, n_partial, gs_out, q, sf, 0, bid - nchunks - 1,
                       (int)gridDim.x - nchunks - 1);
}

}  // namespace nvfp4

using namespace nvfp4;

// Workgroups of the quantize kernel: one per 256 blocks, at most as many as
// the device holds at once (CU count x resident workgroups per CU, queried
// once per device), so the grid-stride loop runs in a single round.
static std::atomic<int> g_quant_resident[kMaxDevices];

static int quant_grid(int64_t nblk) {
  const int dev = nvfp4_current_device();
  int resident = dev >= 0 ? g_quant_resident[dev].load(std::memory_order_relaxed) : 0;
  if (resident == 0) {
    int n_cu = 0, nb = 0;
    if (dev >= 0 && hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, reinterpret_cast<const void*>(quantize_kernel<false>), 256,
                                                     0) == hipSuccess &&
        n_cu > 0 && nb > 0) {
      resident = n_cu * (nb < kQuantPerCu ? nb : kQuantPerCu);
      g_quant_resident[dev].store(resident, std::memory_order_relaxed);
    } else {
      resident = 2048;
    }
  }
  int64_t g = (nblk + 255) / 256;
  if (g > resident) g = resident;
  if (g < 1) g = 1;
  return (int)g;
}

// workgroups of the amax pass per tensor: one round of eight 16-byte loads
// per thread, at most kAmaxGrid workgroups (fixed by the tensor size); every
// quantize workgroup reduces the partials of its tensor, so they are few
constexpr int kAmaxGrid = 512;
int nvfp4_amax_grid(int64_t per_batch) {
  int64_t gx = (per_batch / 8 + kAmaxThreads * 8 - 1) / (kAmaxThreads * 8);
  if (gx > kAmaxGrid) gx = kAmaxGrid;
  if (gx < 1) gx = 1;
  return (int)gx;
}

int nvfp4_launch_fill_u32(uint32_t* p, int n, uint32_t v, hipStream_t stream) {
  hipLaunchKernelGGL(fill_u32_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, p, n, v);
  NVFP4_CHECK_LAUNCH();
  return NVFP4_OK;
}

size_t nvfp4_quant_ws_layout(int64_t B) { return nvfp4_align256((size_t)B * kAmaxGrid * 4); }

// Internal launcher shared by nvfp4_quantize and the layer: two launches
// (amax partials, quantize) or one when amax_in is given.
int nvfp4_launch_quantize(const void* x_bf16, int64_t B, int64_t M, int64_t K, const float* amax_in,
                          const int32_t* rows_dev, uint8_t* q, uint8_t* sf, float* gs_out, void* ws,
                          uint32_t* clear, int n_clear, hipStream_t stream) {
  uint32_t* partial = reinterpret_cast<uint32_t*>(ws);
  const uint16_t* x = reinterpret_cast<const uint16_t*>(x_bf16);
  const int64_t per = M * K;
  const int gx = nvfp4_amax_grid(per);
  if (!amax_in) {
    hipLaunchKernelGGL(amax_kernel, dim3((unsigned)gx, (unsigned)B), dim3(kAmaxThreads), 0, stream, x, per, rows_dev, K,
                       partial, clear, clear ? n_clear : 0);
    NVFP4_CHECK_LAUNCH();
  } else if (clear && n_clear > 0) {
    hipLaunchKernelGGL(fill_u32_kernel, dim3(1), dim3(256), 0, stream, clear, n_clear, 0u);
    NVFP4_CHECK_LAUNCH();
  }
  // M == 0 still launches one workgroup per tensor: it writes gs
  dim3 grid((unsigned)quant_grid(M * (K / 16)), (unsigned)B);
  if (rows_dev)
    hipLaunchKernelGGL(quantize_kernel<true>, grid, dim3(256), 0, stream, x, M, K, rows_dev, nullptr, amax_in, partial,
                       gx, gs_out, q, sf);
  else
    hipLaunchKernelGGL(quantize_kernel<false>, grid, dim3(256), 0, stream, x, M, K, rows_dev, nullptr, amax_in, partial,
                       gx, gs_out, q, sf);
  NVFP4_CHECK_LAUNCH();
  return NVFP4_OK;
}

// Quantize one tensor whose amax partials (n_partial of them) are already in ws.
int nvfp4_launch_quantize_from_partials(const void* x_bf16, int64_t M, int64_t K, const void* ws, int n_partial,
                                        uint8_t* q, uint8_t* sf, float* gs_out, hipStream_t stream) {
  const uint32_t* partial = reinterpret_cast<const uint32_t*>(ws);
  const uint16_t* x = reinterpret_cast<const uint16_t*>(x_bf16);
  dim3 grid((unsigned)quant_grid(M * (K / 16)), 1u);
  hipLaunchKernelGGL(quantize_kernel<false>, grid, dim3(256), 0, stream, x, M, K, nullptr, nullptr, nullptr,
                     partial, n_partial, gs_out, q, sf);
  NVFP4_CHECK_LAUNCH();
  return NVFP4_OK;
}

// Quantize x (amax partials in ws) and, in the same launch, the route's scan
// and scatter from the per-chunk histograms in route_ws (layer, T*k > 1024).
// Returns NVFP4_ERR_ARG when the histograms are too many for the per-workgroup
// base computation (the caller then launches the route kernels).
int nvfp4_launch_quantize_route(const void* x_bf16, int64_t M, int64_t K, const void* ws, int n_partial,
                                uint8_t* q, uint8_t* sf, float* gs_out, const int32_t* topk_ids,
                                const float* topk_w, int32_t T, int32_t k, int32_t expert_start, int32_t num_local,
                                int32_t tile_m, const void* route_ws, int32_t* counts, int32_t* offsets,
                                int32_t* slot_token, int32_t* slot_expert, float* slot_weight, int32_t* token_slot,
                                int32_t* tile_table, hipStream_t stream) {
  const int n = T * k;
  const int nchunks = (int)(((int64_t)n + kRouteChunk - 1) / kRouteChunk);
  const int L = num_local;
  if (nchunks < 1 || (int64_t)nchunks * L > kFusedRouteMaxCounts) return NVFP4_ERR_ARG;
  const int nq = quant_grid(M * (K / 16));
  const int nr = nchunks + 1;
  const int grid = nr + (nq - nr > 1 ? nq - nr : 1);
  hipLaunchKernelGGL(quantize_route_kernel, dim3((unsigned)grid), dim3(256), (size_t)3 * L * 4, stream,
                     reinterpret_cast<const uint16_t*>(x_bf16), M, K, reinterpret_cast<const uint32_t*>(ws),
                     n_partial, gs_out, q, sf, topk_ids, topk_w, n, k, expert_start, L, tile_m, route_nbits(L),
                     reinterpret_cast<const int32_t*>(route_ws), nchunks, counts, offsets, slot_token, slot_expert,
                     slot_weight, token_slot, tile_table);
  NVFP4_CHECK_LAUNCH();
  return NVFP4_OK;
}

// Quantize x [M, K] with the fixed global scale gs_in[0] and, in the same
// launch, the route's per-chunk histograms into route_ws (static layer,
// T*k > 1024; nvfp4_launch_route_from_counts finishes the route).
int nvfp4_launch_quantize_static_count(const void* x_bf16, int64_t M, int64_t K, const float* gs_in, uint8_t* q,
                                       uint8_t* sf, const int32_t* topk_ids, int32_t T, int32_t k,
                                       int32_t expert_start, int32_t num_local, void* route_ws, hipStream_t stream) {
  const int n = T * k;
  const int nchunks = (int)(((int64_t)n + kRouteChunk - 1) / kRouteChunk);
  const int nq = quant_grid(M * (K / 16));
  const int grid = nchunks + (nq - nchunks > 1 ? nq - nchunks : 1);
  hipLaunchKernelGGL(quantize_static_count_kernel, dim3((unsigned)grid), dim3(256), (size_t)num_local * 4, stream,
                     reinterpret_cast<const uint16_t*>(x_bf16), M, K, gs_in, q, sf, topk_ids, n, expert_start,
                     num_local, reinterpret_cast<int32_t*>(route_ws), nchunks);
  NVFP4_CHECK_LAUNCH();
  return NVFP4_OK;
}

// Quantize with fixed global scales gs_in[b]: one launch, no amax pass.
int nvfp4_launch_quantize_static(const void* x_bf16, int64_t B, int64_t M, int64_t K, const float* gs_in,
                                 const int32_t* rows_dev, uint8_t* q, uint8_t* sf, hipStream_t stream) {
  const uint16_t* x = reinterpret_cast<const uint16_t*>(x_bf16);
  dim3 grid((unsigned)quant_grid(M * (K / 16)), (unsigned)B);
  if (rows_dev)
    hipLaunchKernelGGL(quantize_kernel<true>, grid, dim3(256), 0, stream, x, M, K, rows_dev, gs_in, nullptr, nullptr,
                       0, nullptr, q, sf);
  else
    hipLaunchKernelGGL(quantize_kernel<false>, grid, dim3(256), 0, stream, x, M, K, rows_dev, gs_in, nullptr,
                       nullptr, 0, nullptr, q, sf);
  NVFP4_CHECK_LAUNCH();
  return NVFP4_OK;
}

extern "C" int nvfp4_quantize_static(const void* x_bf16, int64_t B, int64_t M, int64_t K, const float* gs_in,
                                     uint8_t* q, uint8_t* sf, void* stream) {
  if (B < 1 || B > 65535 || M < 0 || K <= 0 || K % 32 != 0) return NVFP4_ERR_SHAPE;
  if (!gs_in) return NVFP4_ERR_NULL;
  if (M > 0 && (!x_bf16 || !q || !sf)) return NVFP4_ERR_NULL;
  if (M > 0 && (!nvfp4_aligned16(x_bf16) || !nvfp4_aligned16(q) || !nvfp4_aligned16(sf))) return NVFP4_ERR_ALIGN;
  if (M == 0) return NVFP4_OK;
  return nvfp4_launch_quantize_static(x_bf16, B, M, K, gs_in, nullptr, q, sf, (hipStream_t)stream);
}

// ------------------------------------------- quantize without a workspace
// Amax partials of nvfp4_quantize_noalloc: kAmaxGrid words per tensor for at
// most kNoAllocMaxTensors tensors (256 KB), one copy on every device the
// library runs on, held until the process ends. Every call on a device shares
// that device's copy; the amax pass writes every partial the quantize kernel
// of the same call reads, so nothing has to start at zero.
constexpr int kNoAllocMaxTensors = 128;
static __device__ __align__(256) uint32_t scratch[kNoAllocMaxTensors * kAmaxGrid];

// Device address of `scratch` on each device, taken once with that device
// current (in host code the array's name is only a host-side stand-in).
static std::atomic<uintptr_t> g_scratch_addr[kMaxDevices];

static uint32_t* noalloc_scratch(int dev) {
  uintptr_t a = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (a == 0) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    a = reinterpret_cast<uintptr_t>(p);
    g_scratch_addr[dev].store(a, std::memory_order_release);
  }
  return reinterpret_cast<uint32_t*>(a);
}

extern "C" int nvfp4_quantize_noalloc(const void* x_bf16, int64_t B, int64_t M, int64_t K, const float* amax_in,
                                      uint8_t* q, uint8_t* sf, float* gs_out, void* stream) {
  if (B < 1 || B > 65535 || M < 0 || K <= 0 || K % 32 != 0) return NVFP4_ERR_SHAPE;
  if (B > kNoAllocMaxTensors) return NVFP4_ERR_WORKSPACE;
  if (M > 0 && (!x_bf16 || !q || !sf)) return NVFP4_ERR_NULL;
  if (!gs_out) return NVFP4_ERR_NULL;
  if (M > 0 && (!nvfp4_aligned16(x_bf16) || !nvfp4_aligned16(q) || !nvfp4_aligned16(sf))) return NVFP4_ERR_ALIGN;
  const int dev = nvfp4_current_device();
  if (dev < 0) return NVFP4_ERR_HIP;
  uint32_t* ws = noalloc_scratch(dev);
  if (!ws) return NVFP4_ERR_HIP;
  return nvfp4_launch_quantize(x_bf16, B, M, K, amax_in, nullptr, q, sf, gs_out, ws, nullptr, 0,
                               (hipStream_t)stream);
}

extern "C" size_t nvfp4_quantize_ws_bytes(int64_t B, int64_t M, int64_t K) {
  (void)M;
  (void)K;
  if (B < 1) return 0;
  return nvfp4_quant_ws_layout(B);
}

extern "C" int nvfp4_quantize(const void* x_bf16, int64_t B, int64_t M, int64_t K, const float* amax_in,
                              uint8_t* q, uint8_t* sf, float* gs_out, void* ws, size_t ws_bytes, void* stream) {
  if (B < 1 || B > 65535 || M < 0 || K <= 0 || K % 32 != 0) return NVFP4_ERR_SHAPE;
  if (M > 0 && (!x_bf16 || !q || !sf)) return NVFP4_ERR_NULL;
  if (!gs_out || !ws) return NVFP4_ERR_NULL;
  if ((M > 0 && (!nvfp4_aligned16(x_bf16) || !nvfp4_aligned16(q) || !nvfp4_aligned16(sf))) ||
      !nvfp4_aligned16(ws))
    return NVFP4_ERR_ALIGN;
  if (ws_bytes < nvfp4_quantize_ws_bytes(B, M, K)) return NVFP4_ERR_WORKSPACE;
  return nvfp4_launch_quantize(x_bf16, B, M, K, amax_in, nullptr, q, sf, gs_out, ws, nullptr, 0,
                               (hipStream_t)stream);
}
