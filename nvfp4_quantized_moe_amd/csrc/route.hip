// Slot routing for one rank's share of experts (step a3 of the layer).
//
// nvfp4_mega_moe.py history, local-expert-id commit: top-k ids are global;
//   the rank owning [start, start + L) uses id - start.
// src history, 1-D slot-id commits: one 1-D slot order serves both GEMMs.
// nvfp4_cutedsl.py history, GPU-native routing and int32-offset commits:
//   per-expert counts, int32 prefix-sum offsets, pairs sorted by expert,
//   no host synchronisation.
// The sort here is stable in the flat index t*k + j (histogram, prefix sum,
// stable scatter), so the result is unique and deterministic.
//
// Steps over chunks of kRouteChunk flat entries:
//   count    per-chunk histogram in LDS
//   scan     counts, offsets, per-chunk bases, GEMM tile table
//   scatter  per chunk, in flat order: rank among equal keys from ballots on
//            the key bits, waves taking turns on an LDS running base per
//            expert; also writes the -1 / 0 padding of slots >= S.
// Scan and scatter share one launch (route_scan_scatter_kernel): every
// scatter workgroup sums the histograms for its own chunk's bases, and one
// more workgroup writes counts, offsets and the tile table. Past 65536
// histogram entries a one-workgroup scan kernel computes the bases first
// (route_scan_kernel, then route_scatter_kernel). Batches of at most 1024 flat
// entries (decode) take all steps in one workgroup and one launch
// (route_small_kernel). All paths give the same result.
#include "common.h"
#include "internal.h"
#include "amax.h"
#include "route_body.h"

namespace nvfp4 {

__global__ __launch_bounds__(256) void route_count_kernel(const int32_t* __restrict__ ids, int32_t n,
                                                          int32_t start, int32_t L,
                                                          int32_t* __restrict__ chunk_counts) {
  route_count_body(ids, n, start, L, chunk_counts, blockIdx.x);
}

// The layer's first launch for larger batches: workgroups [0, nchunks) take
// the per-chunk histograms of the route, the others the amax partials of the
// activation tensor. The two steps are independent, so they share one launch;
// the short histogram workgroups come first, so that they are dispatched
// before the amax workgroups fill the device (behind them they would wait for
// the amax pass to drain: 29 us for the pair against 18 us for the amax pass
// alone on the 8192 x 7168 shard).
__global__ __launch_bounds__(kAmaxThreads) void amax_count_kernel(
    const uint16_t* __restrict__ x, int64_t per, int64_t K, uint32_t* __restrict__ partial, int gx,
    uint32_t* __restrict__ clear, int n_clear, const int32_t* __restrict__ ids, int32_t n, int32_t start, int32_t L,
    int32_t* __restrict__ chunk_counts) {
  const int nchunks = (int)gridDim.x - gx;
  if ((int)blockIdx.x < nchunks)
    route_count_body(ids, n, start, L, chunk_counts, (int)blockIdx.x);
  else
    amax_block(x, per, nullptr, K, partial, clear, n_clear, 0, (int)blockIdx.x - nchunks, gx);
}

// One workgroup. Per-expert totals from the per-chunk histograms, then the
// offsets, the tile table and every chunk's first slot per expert. When the
// histograms fit in LDS (stage_cc), all threads first copy them there. Each
// wave takes whole experts and its 64 lanes walk the chunks 64 at a time, so
// a per-expert pass over the chunks is a few wave prefix sums.
__global__ __launch_bounds__(kScanThreads) void route_scan_kernel(
    const int32_t* __restrict__ chunk_counts, int nchunks, int L, int tile_m, int stage_cc,
    int32_t* __restrict__ counts, int32_t* __restrict__ offsets, int32_t* __restrict__ bases,
    int32_t* __restrict__ tile_table) {
  extern __shared__ int32_t sm[];
  int32_t* s_cnt = sm;            // [L]
  int32_t* s_off = sm + L;        // [L]
  int32_t* s_toff = sm + 2 * L;   // [L]
  int32_t* s_cc = sm + 3 * L;     // [nchunks][L] when stage_cc
  __shared__ int wsum[kScanThreads / 64 + 1];
  const int32_t* cc = chunk_counts;
  if (stage_cc) {
    for (int i = threadIdx.x; i < nchunks * L; i += blockDim.x) s_cc[i] = chunk_counts[i];
    __syncthreads();
    cc = s_cc;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kWaves = kScanThreads / 64;
  for (int e = wave; e < L; e += kWaves) {
    int total = 0;
    for (int c0 = 0; c0 < nchunks; c0 += 64) {
      const int ch = c0 + lane;
      const int incl = wave_inclusive_scan(ch < nchunks ? cc[(size_t)ch * L + e] : 0);
      total += __shfl(incl, 63, 64);
    }
    if (lane == 0) s_cnt[e] = total;
  }
  __syncthreads();
  scan_experts(s_cnt, L, tile_m, s_off, s_toff, wsum, counts, offsets, tile_table);
  // scan_experts ends with s_off written and synchronised
  for (int e = wave; e < L; e += kWaves) {
    int run = s_off[e];
    for (int c0 = 0; c0 < nchunks; c0 += 64) {
      const int ch = c0 + lane;
      const int v = ch < nchunks ? cc[(size_t)ch * L + e] : 0;
      const int incl = wave_inclusive_scan(v);
      if (ch < nchunks) bases[(size_t)ch * L + e] = run + incl - v;
      run += __shfl(incl, 63, 64);
    }
  }
}

// The whole route in one workgroup when T*k <= kScanThreads (decode-sized
// batches): histogram, scan and stable scatter, one flat entry per thread,
// the waves taking turns in flat order on the running slot of each expert.
__device__ __forceinline__ void route_small_body(
    const int32_t* __restrict__ ids, const float* __restrict__ w, int32_t n, int32_t k, int32_t start, int32_t L,
    int tile_m, int nbits, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ slot_token, int32_t* __restrict__ slot_expert, float* __restrict__ slot_weight,
    int32_t* __restrict__ token_slot, int32_t* __restrict__ tile_table) {
  extern __shared__ int32_t sm[];
  int32_t* s_cnt = sm;            // [L]
  int32_t* s_off = sm + L;        // [L], then the running slot of each expert
  int32_t* s_toff = sm + 2 * L;   // [L]
  __shared__ int wsum[kScanThreads / 64 + 1];
  for (int e = threadIdx.x; e < L; e += blockDim.x) s_cnt[e] = 0;
  __syncthreads();
  const int f = threadIdx.x;
  int key = L;  // L marks a dropped or absent entry
  if (f < n) {
    int64_t l = (int64_t)ids[f] - start;
    if (l >= 0 && l < L) key = (int)l;
  }
  if (key < L) atomicAdd(&s_cnt[key], 1);
  __syncthreads();
  const int S = scan_experts(s_cnt, L, tile_m, s_off, s_toff, wsum, counts, offsets, tile_table);
  if (f < n && f >= S) {
    slot_token[f] = -1;
    slot_expert[f] = -1;
    slot_weight[f] = 0.0f;
  }
  __syncthreads();  // every slot_* padding store precedes the scattered stores below
  int rank, cnt;
  bool last;
  wave_key_rank(key, nbits, &rank, &cnt, &last);
  const int wave = threadIdx.x >> 6;
  int slot = -1;
  for (int wv = 0; wv < kScanThreads / 64; ++wv) {
    if (wave == wv && key < L) {
      slot = s_off[key] + rank;
      if (last) s_off[key] += cnt;
    }
    __syncthreads();
  }
  if (f < n) {
    token_slot[f] = slot;
    if (slot >= 0) {
      slot_token[slot] = f / k;
      slot_expert[slot] = key;
      slot_weight[slot] = w[f];
    }
  }
}

__global__ __launch_bounds__(256) void route_scatter_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ w, int32_t n, int32_t k, int32_t start, int32_t L,
    int nbits, const int32_t* __restrict__ bases, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ slot_token, int32_t* __restrict__ slot_expert, float* __restrict__ slot_weight,
    int32_t* __restrict__ token_slot) {
  extern __shared__ int32_t running[];
  const int chunk = blockIdx.x;
  for (int e = threadIdx.x; e < L; e += blockDim.x) running[e] = bases[(size_t)chunk * L + e];
  route_scatter_chunk(ids, w, n, k, start, L, nbits, offsets[L], chunk, running, slot_token, slot_expert,
                      slot_weight, token_slot);
}

// Scan and scatter in one launch: workgroups [0, nchunks) scatter one chunk
// each, computing their chunk's first slot per expert from the per-chunk
// histograms; workgroup nchunks writes counts, offsets and the tile table.
__global__ __launch_bounds__(256) void route_scan_scatter_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ w, int32_t n, int32_t k, int32_t start, int32_t L,
    int tile_m, int nbits, const int32_t* __restrict__ chunk_counts, int nchunks, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ slot_token, int32_t* __restrict__ slot_expert,
    float* __restrict__ slot_weight, int32_t* __restrict__ token_slot, int32_t* __restrict__ tile_table) {
  const int bid = (int)blockIdx.x;
  if (bid < nchunks) {
    extern __shared__ int32_t route_lds[];  // running [L], totals [L]
    const int S = route_chunk_bases(chunk_counts, nchunks, L, bid, route_lds, route_lds + L);
    route_scatter_chunk(ids, w, n, k, start, L, nbits, S, bid, route_lds, slot_token, slot_expert, slot_weight,
                        token_slot);
  } else {
    route_tiles_wg(chunk_counts, nchunks, L, tile_m, counts, offsets, tile_table);
  }
}

__global__ __launch_bounds__(kScanThreads) void route_small_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ w, int32_t n, int32_t k, int32_t start, int32_t L,
    int tile_m, int nbits, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ slot_token, int32_t* __restrict__ slot_expert, float* __restrict__ slot_weight,
    int32_t* __restrict__ token_slot, int32_t* __restrict__ tile_table) {
  route_small_body(ids, w, n, k, start, L, tile_m, nbits, counts, offsets, slot_token, slot_expert, slot_weight,
                   token_slot, tile_table);
}

// The layer's first launch for decode-sized batches: workgroups [0, gx) take
// the amax partials of the activation tensor, workgroup gx routes. The two
// steps are independent, so they share one launch.
__global__ __launch_bounds__(kScanThreads) void amax_route_kernel(
    const uint16_t* __restrict__ x, int64_t per, int64_t K, uint32_t* __restrict__ partial, int gx,
    uint32_t* __restrict__ clear, int n_clear, const int32_t* __restrict__ ids, const float* __restrict__ w,
    int32_t n, int32_t k, int32_t start, int32_t L, int tile_m, int nbits, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ slot_token, int32_t* __restrict__ slot_expert,
    float* __restrict__ slot_weight, int32_t* __restrict__ token_slot, int32_t* __restrict__ tile_table) {
  if ((int)blockIdx.x < gx)
    amax_block(x, per, nullptr, K, partial, clear, n_clear, 0, blockIdx.x, gx);
  else
    route_small_body(ids, w, n, k, start, L, tile_m, nbits, counts, offsets, slot_token, slot_expert,
                     slot_weight, token_slot, tile_table);
}

}  // namespace nvfp4

using namespace nvfp4;

static int route_nchunks(int32_t T, int32_t k) { return (int)(((int64_t)T * k + kRouteChunk - 1) / kRouteChunk); }

size_t nvfp4_route_ws(int32_t T, int32_t k, int32_t num_local) {
  size_t per = nvfp4_align256((size_t)route_nchunks(T, k) * num_local * 4);
  return 2 * per + 256;
}

// Scan and scatter of a route whose per-chunk histograms are in ws (T*k > kScanThreads).
int nvfp4_launch_route_from_counts(const int32_t* topk_ids, const float* topk_w, int32_t T, int32_t k,
                                   int32_t expert_start, int32_t num_local, int32_t tile_m, int32_t* counts,
                                   int32_t* offsets, int32_t* slot_token, int32_t* slot_expert, float* slot_weight,
                                   int32_t* token_slot, int32_t* tile_table, void* ws, hipStream_t stream) {
  const int n = T * k;
  const int nchunks = route_nchunks(T, k);
  const int L = num_local;
  size_t per = nvfp4_align256((size_t)nchunks * L * 4);
  int32_t* chunk_counts = reinterpret_cast<int32_t*>(ws);
  int32_t* bases = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + per);
  if (nchunks > 0 && (int64_t)nchunks * L <= kFusedRouteMaxCounts) {
    // one launch: every scatter workgroup derives its chunk's bases itself
    hipLaunchKernelGGL(route_scan_scatter_kernel, dim3((unsigned)(nchunks + 1)), dim3(256), (size_t)3 * L * 4,
                       stream, topk_ids, topk_w, n, k, expert_start, L, tile_m, route_nbits(L), chunk_counts,
                       nchunks, counts, offsets, slot_token, slot_expert, slot_weight, token_slot, tile_table);
    NVFP4_CHECK_LAUNCH();
    return NVFP4_OK;
  }
  // stage the per-chunk histograms in LDS when everything fits in 64 KB
  const int stage_cc = ((int64_t)nchunks * L + 3 * L) * 4 <= 64 * 1024 ? 1 : 0;
  const size_t lds = (size_t)(3 * L + (stage_cc ? nchunks * L : 0)) * 4;
  hipLaunchKernelGGL(route_scan_kernel, dim3(1), dim3(kScanThreads), lds, stream, chunk_counts, nchunks, L, tile_m,
                     stage_cc, counts, offsets, bases, tile_table);
  NVFP4_CHECK_LAUNCH();
  if (nchunks > 0) {
    hipLaunchKernelGGL(route_scatter_kernel, dim3(nchunks), dim3(256), L * 4, stream, topk_ids, topk_w, n, k,
                       expert_start, L, route_nbits(L), bases, offsets, slot_token, slot_expert, slot_weight,
                       token_slot);
    NVFP4_CHECK_LAUNCH();
  }
  return NVFP4_OK;
}

int nvfp4_launch_route(const int32_t* topk_ids, const float* topk_w, int32_t T, int32_t k, int32_t expert_start,
                       int32_t num_local, int32_t tile_m, int32_t* counts, int32_t* offsets, int32_t* slot_token,
                       int32_t* slot_expert, float* slot_weight, int32_t* token_slot, int32_t* tile_table,
                       void* ws, hipStream_t stream) {
  const int n = T * k;
  const int nchunks = route_nchunks(T, k);
  const int L = num_local;
  if (n <= kScanThreads) {
    hipLaunchKernelGGL(route_small_kernel, dim3(1), dim3(kScanThreads), 3 * L * 4, stream, topk_ids, topk_w, n, k,
                       expert_start, L, tile_m, route_nbits(L), counts, offsets, slot_token, slot_expert,
                       slot_weight, token_slot, tile_table);
    NVFP4_CHECK_LAUNCH();
    return NVFP4_OK;
  }
  if (nchunks > 0) {
    hipLaunchKernelGGL(route_count_kernel, dim3(nchunks), dim3(256), L * 4, stream, topk_ids, n, expert_start, L,
                       reinterpret_cast<int32_t*>(ws));
    NVFP4_CHECK_LAUNCH();
  }
  return nvfp4_launch_route_from_counts(topk_ids, topk_w, T, k, expert_start, num_local, tile_m, counts, offsets,
                                        slot_token, slot_expert, slot_weight, token_slot, tile_table, ws, stream);
}

int nvfp4_launch_amax_count(const void* x_bf16, int64_t per, int64_t K, uint32_t* partial, uint32_t* clear,
                            int n_clear, const int32_t* topk_ids, int32_t T, int32_t k, int32_t expert_start,
                            int32_t num_local, void* route_ws, hipStream_t stream) {
  const int gx = nvfp4_amax_grid(per);
  const int nchunks = route_nchunks(T, k);
  hipLaunchKernelGGL(amax_count_kernel, dim3((unsigned)(gx + nchunks)), dim3(kAmaxThreads), num_local * 4, stream,
                     reinterpret_cast<const uint16_t*>(x_bf16), per, K, partial, gx, clear, n_clear, topk_ids, T * k,
                     expert_start, num_local, reinterpret_cast<int32_t*>(route_ws));
  NVFP4_CHECK_LAUNCH();
  return NVFP4_OK;
}

int nvfp4_amax_route_grid(int64_t per) {
  int64_t gx = (per / 8 + kScanThreads - 1) / kScanThreads;
  if (gx > kAmaxRouteMaxGrid) gx = kAmaxRouteMaxGrid;
  if (gx < 1) gx = 1;
  return (int)gx;
}

int nvfp4_launch_amax_route(const void* x_bf16, int64_t per, int64_t K, uint32_t* partial, uint32_t* clear,
                            int n_clear, const int32_t* topk_ids, const float* topk_w, int32_t T, int32_t k,
                            int32_t expert_start, int32_t num_local, int32_t tile_m, int32_t* counts,
                            int32_t* offsets, int32_t* slot_token, int32_t* slot_expert, float* slot_weight,
                            int32_t* token_slot, int32_t* tile_table, hipStream_t stream) {
  const int n = T * k;
  if (n > kScanThreads) return NVFP4_ERR_SHAPE;
  const int L = num_local;
  const int nbits = route_nbits(L);
  const int gx = nvfp4_amax_route_grid(per);
  hipLaunchKernelGGL(amax_route_kernel, dim3(gx + 1), dim3(kScanThreads), 3 * L * 4, stream,
                     reinterpret_cast<const uint16_t*>(x_bf16), per, K, partial, gx, clear, n_clear, topk_ids,
                     topk_w, n, k, expert_start, L, tile_m, nbits, counts, offsets, slot_token, slot_expert,
                     slot_weight, token_slot, tile_table);
  NVFP4_CHECK_LAUNCH();
  return NVFP4_OK;
}

extern "C" size_t moe_route_ws_bytes(int32_t T, int32_t k, int32_t num_local) {
  if (T < 0 || k < 1 || num_local < 1) return 0;
  return nvfp4_route_ws(T, k, num_local);
}

extern "C" int64_t nvfp4_tile_table_len(int64_t slot_capacity, int32_t num_local, int32_t tile_m) {
  if (slot_capacity < 0 || num_local < 1 || tile_m < 1) return 0;
  return 1 + 2 * (slot_capacity / tile_m + num_local);
}

static bool valid_tile_m(int32_t t) { return t >= 16 && t <= 256 && t % 16 == 0; }

extern "C" int moe_route_slots(const int32_t* topk_ids, const float* topk_w, int32_t T, int32_t k,
                               int32_t expert_start, int32_t num_local, int32_t tile_m, int32_t* counts,
                               int32_t* offsets, int32_t* slot_token, int32_t* slot_expert, float* slot_weight,
                               int32_t* token_slot, int32_t* tile_table, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || k < 1 || k > 64 || num_local < 1 || num_local > 4096 || !valid_tile_m(tile_m))
    return NVFP4_ERR_SHAPE;
  if ((int64_t)T * k >= (1ll << 30)) return NVFP4_ERR_SHAPE;
  if (!counts || !offsets || !tile_table || !ws) return NVFP4_ERR_NULL;
  if (T > 0 && (!topk_ids || !topk_w || !slot_token || !slot_expert || !slot_weight || !token_slot))
    return NVFP4_ERR_NULL;
  if (!nvfp4_aligned16(ws)) return NVFP4_ERR_ALIGN;
  if (ws_bytes < moe_route_ws_bytes(T, k, num_local)) return NVFP4_ERR_WORKSPACE;
  return nvfp4_launch_route(topk_ids, topk_w, T, k, expert_start, num_local, tile_m, counts, offsets, slot_token,
                            slot_expert, slot_weight, token_slot, tile_table, ws, (hipStream_t)stream);
}
