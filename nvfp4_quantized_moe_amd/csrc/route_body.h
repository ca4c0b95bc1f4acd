// Device code of the slot routing (step a3), shared by the route kernels and
// by the layer's fused quantize + route launch.
//
// nvfp4_mega_moe.py history, local-expert-id commit: top-k ids are global;
//   the rank owning [start, start + L) uses id - start.
// nvfp4_cutedsl.py history, GPU-native routing commits: per-expert counts,
//   prefix-sum offsets, pairs sorted by expert, no host synchronisation.
// The sort is stable in the flat index t*k + j (histogram, prefix sum, stable
// scatter), so the result is unique and deterministic.
#pragma once
#include "common.h"
#include "internal.h"

namespace nvfp4 {

constexpr int kScanThreads = 1024;

// Histogram of chunk `chunk`'s local expert ids (any workgroup size).
__device__ __forceinline__ void route_count_body(const int32_t* __restrict__ ids, int32_t n, int32_t start, int32_t L,
                                                 int32_t* __restrict__ chunk_counts, int chunk) {
  extern __shared__ int32_t hist[];
  for (int e = threadIdx.x; e < L; e += blockDim.x) hist[e] = 0;
  __syncthreads();
  const int base = chunk * kRouteChunk;
  for (int i = threadIdx.x; i < kRouteChunk; i += blockDim.x) {
    int f = base + i;
    if (f < n) {
      int64_t l = (int64_t)ids[f] - start;
      if (l >= 0 && l < L) atomicAdd(&hist[l], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < L; e += blockDim.x) chunk_counts[(size_t)chunk * L + e] = hist[e];
}

// Exclusive prefix sum over a workgroup of up to kScanThreads threads (a
// multiple of 64); *total receives the sum.
__device__ int block_exclusive_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < (int)blockDim.x / 64; ++w) {
      int t = wsum[w];
      wsum[w] = run;
      run += t;
    }
    wsum[blockDim.x / 64] = run;
  }
  __syncthreads();
  int r = wsum[wave] + incl - v;
  *total = wsum[blockDim.x / 64];
  __syncthreads();
  return r;
}

// Offsets and tile bases of every expert from s_cnt (one workgroup of up to
// kScanThreads threads; experts in contiguous runs of `per` per thread): writes
// s_off, s_toff, counts, offsets, tile_table; returns S.
__device__ int scan_experts(const int32_t* s_cnt, int L, int tile_m, int32_t* s_off, int32_t* s_toff, int* wsum,
                            int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                            int32_t* __restrict__ tile_table) {
  const int per = (L + (int)blockDim.x - 1) / (int)blockDim.x;
  const int e0 = threadIdx.x * per;
  int rows = 0, tiles = 0;
  for (int e = e0; e < min(L, e0 + per); ++e) {
    rows += s_cnt[e];
    tiles += (s_cnt[e] + tile_m - 1) / tile_m;
  }
  int total_rows, total_tiles;
  int row_base = block_exclusive_scan(rows, wsum, &total_rows);
  int tile_base = block_exclusive_scan(tiles, wsum, &total_tiles);
  for (int e = e0; e < min(L, e0 + per); ++e) {
    s_off[e] = row_base;
    s_toff[e] = tile_base;
    row_base += s_cnt[e];
    tile_base += (s_cnt[e] + tile_m - 1) / tile_m;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < L; e += blockDim.x) {
    counts[e] = s_cnt[e];
    offsets[e] = s_off[e];
    int nt = (s_cnt[e] + tile_m - 1) / tile_m;
    for (int mt = 0; mt < nt; ++mt) {
      int t = s_toff[e] + mt;
      tile_table[1 + 2 * t] = e;
      tile_table[2 + 2 * t] = s_off[e] + mt * tile_m;
    }
  }
  if (threadIdx.x == 0) {
    offsets[L] = total_rows;
    tile_table[0] = total_tiles;
  }
  return total_rows;
}

// Rank of this lane's key among the lanes of its wave with the same key
// (lower lanes first), the number of such lanes, and whether this lane is
// the highest of them. Keys are compared on their nbits low bits.
__device__ __forceinline__ void wave_key_rank(int key, int nbits, int* rank, int* cnt, bool* last) {
  const int lane = threadIdx.x & 63;
  const unsigned long long below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  unsigned long long match = ~0ull;
  for (int b = 0; b < nbits; ++b) {
    int bit = (key >> b) & 1;
    unsigned long long m = __ballot(bit);
    match &= bit ? m : ~m;
  }
  *rank = __popcll(match & below);
  *cnt = __popcll(match);
  *last = (match >> lane) == 1ull;
}

// Inclusive prefix sum across the 64 lanes of a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & 63;
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o, 64);
    if (lane >= o) v += t;
  }
  return v;
}

// Sum over the 64 lanes of a wave (every lane gets it).
__device__ __forceinline__ int wave_sum_i32(int v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Per-expert totals of the per-chunk histograms cc [nchunks][L] into s_cnt:
// each wave takes whole experts, its lanes 64 chunks at a time.
__device__ __forceinline__ void route_expert_totals(const int32_t* __restrict__ cc, int nchunks, int L,
                                                    int32_t* s_cnt) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  for (int e = wave; e < L; e += nwaves) {
    int tot = 0;
    for (int c0 = 0; c0 < nchunks; c0 += 64) {
      const int ch = c0 + lane;
      tot += wave_sum_i32(ch < nchunks ? cc[(size_t)ch * L + e] : 0);
    }
    if (lane == 0) s_cnt[e] = tot;
  }
  __syncthreads();
}

// One workgroup: counts, offsets and the GEMM tile table from the per-chunk
// histograms (dynamic LDS: 3 L words).
__device__ __forceinline__ void route_tiles_wg(const int32_t* __restrict__ cc, int nchunks, int L, int tile_m,
                                               int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                               int32_t* __restrict__ tile_table) {
  extern __shared__ int32_t sm[];
  __shared__ int wsum[kScanThreads / 64 + 1];
  route_expert_totals(cc, nchunks, L, sm);
  scan_experts(sm, L, tile_m, sm + L, sm + 2 * L, wsum, counts, offsets, tile_table);
}

// First slot of every expert for chunk `chunk`, from the histograms alone:
// running[e] = (entries of experts < e over all chunks) + (entries of e in
// chunks < chunk). s_tot: LDS [L]. Returns S, the number of local slots.
__device__ __forceinline__ int route_chunk_bases(const int32_t* __restrict__ cc, int nchunks, int L, int chunk,
                                                 int32_t* running, int32_t* s_tot) {
  __shared__ int wsum[kScanThreads / 64 + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nwaves = blockDim.x >> 6;
  for (int e = wave; e < L; e += nwaves) {
    int tot = 0, pre = 0;
    for (int c0 = 0; c0 < nchunks; c0 += 64) {
      const int ch = c0 + lane;
      const int v = ch < nchunks ? cc[(size_t)ch * L + e] : 0;
      tot += wave_sum_i32(v);
      pre += wave_sum_i32(ch < chunk ? v : 0);
    }
    if (lane == 0) {
      s_tot[e] = tot;
      running[e] = pre;
    }
  }
  __syncthreads();
  const int per = (L + (int)blockDim.x - 1) / (int)blockDim.x;
  const int e0 = threadIdx.x * per;
  int rows = 0;
  for (int e = e0; e < min(L, e0 + per); ++e) rows += s_tot[e];
  int total;
  int base = block_exclusive_scan(rows, wsum, &total);
  for (int e = e0; e < min(L, e0 + per); ++e) {
    running[e] += base;
    base += s_tot[e];
  }
  __syncthreads();
  return total;
}

// Stable scatter of chunk `chunk` (a workgroup of 256 threads) with
// running[e] (LDS) holding the chunk's first slot of expert e and S the
// number of local slots: writes the -1 / 0 padding of the chunk's slots >= S,
// then, in flat order, each entry's slot (rank among equal keys from ballots
// on the key bits, the 4 waves taking turns on running[]).
__device__ __forceinline__ void route_scatter_chunk(
    const int32_t* __restrict__ ids, const float* __restrict__ w, int32_t n, int32_t k, int32_t start, int32_t L,
    int nbits, int S, int chunk, int32_t* running, int32_t* __restrict__ slot_token,
    int32_t* __restrict__ slot_expert, float* __restrict__ slot_weight, int32_t* __restrict__ token_slot) {
  for (int i = threadIdx.x; i < kRouteChunk; i += blockDim.x) {
    int s = chunk * kRouteChunk + i;
    if (s >= S && s < n) {
      slot_token[s] = -1;
      slot_expert[s] = -1;
      slot_weight[s] = 0.0f;
    }
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6;
  for (int round = 0; round < kRouteChunk / 256; ++round) {
    const int f = chunk * kRouteChunk + round * 256 + threadIdx.x;
    int key = L;  // L marks a dropped or absent entry
    if (f < n) {
      int64_t l = (int64_t)ids[f] - start;
      if (l >= 0 && l < L) key = (int)l;
    }
    int rank, cnt;
    bool last;
    wave_key_rank(key, nbits, &rank, &cnt, &last);
    int slot = -1;
    for (int wv = 0; wv < 4; ++wv) {
      if (wave == wv && key < L) {
        slot = running[key] + rank;
        if (last) running[key] += cnt;
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
}

// Route kernels' bit count of the keys 0..L (L marks a dropped entry).
__host__ __device__ __forceinline__ int route_nbits(int L) {
  int nbits = 1;
  while ((1 << nbits) <= L) ++nbits;
  return nbits;
}

}  // namespace nvfp4
