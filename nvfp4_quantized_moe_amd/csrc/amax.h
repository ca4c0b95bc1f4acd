// Per-workgroup partial maximum of |x| (step a1), shared by the quantizer's
// amax pass and the layer's fused amax + route launch.
#pragma once
#include "common.h"

namespace nvfp4 {

constexpr int kAmaxThreads = 1024;  // threads per workgroup of the amax passes over large tensors

// Workgroup blk of nblk over tensor b: partial[b * nblk + blk] = max |x| over
// the workgroup's grid-stride share of the first min(per_batch, rows_dev[0] * K)
// elements of x[b], as float32 bits (|x| >= 0, so the unsigned order of the
// bits is the order of the values). Every workgroup writes its slot, so
// nothing has to be cleared first. Workgroup 0 of tensor 0 also zeroes
// clear[0..n_clear), which later kernels of the same stream use as
// atomic-max targets. Any workgroup size up to 1024.
__device__ __forceinline__ void amax_block(const uint16_t* __restrict__ x, int64_t per_batch,
                                           const int32_t* __restrict__ rows_dev, int64_t K,
                                           uint32_t* __restrict__ partial, uint32_t* __restrict__ clear,
                                           int n_clear, int b, int blk, int nblk) {
  if (blk == 0 && b == 0)
    for (int i = threadIdx.x; i < n_clear; i += blockDim.x) clear[i] = 0u;
  int64_t n = per_batch;
  if (rows_dev) {
    int64_t r = rows_dev[0];
    n = min(n, r * K);
  }
  const uint4* xv = reinterpret_cast<const uint4*>(x + (int64_t)b * per_batch);
  const int64_t nv = n / 8;
  const int64_t stride = (int64_t)nblk * blockDim.x;
  uint32_t m = 0;
  auto fold = [&](const uint4& v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) m = max(m, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
  };
  // eight independent 16-byte loads in flight per thread (the maximum is
  // order-free); a load past the end re-reads the thread's first vector of
  // the round, so every round issues all eight at once
  for (int64_t i = (int64_t)blk * blockDim.x + threadIdx.x; i < nv; i += 8 * stride) {
    uint4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t k = i + u * stride;
      v[u] = xv[k < nv ? k : i];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) fold(v[u]);
  }
  m = wave_max_u32(m);
  __shared__ uint32_t red[16];
  const int nwaves = (int)(blockDim.x + 63) / 64;
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t r = 0;
    for (int i = 0; i < nwaves; ++i) r = max(r, red[i]);
    partial[(size_t)b * nblk + blk] = r << 16;
  }
}

}  // namespace nvfp4
