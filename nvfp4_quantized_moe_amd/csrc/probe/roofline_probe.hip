// Achievable-peak probes for the benchmark's roofline figures (not part of the
// layer): a streaming read of a large buffer (HBM) and a loop of independent
// fp16 MFMAs with no memory traffic (matrix cores). Built into
// libnvfp4probe.so, apart from the layer's library.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Every thread reads 16-byte vectors grid-stride with non-temporal loads,
// eight in flight, and folds them with XOR; one word per workgroup is stored
// so that nothing is dropped. n16 = number of 16-byte vectors. (Of the shapes
// tried on MI355X -- 4 to 32 workgroups per CU, 4 to 16 loads in flight,
// plain or non-temporal, grid-stride or one contiguous chunk per workgroup --
// this one reads fastest.)
__global__ __launch_bounds__(256) void read_kernel(const uint4* __restrict__ p, int64_t n16,
                                                   uint32_t* __restrict__ out) {
  const u32x4_t* q = reinterpret_cast<const u32x4_t*>(p);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 7 * stride < n16; i += 8 * stride) {
    u32x4_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(q + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4_t v = __builtin_nontemporal_load(q + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  __shared__ uint32_t red[4];
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

// Each wave runs `iters` rounds of four independent v_mfma_f32_32x32x16_f16 on
// register operands (32768 FLOP each); lane 0 of every wave stores a sum of its
// accumulators.
__global__ __launch_bounds__(256) void mfma_kernel(int iters, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  half8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(0.001f * (float)((lane + i) & 7));
    b[i] = (_Float16)(0.002f * (float)((lane * 3 + i) & 7));
  }
  float16_t acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[j][v] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[j][v];
  if (lane == 0) out[blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6)] = s;
}

}  // namespace

// bytes: a multiple of 16; out: uint32 [grid]. Returns 0, or 1 on a bad argument
// or a failed launch.
extern "C" int nvfp4probe_read(const void* p, int64_t bytes, uint32_t* out, int grid, void* stream) {
  if (!p || !out || bytes <= 0 || bytes % 16 != 0 || grid < 1) return 1;
  hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, reinterpret_cast<const uint4*>(p),
                     bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}

// out: float [grid * 4]; FLOP = grid * 4 waves * iters * 4 * 32768.
extern "C" int nvfp4probe_mfma(int iters, float* out, int grid, void* stream) {
  if (!out || iters < 1 || grid < 1) return 1;
  hipLaunchKernelGGL(mfma_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, iters, out);
  return hipGetLastError() == hipSuccess ? 0 : 1;
}
