// Check of the gfx950 float32 -> BF16 conversion the layer's kernels use
// (v_cvt_pk_bf16_f32, the compiler's float -> __bf16 conversion) against
// round-to-nearest-even written out on the bits: (u + 0x7FFF + bit 16 of u)
// >> 16, over every finite float32 pattern. Built into libnvfp4probe.so (not
// part of the layer); the GPU tests call it.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t rne_bits(uint32_t u) { return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16; }

// thread i takes pattern base + i (sign bit clear) and its negative
__global__ __launch_bounds__(256) void bf16_check_kernel(uint32_t base, uint32_t* __restrict__ result) {
  const uint32_t pa = base + blockIdx.x * blockDim.x + threadIdx.x;
  if ((pa & 0x7F800000u) == 0x7F800000u) return;  // infinities and NaNs: not inputs of the layer
  const uint32_t pb = pa | 0x80000000u;
  const float2_t v = {__uint_as_float(pa), __uint_as_float(pb)};
  const uint32_t hw = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
  const uint32_t sw = rne_bits(pa) | (rne_bits(pb) << 16);
  if (hw != sw && atomicAdd(&result[0], 1u) == 0u) result[1] = pa;
}

}  // namespace

// result: device uint32 [2], zeroed by the caller: the number of mismatching
// patterns and the first one found. Returns 0, or 1 on a failed launch.
extern "C" int nvfp4probe_bf16_check(uint32_t* result, void* stream) {
  if (!result) return 1;
  constexpr uint32_t kChunk = 1u << 28;  // patterns per launch
  for (uint32_t base = 0; base < 0x80000000u; base += kChunk) {
    hipLaunchKernelGGL(bf16_check_kernel, dim3(kChunk / 256), dim3(256), 0, (hipStream_t)stream, base, result);
    if (hipGetLastError() != hipSuccess) return 1;
  }
  return 0;
}
