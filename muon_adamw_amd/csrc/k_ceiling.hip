// Measured ceiling of the bf16 matrix cores: an MFMA-only loop with no
// memory traffic, the reference beside the nominal peak that the
// Newton-Schulz GEMMs are reported against. Each wave keeps eight
// independent 32x32 accumulators and runs `iters` rounds of eight
// v_mfma_f32_32x32x16_bf16 (32768 flops each); one value per block goes to
// `sink` so the multiplies cannot be dropped.
#include "kernels.hpp"

namespace ma {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_ceiling_kernel(float* sink, int iters) {
  const int l = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    a[k] = static_cast<__bf16>(0.125f * ((l + k) & 7));
    b[k] = static_cast<__bf16>(0.0625f * ((l + 3 * k) & 15));
  }
  f32x16 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[k][v] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[k][v];
  if (threadIdx.x == 0) gmem(sink)[blockIdx.x] = s;
}

}  // namespace

void launch_mfma_ceiling(float* sink, int blocks, int iters, hipStream_t s) {
  hipLaunchKernelGGL(mfma_ceiling_kernel, dim3(blocks), dim3(256), 0, s, sink, iters);
}

}  // namespace ma
