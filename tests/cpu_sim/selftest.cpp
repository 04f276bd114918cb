// Kernels that check the CPU simulator itself (test infrastructure): each
// exercises one piece of device semantics the library's kernels rely on, or
// one mistake the simulator must expose. Built with runtime.cpp into
// libhipsim_selftest.so; tests/test_cpu_sim.py calls the st_* entry points.
#include <hip/hip_runtime.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

namespace {

// One 32 x 32 x 16 product: A row-major 32 x 16, B row-major 16 x 32 (bf16
// bits), D row-major 32 x 32, in the matrix-core operand layout.
__global__ void mfma_kernel(const uint16_t* A, const uint16_t* B, const float* C, float* D) {
  const int l = threadIdx.x;
  bf16x8 a, b;
  for (int j = 0; j < 8; ++j) {
    a[j] = __builtin_bit_cast(__bf16, A[(l % 32) * 16 + 8 * (l / 32) + j]);
    b[j] = __builtin_bit_cast(__bf16, B[(8 * (l / 32) + j) * 32 + l % 32]);
  }
  f32x16 c;
  for (int r = 0; r < 16; ++r) c[r] = C[(8 * (r / 4) + 4 * (l / 32) + r % 4) * 32 + l % 32];
  const f32x16 d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  for (int r = 0; r < 16; ++r) D[(8 * (r / 4) + 4 * (l / 32) + r % 4) * 32 + l % 32] = d[r];
}

// Transposing LDS read of a 4 x 16 block of 16-bit values stored row-major
// (as the library's k-major operands are read): lane i of each group of 16
// gets column i, rows 0..3.
__global__ void tr16_kernel(const short* src, short* out) {
  __shared__ __attribute__((aligned(16))) short tile[4][64];
  const int l = threadIdx.x;
  for (int k = 0; k < 4; ++k) tile[k][l] = src[k * 64 + l];
  __syncthreads();
  const int g = l / 16, i = l % 16;
  // lane j of the group names row j / 4, columns 4 (j % 4) .. + 3 of its block
  const short* p = &tile[i / 4][16 * g + 4 * (i % 4)];
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
  for (int e = 0; e < 4; ++e) out[l * 4 + e] = v[e];
}

// Cross-lane reductions and broadcasts.
__global__ void lanes_kernel(const float* x, float* out) {
  const int l = threadIdx.x;
  float v = x[blockIdx.x * 64 + l];
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  const float first = __builtin_amdgcn_readfirstlane(x[blockIdx.x * 64 + l] + 1.0f);
  const int q = __builtin_amdgcn_mov_dpp(static_cast<int>(l), 0x4E, 0xF, 0xF, false);
  out[blockIdx.x * 192 + l] = v;
  out[blockIdx.x * 192 + 64 + l] = first;
  out[blockIdx.x * 192 + 128 + l] = static_cast<float>(q);
}

// Wave 1 reads what wave 0 wrote to LDS, with or without the barrier
// between: without it the result depends on the schedule.
__global__ void handoff_kernel(int with_barrier, int base, int* out) {
  __shared__ int box[64];
  const int l = threadIdx.x;
  if (l < 64) box[l] = base + l;
  // a cross-lane operation: a point where the simulator switches lanes
  const int dummy = __builtin_amdgcn_readfirstlane(l);
  if (with_barrier) __syncthreads();
  if (l >= 64) out[l - 64] = box[l - 64] + 0 * dummy;
}

// A direct load into LDS, read back with or without waiting for it.
__global__ void dma_kernel(const uint16_t* src, int wait, uint16_t* out) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[64 * 8];
  const int l = threadIdx.x;
  for (int k = 0; k < 8; ++k) lds[l * 8 + k] = 0xFFFF;
  __syncthreads();
  const uint32_t base = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) char*)(reinterpret_cast<char*>(lds))));
  ::hipsim::dma16(src + 8 * l, __builtin_amdgcn_readfirstlane(base));
  if (wait) ::hipsim::wait_vm(0);
  __syncthreads();
  for (int k = 0; k < 8; ++k) out[l * 8 + k] = lds[l * 8 + k];
}

// A cross-lane operation under a lane-dependent branch on two sides.
__global__ void divergent_kernel(float* out) {
  const int l = threadIdx.x;
  float v;
  if (l & 1) v = __builtin_amdgcn_readfirstlane(1.0f);
  else v = __builtin_amdgcn_readfirstlane(2.0f);
  out[l] = v;
}

// Writes n + extra floats from `n` threads: an access past the buffer.
__global__ void overrun_kernel(float* out, int n, int extra) {
  const int l = threadIdx.x;
  if (l < n + extra) out[l] = 1.0f;
}

}  // namespace

extern "C" {
int st_mfma(const uint16_t* A, const uint16_t* B, const float* C, float* D) {
  hipLaunchKernelGGL(mfma_kernel, dim3(1), dim3(64), 0, nullptr, A, B, C, D);
  return hipGetLastError();
}
int st_tr16(const short* src, short* out) {
  hipLaunchKernelGGL(tr16_kernel, dim3(1), dim3(64), 0, nullptr, src, out);
  return hipGetLastError();
}
int st_lanes(const float* x, float* out, int blocks) {
  hipLaunchKernelGGL(lanes_kernel, dim3(blocks), dim3(64), 0, nullptr, x, out);
  return hipGetLastError();
}
int st_handoff(int with_barrier, int base, int* out) {
  hipLaunchKernelGGL(handoff_kernel, dim3(1), dim3(128), 0, nullptr, with_barrier, base, out);
  return hipGetLastError();
}
int st_dma(const uint16_t* src, int wait, uint16_t* out) {
  hipLaunchKernelGGL(dma_kernel, dim3(1), dim3(64), 0, nullptr, src, wait, out);
  return hipGetLastError();
}
int st_divergent(float* out) {
  hipLaunchKernelGGL(divergent_kernel, dim3(1), dim3(64), 0, nullptr, out);
  return hipGetLastError();
}
int st_overrun(float* out, int n, int extra) {
  hipLaunchKernelGGL(overrun_kernel, dim3(1), dim3(256), 0, nullptr, out, n, extra);
  return hipGetLastError();
}
}
