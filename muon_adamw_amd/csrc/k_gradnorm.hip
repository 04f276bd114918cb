// Global gradient norm over every gradient of the hybrid step, ahead of both
// optimizers (dew.training.optim "build_optimizer": the global-norm clip reads
// every gradient together, before the parameter groups split them; kimi-k3
// "Optimization": clip the global norm when max_grad_norm > 0, observe it
// otherwise, and skip the whole hybrid update on an overflow).
//
// Pass 1: each block sums g^2 over one chunk of one tensor in fp64 (per-lane
// running sums, then the fixed-order wave and block reduction) and writes one
// partial; in fp32 a single square overflows above |g| ~ 1.8e19, where the
// norm, and the clip it asks for, are still finite. Pass 2: one block of 1024
// threads adds the partials in fp64: thread t the partials t, t + 1024, ... in
// order, then a fixed tree. The state it writes, read by every kernel of the
// step:
//   [0] ||g||, [1] clip factor min(1, max_norm / ||g||) (1 when max_norm <= 0
//   or the norm is 0), [2] 1 when ||g|| is not finite (the step is skipped),
//   else 0, [3] 0.
// HBM-bound: one read of every gradient (4 B or 2 B per element).
#include "kernels.hpp"

namespace ma {

namespace {

__global__ __launch_bounds__(256) void grad_sumsq_kernel(const GradNormLaunch L) {
  __shared__ double red[4];
  int ti = 0;
  while (ti + 1 < L.nt && L.block_start[ti + 1] <= static_cast<int>(blockIdx.x)) ++ti;
  const GradNormArg& T = L.t[ti];
  const int64_t c0 = (int64_t)(blockIdx.x - L.block_start[ti]) * kGradNormChunk;
  const int64_t c1 = c0 + kGradNormChunk < T.numel ? c0 + kGradNormChunk : T.numel;
  double s = 0.0;
  auto sq = [](float v) { return static_cast<double>(v) * static_cast<double>(v); };
  if (T.dt == DT_F32 && (reinterpret_cast<uintptr_t>(T.g) & 15) == 0 && c1 - c0 == kGradNormChunk) {
    typedef __attribute__((address_space(1))) const gf4 cgf4;
    cgf4* G4 = reinterpret_cast<cgf4*>(gmem(static_cast<const float*>(T.g) + c0));
    gf4 x[kGradNormChunk / 1024];
#pragma unroll
    for (int u = 0; u < kGradNormChunk / 1024; ++u) x[u] = __builtin_nontemporal_load(G4 + threadIdx.x + 256 * u);
#pragma unroll
    for (int u = 0; u < kGradNormChunk / 1024; ++u)
      s += (sq(x[u].x) + sq(x[u].y)) + (sq(x[u].z) + sq(x[u].w));
  } else {
    for (int64_t i = c0 + threadIdx.x; i < c1; i += 256) s += sq(load_elem(T.g, i, T.dt));
  }
  s = wave_sum(s);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) red[w] = s;
  __syncthreads();
  if (threadIdx.x == 0) gmem(L.partial)[L.partial_off + blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(1024) void grad_norm_finalize_kernel(const double* partial, int n, float max_norm,
                                                                  float* state) {
  __shared__ double red[1024];
  // thread t adds partials t, t + 1024, ... in that order; eight loads in
  // flight at a time (the order of the additions does not depend on them)
  double s = 0.0;
  for (int base = threadIdx.x; base < n; base += 8 * 1024) {
    double x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * 1024;
      x[u] = i < n ? gmem(partial)[i] : 0.0;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) s += x[u];
  }
  red[threadIdx.x] = s;
  __syncthreads();
  for (int h = 512; h >= 1; h >>= 1) {
    if (static_cast<int>(threadIdx.x) < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double norm = sqrt(red[0]);
    const bool finite = isfinite(norm);
    double f = 1.0;
    if (finite && max_norm > 0.f && norm > static_cast<double>(max_norm)) f = static_cast<double>(max_norm) / norm;
    gmem(state)[0] = static_cast<float>(norm);
    gmem(state)[1] = static_cast<float>(f);
    gmem(state)[2] = finite ? 0.f : 1.f;
    gmem(state)[3] = 0.f;
  }
}

}  // namespace

void launch_grad_sumsq(const GradNormLaunch& L, int nblocks, hipStream_t s) {
  if (nblocks <= 0) return;
  hipLaunchKernelGGL(grad_sumsq_kernel, dim3(nblocks), dim3(256), 0, s, L);
}

void launch_grad_norm_finalize(const double* partial, int n, float max_norm, float* state, hipStream_t s) {
  hipLaunchKernelGGL(grad_norm_finalize_kernel, dim3(1), dim3(1024), 0, s, partial, n, max_norm, state);
}

}  // namespace ma
