// Multi-tensor AdamW (dew.training.optim page: optax.adamw through
// OPTIMIZER_MAP; speedtronic "v2 optimizers" page: torch AdamW):
//   m <- b1 m + (1-b1) g;  v <- b2 v + (1-b2) g^2
//   p <- p - lr ( (m / (1-b1^t)) / (sqrt(v / (1-b2^t)) + eps) + wd p )
// Pure HBM streaming: 28 B per fp32 element (read p, g, m, v; write p, m, v).
// Up to 32 tensors per launch travel in the kernel arguments; each block owns
// one contiguous chunk of one tensor. A full chunk of fp32 tensors (the common
// case) is exactly two 16-byte slots per stream per thread: all eight loads
// are issued before any use, and every access is nontemporal, since nothing
// here is read again within the step (measured on MI355X: 74% of HBM peak
// against 64% with cached accesses; the stores are what matters).
// IEEE sqrt and division (no approximate reciprocal square root).
#include "kernels.hpp"

namespace ma {

namespace {

__device__ __forceinline__ void adam_elem(float& p, float g, float& m, float& v, const AdamLaunch& L,
                                          float lr, float wd) {
  m = L.b1 * m + L.omb1 * g;
  v = L.b2 * v + L.omb2 * (g * g);
  const float denom = sqrtf(v) * L.inv_sqrt_bc2 + L.eps;
  p = p - lr * ((m * L.inv_bc1) / denom + wd * p);
}

__global__ __launch_bounds__(256) void adamw_kernel(const AdamLaunch L) {
  int ti = 0;
  while (ti + 1 < L.nt && L.block_start[ti + 1] <= static_cast<int>(blockIdx.x)) ++ti;
  const AdamTensorArg& T = L.t[ti];
  const int64_t c0 = (int64_t)(blockIdx.x - L.block_start[ti]) * kAdamChunk;
  const int64_t c1 = c0 + kAdamChunk < T.numel ? c0 + kAdamChunk : T.numel;
  const float lr = T.lr, wd = T.wd;
  const bool vec = T.pdt == DT_F32 && T.gdt == DT_F32 &&
                   ((reinterpret_cast<uintptr_t>(T.p) | reinterpret_cast<uintptr_t>(T.g) |
                     reinterpret_cast<uintptr_t>(T.m) | reinterpret_cast<uintptr_t>(T.v)) & 15) == 0;
  if (vec && c1 - c0 == kAdamChunk) {
    static_assert(kAdamChunk == 2 * 256 * 4, "a full chunk is two float4 slots per thread");
    typedef __attribute__((address_space(1))) gf4 ggf4;
    ggf4* P4 = reinterpret_cast<ggf4*>(gmem(static_cast<float*>(T.p) + c0));
    const ggf4* G4 = reinterpret_cast<const ggf4*>(gmem(static_cast<const float*>(T.g) + c0));
    ggf4* M4 = reinterpret_cast<ggf4*>(gmem(T.m + c0));
    ggf4* V4 = reinterpret_cast<ggf4*>(gmem(T.v + c0));
    gf4 p[2], g[2], m[2], v[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = threadIdx.x + 256 * u;
      p[u] = __builtin_nontemporal_load(P4 + i);
      g[u] = __builtin_nontemporal_load(G4 + i);
      m[u] = __builtin_nontemporal_load(M4 + i);
      v[u] = __builtin_nontemporal_load(V4 + i);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i = threadIdx.x + 256 * u;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        float pk = p[u][k], mk = m[u][k], vk = v[u][k];
        adam_elem(pk, g[u][k], mk, vk, L, lr, wd);
        p[u][k] = pk; m[u][k] = mk; v[u][k] = vk;
      }
      __builtin_nontemporal_store(p[u], P4 + i);
      __builtin_nontemporal_store(m[u], M4 + i);
      __builtin_nontemporal_store(v[u], V4 + i);
    }
  } else if (vec) {
    float* P = static_cast<float*>(T.p);
    const float* G = static_cast<const float*>(T.g);
    const int64_t nvec_end = c0 + ((c1 - c0) & ~int64_t(3));
    for (int64_t i = c0 + threadIdx.x * 4; i < nvec_end; i += 256 * 4) {
      float4 p = *reinterpret_cast<const float4*>(P + i);
      const float4 g = *reinterpret_cast<const float4*>(G + i);
      float4 m = *reinterpret_cast<const float4*>(T.m + i);
      float4 v = *reinterpret_cast<const float4*>(T.v + i);
      adam_elem(p.x, g.x, m.x, v.x, L, lr, wd);
      adam_elem(p.y, g.y, m.y, v.y, L, lr, wd);
      adam_elem(p.z, g.z, m.z, v.z, L, lr, wd);
      adam_elem(p.w, g.w, m.w, v.w, L, lr, wd);
      *reinterpret_cast<float4*>(P + i) = p;
      *reinterpret_cast<float4*>(T.m + i) = m;
      *reinterpret_cast<float4*>(T.v + i) = v;
    }
    for (int64_t i = nvec_end + threadIdx.x; i < c1; i += 256) {
      float p = P[i], m = T.m[i], v = T.v[i];
      adam_elem(p, G[i], m, v, L, lr, wd);
      P[i] = p; T.m[i] = m; T.v[i] = v;
    }
  } else {
    for (int64_t i = c0 + threadIdx.x; i < c1; i += 256) {
      float p = load_elem(T.p, i, T.pdt), m = T.m[i], v = T.v[i];
      adam_elem(p, load_elem(T.g, i, T.gdt), m, v, L, lr, wd);
      store_elem(T.p, i, T.pdt, p);
      T.m[i] = m;
      T.v[i] = v;
    }
  }
}

}  // namespace

void launch_adamw(const AdamLaunch& L, int nblocks, hipStream_t s) {
  if (nblocks <= 0) return;
  hipLaunchKernelGGL(adamw_kernel, dim3(nblocks), dim3(256), 0, s, L);
}

}  // namespace ma
