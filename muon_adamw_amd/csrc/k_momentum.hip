// Fused momentum pass: B <- beta B + (1-beta) G; Q <- lerp(G, B, beta)
// (speedtronic "v2 optimizers" page, "Muon update"; flaxchat "Optimizer" page,
// "Muon Algorithm" step 1), written once in the canonical orientation
// (r = min(m, n) rows) for Newton-Schulz, with the per-tile sum of squares of Q
// for the Frobenius normalisation (speedtronic "Newton-Schulz").
//
// HBM-bound: reads G and B, writes B and Q (4+4+4+2 = 14 B per fp32-grad
// element with a bf16 Q). One 64x64 canonical tile per block; a tall matrix is
// transposed through LDS. The reduction always walks the canonical tile in the
// same thread order, so a tall matrix and its transposed wide twin produce the
// same bits. Squares and partials are fp64, so no finite Q overflows them.
#include "kernels.hpp"

namespace ma {

namespace {

template <typename XT>
__device__ __forceinline__ void store4(XT* dst, const float* v);

template <>
__device__ __forceinline__ void store4<float>(float* dst, const float* v) {
  *gmem(reinterpret_cast<gf4*>(dst)) = gf4{v[0], v[1], v[2], v[3]};
}
template <>
__device__ __forceinline__ void store4<uint16_t>(uint16_t* dst, const float* v) {
  gu2 p;
  p.x = pack_bf16x2(v[0], v[1]);
  p.y = pack_bf16x2(v[2], v[3]);
  *gmem(reinterpret_cast<gu2*>(dst)) = p;
}

__device__ __forceinline__ double block_sum_256(double v, double* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) red[w] = v;
  __syncthreads();
  double t = ((red[0] + red[1]) + red[2]) + red[3];
  __syncthreads();
  return t;
}

template <typename XT>
__global__ __launch_bounds__(256) void momentum_kernel(const MatDesc* __restrict__ mats, TileMap tm,
                                                       float beta, float omb, int nesterov) {
  __shared__ float qs[kEw][kEw + 1];
  __shared__ double red[4];
  const int blk = blockIdx.x;
  const int e = find_entry(tm, blk);
  const MatDesc& d = mats[tm.perm[e]];
  if (step_skipped(d.clip)) return;   // the whole block: momentum untouched
  const float cf = clip_factor(d.clip);   // G is read scaled by the global-norm clip
  const int t = blk - tm.start[e];
  const int tiles_c = d.cp / kEw;
  const int i0 = (t / tiles_c) * kEw, j0 = (t % tiles_c) * kEw;   // canonical origin
  const int sr0 = d.tall ? j0 : i0, sc0 = d.tall ? i0 : j0;       // stored origin
  const int tr = threadIdx.x >> 4, tc = (threadIdx.x & 15) * 4;
  const int m = d.m, n = d.n;

  // Phase 1: stored tile, coalesced along stored rows. A full, aligned tile
  // (the common case) issues all of a thread's loads before any use, so
  // they are in flight together; edge tiles take the element-wise path.
  // G and B are touched once per step: nontemporal accesses. Q stays
  // cached, since Newton-Schulz reads it next.
  const bool full = d.vec && sr0 + kEw <= m && sc0 + kEw <= n;
  if (full) {
    float g[4][4];
    gf4 bm[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int64_t idx = (int64_t)(sr0 + tr + 16 * p) * n + sc0 + tc;
      if (d.gdt == DT_BF16) {
        const gu2 raw = __builtin_nontemporal_load(gmem(reinterpret_cast<const gu2*>(static_cast<const uint16_t*>(d.grad) + idx)));
        g[p][0] = cf * __uint_as_float(raw.x << 16); g[p][1] = cf * __uint_as_float(raw.x & 0xffff0000u);
        g[p][2] = cf * __uint_as_float(raw.y << 16); g[p][3] = cf * __uint_as_float(raw.y & 0xffff0000u);
      } else {
        const gf4 raw = __builtin_nontemporal_load(gmem(reinterpret_cast<const gf4*>(static_cast<const float*>(d.grad) + idx)));
        g[p][0] = cf * raw.x; g[p][1] = cf * raw.y; g[p][2] = cf * raw.z; g[p][3] = cf * raw.w;
      }
      if (d.mom) bm[p] = __builtin_nontemporal_load(gmem(reinterpret_cast<const gf4*>(d.mom + idx)));
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int lr = tr + 16 * p;
      const int64_t idx = (int64_t)(sr0 + lr) * n + sc0 + tc;
      float q[4];
      if (d.mom) {
        float b[4] = {bm[p].x, bm[p].y, bm[p].z, bm[p].w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          b[u] = beta * b[u] + omb * g[p][u];
          q[u] = nesterov ? g[p][u] + beta * (b[u] - g[p][u]) : b[u];
        }
        __builtin_nontemporal_store(gf4{b[0], b[1], b[2], b[3]}, gmem(reinterpret_cast<gf4*>(d.mom + idx)));
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) q[u] = g[p][u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) qs[lr][tc + u] = q[u];
    }
  } else {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int lr = tr + 16 * p, sr = sr0 + lr, sc = sc0 + tc;
      float q[4] = {0.f, 0.f, 0.f, 0.f};
      if (sr < m) {
        const int64_t idx = (int64_t)sr * n + sc;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (sc + u < n) {
            const float gu = cf * load_elem(d.grad, idx + u, d.gdt);
            if (d.mom) {
              float b = gmem(d.mom)[idx + u];
              b = beta * b + omb * gu;
              gmem(d.mom)[idx + u] = b;
              q[u] = nesterov ? gu + beta * (b - gu) : b;
            } else {
              q[u] = gu;
            }
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) qs[lr][tc + u] = q[u];
    }
  }
  __syncthreads();

  // Phase 2: canonical tile, same thread order for both orientations. The
  // squares are summed in fp64: an fp32 square overflows above |Q| ~ 1.8e19,
  // where the norm itself is still finite.
  XT* X = static_cast<XT*>(d.x0);
  double ss = 0.0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int ci = tr + 16 * p;
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      v[u] = d.tall ? qs[tc + u][ci] : qs[ci][tc + u];
      ss += static_cast<double>(v[u]) * static_cast<double>(v[u]);
    }
    store4<XT>(X + (int64_t)(i0 + ci) * d.cp + j0 + tc, v);
  }
  const double tot = block_sum_256(ss, red);
  if (threadIdx.x == 0) gmem(d.part)[t] = tot;
}

// Above this Frobenius norm of Q the first Gram's fp32 sums, which are
// bounded by ||Q||_F^2 and computed before sigma^2 is applied, could reach the
// fp32 range (2^128); such an X0 is scaled down to a norm near 2^kGuardTarget.
constexpr int kGuardExp = 60;
constexpr int kGuardTarget = 30;

template <typename XT>
__global__ __launch_bounds__(256) void norm_finalize_kernel(const MatDesc* __restrict__ mats, TileMap tm,
                                                            float eps, float scale) {
  __shared__ double red[4];
  const MatDesc& d = mats[tm.perm[blockIdx.x]];
  double s = 0.0;
  for (int i = threadIdx.x; i < d.ntile_ew; i += 256) s += gmem(d.part)[i];
  const double tot = block_sum_256(s, red);
  const double norm = sqrt(tot);
  // X = Q / (norm * scale + eps) = (2^-k Q) * 2^k / (norm * scale + eps):
  // with k > 0 the stored X0 is scaled by the power of two 2^-k (exact) and
  // sigma carries 2^k
  int k = 0;
  if (isfinite(norm) && norm >= ldexp(1.0, kGuardExp)) k = ilogb(norm) - kGuardTarget;
  const double sigma = 1.0 / (norm * static_cast<double>(scale) + static_cast<double>(eps));
  if (threadIdx.x == 0) {
    gmem(d.stat)[0] = static_cast<float>(ldexp(sigma, k));
    gmem(d.stat)[1] = ldexpf(1.0f, -k);
  }
  if (k == 0 || step_skipped(d.clip)) return;
  const float f = ldexpf(1.0f, -k);
  XT* X = static_cast<XT*>(d.x0);
  const int64_t n = static_cast<int64_t>(d.rp) * d.cp;
  for (int64_t i = threadIdx.x; i < n; i += 256) {
    if constexpr (sizeof(XT) == 2)
      gmem(X)[i] = f32_to_bf16(bf16_to_f32(gmem(X)[i]) * f);
    else
      gmem(X)[i] = gmem(X)[i] * f;
  }
}

}  // namespace

void launch_momentum(const MatDesc* mats, TileMap tm, int ns_dt, float beta, float omb, int nesterov,
                     hipStream_t s) {
  if (tm.total == 0) return;
  if (ns_dt == DT_BF16)
    hipLaunchKernelGGL(momentum_kernel<uint16_t>, dim3(tm.grid), dim3(256), 0, s, mats, tm, beta, omb, nesterov);
  else
    hipLaunchKernelGGL(momentum_kernel<float>, dim3(tm.grid), dim3(256), 0, s, mats, tm, beta, omb, nesterov);
}

void launch_norm_finalize(const MatDesc* mats, TileMap tm, int ns_dt, float eps, float scale, hipStream_t s) {
  if (tm.total == 0) return;
  if (ns_dt == DT_BF16)
    hipLaunchKernelGGL(norm_finalize_kernel<uint16_t>, dim3(tm.grid), dim3(256), 0, s, mats, tm, eps, scale);
  else
    hipLaunchKernelGGL(norm_finalize_kernel<float>, dim3(tm.grid), dim3(256), 0, s, mats, tm, eps, scale);
}

}  // namespace ma
