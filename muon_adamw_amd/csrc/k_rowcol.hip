// Row / column statistics of the orthogonalised update for NorMuon (flaxchat
// "Optimizer" page, "Muon Algorithm" step 3) and Muon+ row_col (speedtronic
// "v2 optimizers" page, "Muon+").
//
// The final Newton-Schulz output U sits in the workspace in canonical
// orientation (r x c, r <= c). A stored row is a canonical row when the
// parameter is wide and a canonical column when it is tall, so both reduction
// directions exist; each is a deterministic fixed-order sum. HBM-bound: one
// read of U per pass (2 B/element for bf16).
#include "kernels.hpp"

namespace ma {

namespace {

template <typename XT>
__device__ __forceinline__ float ld_x(const XT* p, int64_t i);
template <>
__device__ __forceinline__ float ld_x<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld_x<uint16_t>(const uint16_t* p, int64_t i) { return bf16_to_f32(p[i]); }

// One wave per canonical row, 4 rows per block. A lane reads 16 bytes at a
// time (8 bf16 or 4 fp32 elements) and keeps four such loads in flight: a
// wave moves 4 KB per round instead of 128 B per load. The whole vectors
// cover the row's first c - c mod V elements; a scalar tail takes the rest.
// Each lane adds its elements in a fixed order, then the fixed butterfly.
// weighted: each column j is scaled by rfac[j]^2 (tall matrices: canonical
// column j is stored row j).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4_t g_u32x4_t;

__device__ __forceinline__ void unpack_vec(const u32x4_t& w, float* f, float*) {   // 4 fp32
  f[0] = __uint_as_float(w.x); f[1] = __uint_as_float(w.y); f[2] = __uint_as_float(w.z); f[3] = __uint_as_float(w.w);
}
__device__ __forceinline__ void unpack_vec(const u32x4_t& w, float* f, uint16_t*) {   // 8 bf16
  f[0] = __uint_as_float(w.x << 16); f[1] = __uint_as_float(w.x & 0xffff0000u);
  f[2] = __uint_as_float(w.y << 16); f[3] = __uint_as_float(w.y & 0xffff0000u);
  f[4] = __uint_as_float(w.z << 16); f[5] = __uint_as_float(w.z & 0xffff0000u);
  f[6] = __uint_as_float(w.w << 16); f[7] = __uint_as_float(w.w & 0xffff0000u);
}

template <typename XT>
__global__ __launch_bounds__(256) void canon_rowsum_kernel(const MatDesc* __restrict__ mats, TileMap tm,
                                                           int src, int weighted) {
  constexpr int V = 16 / static_cast<int>(sizeof(XT));   // elements per 16-byte load
  constexpr int R = 4;                                   // loads in flight per lane
  const int blk = blockIdx.x;
  const int e = find_entry(tm, blk);
  const MatDesc& d = mats[tm.perm[e]];
  const int row = (blk - tm.start[e]) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= d.r) return;
  const XT* U = static_cast<const XT*>(src ? d.x1 : d.x0) + (int64_t)row * d.cp;   // 16-byte aligned row
  const int nv = d.c / V;
  float s = 0.f;
  for (int v0 = lane; v0 < nv; v0 += R * 64) {
    u32x4_t raw[R];
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int v = v0 + 64 * u;
      raw[u] = v < nv ? *reinterpret_cast<g_u32x4_t*>(gmem(U) + (int64_t)v * V) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < R; ++u) {
      const int v = v0 + 64 * u;
      float x[V];
      unpack_vec(raw[u], x, static_cast<XT*>(nullptr));
      if (weighted) {
        if (v < nv) {
#pragma unroll
          for (int q = 0; q < V; ++q) {
            const float f = gmem(d.rfac)[v * V + q];
            s += (x[q] * x[q]) * (f * f);
          }
        }
      } else {
#pragma unroll
        for (int q = 0; q < V; ++q) s += x[q] * x[q];
      }
    }
  }
  for (int j = nv * V + lane; j < d.c; j += 64) {
    const float u = ld_x<XT>(U, j);
    const float f = weighted ? gmem(d.rfac)[j] : 1.f;
    s += (u * u) * (f * f);
  }
  s = wave_sum(s);
  if (lane == 0) gmem(d.csum_r)[row] = s;
}

// 64 canonical columns per block: 16 row groups x 16 column quads; partials
// combined in LDS in row-group order. weighted: row i scaled by rfac[i]^2.
template <typename XT>
__global__ __launch_bounds__(256) void canon_colsum_kernel(const MatDesc* __restrict__ mats, TileMap tm,
                                                           int src, int weighted) {
  __shared__ float part[16][65];
  const int blk = blockIdx.x;
  const int e = find_entry(tm, blk);
  const MatDesc& d = mats[tm.perm[e]];
  const int c0 = (blk - tm.start[e]) * 64;
  const int g = threadIdx.x >> 4, cq = (threadIdx.x & 15) * 4;
  const XT* U = static_cast<const XT*>(src ? d.x1 : d.x0);
  float s[4] = {0.f, 0.f, 0.f, 0.f};
  for (int i = g; i < d.r; i += 16) {
    const float w = weighted ? gmem(d.rfac)[i] * gmem(d.rfac)[i] : 1.f;
    const int64_t base = (int64_t)i * d.cp + c0 + cq;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float x = ld_x<XT>(U, base + u);
      s[u] += (x * x) * w;
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) part[g][cq + u] = s[u];
  __syncthreads();
  if (threadIdx.x < 64) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k) t += part[k][threadIdx.x];
    const int col = c0 + threadIdx.x;
    if (col < d.c) gmem(d.csum_c)[col] = t;
  }
}

__device__ __forceinline__ float block_sum_256(float v, float* red) {
  v = wave_sum(v);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = ((red[0] + red[1]) + red[2]) + red[3];
  __syncthreads();
  return t;
}

// NorMuon, one block per matrix: rho_i = (stored row sum)/n;
// V_i <- V_i + (1 - beta2)(rho_i - V_i); d_i = max(V_i, 1e-30)^-1/2;
// kappa = ||U||_F / max(||diag(d) U||_F, 1e-30); rfac_i = d_i kappa.
__global__ __launch_bounds__(256) void finalize_normuon_kernel(const MatDesc* __restrict__ mats, TileMap tm,
                                                               float omb2) {
  __shared__ float red[4];
  const MatDesc& d = mats[tm.perm[blockIdx.x]];
  if (step_skipped(d.clip)) return;   // V untouched
  const float* rs = d.tall ? d.csum_c : d.csum_r;
  const float inv_n = 1.0f / static_cast<float>(d.n);
  float tot = 0.f, toth = 0.f;
  for (int i = threadIdx.x; i < d.m; i += 256) {
    const float s = rs[i];
    float v = gmem(d.row_v)[i];
    v = v + omb2 * (s * inv_n - v);
    gmem(d.row_v)[i] = v;
    const float di = 1.0f / sqrtf(fmaxf(v, 1e-30f));
    gmem(d.rfac)[i] = di;
    tot += s;
    toth += s * (di * di);
  }
  tot = block_sum_256(tot, red);
  toth = block_sum_256(toth, red);
  const float kappa = sqrtf(tot) / fmaxf(sqrtf(toth), 1e-30f);
  __syncthreads();
  for (int i = threadIdx.x; i < d.m; i += 256) gmem(d.rfac)[i] *= kappa;
}

// Muon+: stage 1 rfac_i = 1/sqrt(stored row sum + eps); stage 2
// cfac_j = 1/sqrt(weighted stored column sum + eps).
__global__ __launch_bounds__(256) void finalize_muon_plus_kernel(const MatDesc* __restrict__ mats, TileMap tm,
                                                                 int stage, float eps) {
  const MatDesc& d = mats[tm.perm[blockIdx.x]];
  if (stage == 1) {
    const float* rs = d.tall ? d.csum_c : d.csum_r;
    for (int i = threadIdx.x; i < d.m; i += 256) gmem(d.rfac)[i] = 1.0f / sqrtf(rs[i] + eps);
  } else {
    const float* cs = d.tall ? d.csum_r : d.csum_c;
    for (int j = threadIdx.x; j < d.n; j += 256) gmem(d.cfac)[j] = 1.0f / sqrtf(cs[j] + eps);
  }
}

}  // namespace

void launch_canon_rowsum(const MatDesc* mats, TileMap tm, int ns_dt, int src, int weighted, hipStream_t s) {
  if (tm.total == 0) return;
  if (ns_dt == DT_BF16)
    hipLaunchKernelGGL(canon_rowsum_kernel<uint16_t>, dim3(tm.grid), dim3(256), 0, s, mats, tm, src, weighted);
  else
    hipLaunchKernelGGL(canon_rowsum_kernel<float>, dim3(tm.grid), dim3(256), 0, s, mats, tm, src, weighted);
}

void launch_canon_colsum(const MatDesc* mats, TileMap tm, int ns_dt, int src, int weighted, hipStream_t s) {
  if (tm.total == 0) return;
  if (ns_dt == DT_BF16)
    hipLaunchKernelGGL(canon_colsum_kernel<uint16_t>, dim3(tm.grid), dim3(256), 0, s, mats, tm, src, weighted);
  else
    hipLaunchKernelGGL(canon_colsum_kernel<float>, dim3(tm.grid), dim3(256), 0, s, mats, tm, src, weighted);
}

void launch_finalize_normuon(const MatDesc* mats, TileMap tm, float one_minus_beta2, hipStream_t s) {
  if (tm.total == 0) return;
  hipLaunchKernelGGL(finalize_normuon_kernel, dim3(tm.grid), dim3(256), 0, s, mats, tm, one_minus_beta2);
}

void launch_finalize_muon_plus(const MatDesc* mats, TileMap tm, int stage, float eps, hipStream_t s) {
  if (tm.total == 0) return;
  hipLaunchKernelGGL(finalize_muon_plus_kernel, dim3(tm.grid), dim3(256), 0, s, mats, tm, stage, eps);
}

}  // namespace ma
