// Fused scale + decoupled weight decay + apply (speedtronic "v2 optimizers"
// page, "Muon update": W <- (1 - lr wd) W - lr max(1, rows/cols)^0.5 U), in the
// stored orientation, with the optional per-row / per-column factors of
// NorMuon and Muon+ and the two cautious forms:
//   weight-decay mask (flaxchat "Optimizer" page, "Muon Algorithm" step 4):
//     W <- W - lr s U - [U W >= 0] lr wd W
//   wrapper (speedtronic "Cautious updates"):
//     D = lr wd W + lr s U;  W <- (D G > 0) ? W - D : W
// HBM-bound: reads U (canonical, transposed back through LDS for a tall
// matrix) and W (and G for the wrapper), writes W, rounded to nearest even for
// bf16 parameters. One 64 x 64 stored tile per block.
#include "kernels.hpp"

namespace ma {

namespace {

template <typename XT>
__device__ __forceinline__ void load4(const XT* p, float* v);
template <>
__device__ __forceinline__ void load4<float>(const float* p, float* v) {
  const gf4 x = __builtin_nontemporal_load(gmem(reinterpret_cast<const gf4*>(p)));
  v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
}
template <>
__device__ __forceinline__ void load4<uint16_t>(const uint16_t* p, float* v) {
  const gu2 x = __builtin_nontemporal_load(gmem(reinterpret_cast<const gu2*>(p)));
  v[0] = __uint_as_float(x.x << 16); v[1] = __uint_as_float(x.x & 0xffff0000u);
  v[2] = __uint_as_float(x.y << 16); v[3] = __uint_as_float(x.y & 0xffff0000u);
}

// Four consecutive stored elements (the caller guarantees 16-byte alignment
// for fp32 and 8-byte alignment for bf16 via the descriptor's vec flag).
// The vector accesses of U, W and G are nontemporal: each is touched once.
__device__ __forceinline__ void load4v(const void* p, int64_t i, int dt, float* v) {
  if (dt == DT_BF16) {
    load4<uint16_t>(static_cast<const uint16_t*>(p) + i, v);
  } else {
    load4<float>(static_cast<const float*>(p) + i, v);
  }
}
__device__ __forceinline__ void store4v(void* p, int64_t i, int dt, const float* v) {
  if (dt == DT_BF16) {
    gu2 x;
    x.x = pack_bf16x2(v[0], v[1]);
    x.y = pack_bf16x2(v[2], v[3]);
    __builtin_nontemporal_store(x, gmem(reinterpret_cast<gu2*>(static_cast<uint16_t*>(p) + i)));
  } else {
    __builtin_nontemporal_store(gf4{v[0], v[1], v[2], v[3]}, gmem(reinterpret_cast<gf4*>(static_cast<float*>(p) + i)));
  }
}

template <typename XT>
__global__ __launch_bounds__(256) void apply_kernel(const MatDesc* __restrict__ mats, TileMap tm, int src,
                                                    int mode, int cautious, int use_rfac, int use_cfac) {
  __shared__ float us[kEw][kEw + 1];
  const int blk = blockIdx.x;
  const int e = find_entry(tm, blk);
  const MatDesc& d = mats[tm.perm[e]];
  if (step_skipped(d.clip)) return;   // the whole block: parameters untouched
  const int t = blk - tm.start[e];
  const int m = d.m, n = d.n;
  const int tiles_n = (n + kEw - 1) / kEw;
  const int s0 = (t / tiles_n) * kEw, c0 = (t % tiles_n) * kEw;   // stored origin
  const int tr = threadIdx.x >> 4, tc = (threadIdx.x & 15) * 4;
  const XT* U = static_cast<const XT*>(src ? d.x1 : d.x0);

  // A full, aligned stored tile (the common case) issues its parameter (and
  // gradient) loads first, so they are in flight together with the loads of
  // U; edge tiles take the element-wise path below.
  const bool full = d.vec && s0 + kEw <= m && c0 + kEw <= n;
  float wf[4][4], gf[4][4];
  if (full && mode != APPLY_COPY) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int64_t idx = (int64_t)(s0 + tr + 16 * p) * n + c0 + tc;
      load4v(d.param, idx, d.pdt, wf[p]);
      if (cautious == CAUT_WRAPPER) load4v(d.grad, idx, d.gdt, gf[p]);
    }
  }

  // canonical tile covering this stored tile; the padded canonical buffer is
  // at least as large as the stored extent rounded up to 64, so all reads are
  // in bounds.
  const int ci0 = d.tall ? c0 : s0, cj0 = d.tall ? s0 : c0;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int lr = tr + 16 * p;
    float v[4];
    load4<XT>(U + (int64_t)(ci0 + lr) * d.cp + cj0 + tc, v);
#pragma unroll
    for (int u = 0; u < 4; ++u) us[lr][tc + u] = v[u];
  }
  __syncthreads();

  if (full) {
    float cf[4] = {1.f, 1.f, 1.f, 1.f};
    if (use_cfac) {
      const gf4 c4 = *gmem(reinterpret_cast<const gf4*>(d.cfac + c0 + tc));
      cf[0] = c4.x; cf[1] = c4.y; cf[2] = c4.z; cf[3] = c4.w;
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int lr = tr + 16 * p;
      const int64_t idx = (int64_t)(s0 + lr) * n + c0 + tc;
      const float rf = use_rfac ? gmem(d.rfac)[s0 + lr] : 1.f;
      float uu[4], wn[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) uu[u] = (d.tall ? us[tc + u][lr] : us[lr][tc + u]) * rf * cf[u];
      if (mode == APPLY_COPY) {
#pragma unroll
        for (int u = 0; u < 4; ++u) wn[u] = uu[u];
      } else if (cautious == CAUT_NONE) {
#pragma unroll
        for (int u = 0; u < 4; ++u) wn[u] = d.decay * wf[p][u] - d.step * uu[u];
      } else if (cautious == CAUT_WD_MASK) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          wn[u] = wf[p][u] - d.step * uu[u];
          if (uu[u] * wf[p][u] >= 0.f) wn[u] -= d.lrwd * wf[p][u];
        }
      } else {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float delta = d.lrwd * wf[p][u] + d.step * uu[u];
          wn[u] = (delta * gf[p][u] > 0.f) ? wf[p][u] - delta : wf[p][u];
        }
      }
      store4v(d.param, idx, d.pdt, wn);
    }
    return;
  }

#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int lr = tr + 16 * p, si = s0 + lr;
    if (si >= m) continue;
    const float rf = use_rfac ? gmem(d.rfac)[si] : 1.f;
    const int sj0 = c0 + tc;
    if (sj0 >= n) continue;
    float uu[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uu[u] = d.tall ? us[tc + u][lr] : us[lr][tc + u];
      if (use_rfac) uu[u] *= rf;
    }
    const int64_t idx = (int64_t)si * n + sj0;
    if (d.vec && sj0 + 3 < n) {
      // four consecutive elements of the stored row: one 16-byte (fp32) or
      // 8-byte (bf16) access per operand
      if (use_cfac) {
        const gf4 cf = *gmem(reinterpret_cast<const gf4*>(d.cfac + sj0));
        uu[0] *= cf.x; uu[1] *= cf.y; uu[2] *= cf.z; uu[3] *= cf.w;
      }
      float w[4], wn[4];
      if (mode != APPLY_COPY) load4v(d.param, idx, d.pdt, w);
      if (mode == APPLY_COPY) {
#pragma unroll
        for (int u = 0; u < 4; ++u) wn[u] = uu[u];
      } else if (cautious == CAUT_NONE) {
#pragma unroll
        for (int u = 0; u < 4; ++u) wn[u] = d.decay * w[u] - d.step * uu[u];
      } else if (cautious == CAUT_WD_MASK) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          wn[u] = w[u] - d.step * uu[u];
          if (uu[u] * w[u] >= 0.f) wn[u] -= d.lrwd * w[u];
        }
      } else {
        float g[4];
        load4v(d.grad, idx, d.gdt, g);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float delta = d.lrwd * w[u] + d.step * uu[u];
          wn[u] = (delta * g[u] > 0.f) ? w[u] - delta : w[u];
        }
      }
      store4v(d.param, idx, d.pdt, wn);
      continue;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int sj = sj0 + u;
      if (sj >= n) continue;
      float uv = uu[u];
      if (use_cfac) uv *= gmem(d.cfac)[sj];
      const int64_t ix = idx + u;
      if (mode == APPLY_COPY) {
        store_elem(d.param, ix, d.pdt, uv);
        continue;
      }
      const float w = load_elem(d.param, ix, d.pdt);
      float wn;
      if (cautious == CAUT_NONE) {
        wn = d.decay * w - d.step * uv;
      } else if (cautious == CAUT_WD_MASK) {
        wn = w - d.step * uv;
        if (uv * w >= 0.f) wn -= d.lrwd * w;
      } else {
        const float g = load_elem(d.grad, ix, d.gdt);
        const float delta = d.lrwd * w + d.step * uv;
        wn = (delta * g > 0.f) ? w - delta : w;
      }
      store_elem(d.param, ix, d.pdt, wn);
    }
  }
}

}  // namespace

void launch_apply(const MatDesc* mats, TileMap tm, int ns_dt, int src, int mode, int cautious, int use_rfac,
                  int use_cfac, hipStream_t s) {
  if (tm.total == 0) return;
  if (ns_dt == DT_BF16)
    hipLaunchKernelGGL(apply_kernel<uint16_t>, dim3(tm.grid), dim3(256), 0, s, mats, tm, src, mode, cautious,
                       use_rfac, use_cfac);
  else
    hipLaunchKernelGGL(apply_kernel<float>, dim3(tm.grid), dim3(256), 0, s, mats, tm, src, mode, cautious,
                       use_rfac, use_cfac);
}

}  // namespace ma
