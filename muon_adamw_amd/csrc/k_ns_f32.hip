// Newton-Schulz GEMMs in fp32 (speedtronic "v2 optimizers" page,
// "Newton-Schulz", in full single precision), batched over every matrix.
//
// Same three products as the bf16 matrix-core path (Gram with mirrored lower
// triangle, b A + c A A^T, s1 (a X + B X)), on the vector ALUs: 64 x 64 tiles,
// 256 threads each owning a 4 x 4 block, K in steps of 16 through LDS. This
// path serves small matrices (latency-bound) and fp32-exact checks; the
// large-matrix path is the bf16 one.
#include "kernels.hpp"

namespace ma {

namespace {

constexpr int T = 64;
constexpr int TK = 16;
constexpr int SP = T + 4;

enum { OP_GRAM = 0, OP_SQUARE = 1, OP_APPLY = 2 };

struct NsArgs {
  const MatDesc* mats;
  TileMap tm;
  int src;
  int first;
  float a, b, c;
};

__device__ __forceinline__ void tri_decode(int k, int& ti, int& tj) {
  int i = static_cast<int>((sqrtf(8.0f * k + 1.0f) - 1.0f) * 0.5f);
  while ((i + 1) * (i + 2) / 2 <= k) ++i;
  while (i * (i + 1) / 2 > k) --i;
  ti = i;
  tj = k - i * (i + 1) / 2;
}

template <int OP>
__global__ __launch_bounds__(256) void ns_f32_kernel(NsArgs args) {
  __shared__ __attribute__((aligned(16))) float As[TK][SP];
  __shared__ __attribute__((aligned(16))) float Bs[TK][SP];

  const int blk = blockIdx.x;
  const int e = find_entry(args.tm, blk);
  const MatDesc& d = args.mats[args.tm.perm[e]];
  const int t = blk - args.tm.start[e];
  int ti, tj;
  if (OP == OP_APPLY) {
    const int ntc = d.cp / T;
    ti = t / ntc;
    tj = t % ntc;
  } else {
    tri_decode(t, ti, tj);
  }
  const float* Xin = static_cast<const float*>(args.src ? d.x1 : d.x0);
  const int rp = d.rp, cp = d.cp;
  const float* Aop;
  const float* Bop;
  int lda, ldb, K;
  if (OP == OP_GRAM) {
    Aop = Xin + (int64_t)ti * T * cp; Bop = Xin + (int64_t)tj * T * cp; lda = ldb = cp; K = cp;
  } else if (OP == OP_SQUARE) {
    const float* A = static_cast<const float*>(d.a);
    Aop = A + (int64_t)ti * T * rp; Bop = A + (int64_t)tj * T * rp; lda = ldb = rp; K = rp;
  } else {
    const float* B = static_cast<const float*>(d.b);
    Aop = B + (int64_t)ti * T * rp; lda = rp;
    Bop = Xin + tj * T; ldb = cp; K = rp;
  }

  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

  const int lrow = threadIdx.x >> 2, lk = (threadIdx.x & 3) * 4;  // NT loads: 64 rows x 16 k
  const int nk = threadIdx.x >> 4, nc = (threadIdx.x & 15) * 4;   // NN loads: 16 k x 64 cols
  for (int k0 = 0; k0 < K; k0 += TK) {
    const gf4 va = *gmem(reinterpret_cast<const gf4*>(Aop + (int64_t)lrow * lda + k0 + lk));
    As[lk + 0][lrow] = va.x; As[lk + 1][lrow] = va.y; As[lk + 2][lrow] = va.z; As[lk + 3][lrow] = va.w;
    if (OP == OP_APPLY) {
      const gf4 vb = *gmem(reinterpret_cast<const gf4*>(Bop + (int64_t)(k0 + nk) * ldb + nc));
      *reinterpret_cast<gf4*>(&Bs[nk][nc]) = vb;
    } else {
      const gf4 vb = *gmem(reinterpret_cast<const gf4*>(Bop + (int64_t)lrow * ldb + k0 + lk));
      Bs[lk + 0][lrow] = vb.x; Bs[lk + 1][lrow] = vb.y; Bs[lk + 2][lrow] = vb.z; Bs[lk + 3][lrow] = vb.w;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      const float4 a4 = *reinterpret_cast<const float4*>(&As[kk][ty * 4]);
      const float4 b4 = *reinterpret_cast<const float4*>(&Bs[kk][tx * 4]);
      const float av[4] = {a4.x, a4.y, a4.z, a4.w};
      const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }

  float alpha = 1.f;
  if (args.first) {
    const float sg = gmem(d.stat)[0];
    alpha = (OP == OP_GRAM) ? sg * sg : (OP == OP_APPLY ? sg : 1.f);
  }
  float* out;
  int ldo;
  const float* extra = nullptr;
  if (OP == OP_GRAM) { out = static_cast<float*>(d.a); ldo = rp; }
  else if (OP == OP_SQUARE) { out = static_cast<float*>(d.b); ldo = rp; extra = static_cast<const float*>(d.a); }
  else { out = static_cast<float*>(args.src ? d.x0 : d.x1); ldo = cp; extra = Xin; }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t go = (int64_t)(ti * T + ty * 4 + i) * ldo + tj * T + tx * 4;
    float v[4] = {acc[i][0], acc[i][1], acc[i][2], acc[i][3]};
    if (OP == OP_GRAM) {
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] *= alpha;
    } else {
      const gf4 x = *gmem(reinterpret_cast<const gf4*>(extra + go));
      const float xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v[j] = (OP == OP_SQUARE) ? args.b * xv[j] + args.c * v[j] : alpha * (args.a * xv[j] + v[j]);
    }
    *gmem(reinterpret_cast<gf4*>(out + go)) = gf4{v[0], v[1], v[2], v[3]};
  }
  if (OP != OP_APPLY && ti != tj) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t go = (int64_t)(tj * T + tx * 4 + j) * ldo + ti * T + ty * 4;
      float v[4] = {acc[0][j], acc[1][j], acc[2][j], acc[3][j]};
      if (OP == OP_GRAM) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] *= alpha;
      } else {
        const gf4 x = *gmem(reinterpret_cast<const gf4*>(extra + go));
        const float xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = args.b * xv[i] + args.c * v[i];
      }
      *gmem(reinterpret_cast<gf4*>(out + go)) = gf4{v[0], v[1], v[2], v[3]};
    }
  }
}

}  // namespace

void launch_ns_f32(int op, const MatDesc* mats, TileMap tm, int src, int first, float a, float b, float c,
                    hipStream_t s) {
  if (tm.total == 0) return;
  NsArgs g{mats, tm, src, first, a, b, c};
  if (op == NS_GRAM)
    hipLaunchKernelGGL(ns_f32_kernel<OP_GRAM>, dim3(tm.grid), dim3(256), 0, s, g);
  else if (op == NS_SQUARE)
    hipLaunchKernelGGL(ns_f32_kernel<OP_SQUARE>, dim3(tm.grid), dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL(ns_f32_kernel<OP_APPLY>, dim3(tm.grid), dim3(256), 0, s, g);
}

}  // namespace ma
