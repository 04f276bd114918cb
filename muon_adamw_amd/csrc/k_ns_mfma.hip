// Newton-Schulz GEMMs on the gfx950 matrix cores (bf16 operands, fp32
// accumulation), batched over every matrix of a step.
//
// One quintic iteration (speedtronic "v2 optimizers" page, "Newton-Schulz";
// flaxchat "Optimizer" page, "Muon Algorithm" step 2, wide form) is three
// launches over the canonical r x c matrices (r <= c):
//   GRAM    A  = s2 * X X^T          contraction over c; symmetric, so only
//                                     tiles on and below the diagonal are
//                                     computed and each is stored twice
//   SQUARE  B  = b A + c A A^T       A is symmetric, so A^2 = A A^T: the same
//                                     row-by-row contraction; B is symmetric
//   APPLY   X' = s1 * (a X + B X)    contraction over r with X read k-major
// Storage is row-major bf16 everywhere; the first two are "NT" products (both
// operands contiguous along the contraction), the third reads X transposed
// into LDS.
//
// Tiles: 128 x 128 outputs per 256-thread block, four waves of 64 x 64, each
// wave a 2 x 2 grid of v_mfma_f32_32x32x16_bf16. K advances 64 per stage
// through a double-buffered LDS pipeline (global loads for stage k+1 are in
// flight while stage k computes). The epilogue stages the fp32 accumulators
// in LDS and writes 16-byte rows (and the mirrored tile for the symmetric
// products), folding in the combine terms and the first iteration's
// normalisation sigma = 1/(||Q||_F + eps).
#include "kernels.hpp"

namespace ma {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 128;        // tile rows
constexpr int BN = 128;        // tile cols
constexpr int BK = 64;         // contraction per stage
constexpr int LDA = BK + 8;    // LDS row pitch in bf16 (144 B: rows stay 16-B aligned, reads spread over banks)
constexpr int OPS = BM * LDA;  // one operand stage
constexpr int CP = BN + 4;     // fp32 epilogue pitch

enum { OP_GRAM = 0, OP_SQUARE = 1, OP_APPLY = 2 };

struct NsArgs {
  const MatDesc* mats;
  TileMap tm;
  int src;     // which ping-pong buffer holds the current X
  int first;   // first iteration: fold sigma in
  float a, b, c;
};

__device__ __forceinline__ void tri_decode(int k, int& ti, int& tj) {
  int i = static_cast<int>((sqrtf(8.0f * k + 1.0f) - 1.0f) * 0.5f);
  while ((i + 1) * (i + 2) / 2 <= k) ++i;
  while (i * (i + 1) / 2 > k) --i;
  ti = i;
  tj = k - i * (i + 1) / 2;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) const u32x4 g_u32x4;

// 16-byte load through a global-address-space pointer (a plain generic
// pointer would become a flat load, which also counts against the LDS
// counter and forces early waits).
__device__ __forceinline__ u32x4 gload16(const uint16_t* p) { return *(g_u32x4*)(p); }

// Operand staging registers for one 64-deep stage: four 16-byte chunks.
struct Stage4 {
  u32x4 v0, v1, v2, v3;
};

// 128 rows x 64 k of a row-major matrix, contraction contiguous.
__device__ __forceinline__ Stage4 load_nt(const uint16_t* base, int ld, int k0) {
  const int q = threadIdx.x, row = q >> 3, kc = (q & 7) * 8;
  const uint16_t* p = base + (int64_t)row * ld + k0 + kc;
  const int64_t step = (int64_t)32 * ld;   // 256 threads cover 32 rows per chunk
  Stage4 r;
  r.v0 = gload16(p);
  r.v1 = gload16(p + step);
  r.v2 = gload16(p + 2 * step);
  r.v3 = gload16(p + 3 * step);
  return r;
}
__device__ __forceinline__ void store_nt(uint16_t* sm, const Stage4& r) {
  const int q = threadIdx.x, row = q >> 3, kc = (q & 7) * 8;
  uint16_t* p = sm + row * LDA + kc;
  *reinterpret_cast<u32x4*>(p) = r.v0;
  *reinterpret_cast<u32x4*>(p + 32 * LDA) = r.v1;
  *reinterpret_cast<u32x4*>(p + 64 * LDA) = r.v2;
  *reinterpret_cast<u32x4*>(p + 96 * LDA) = r.v3;
}
// 64 k-rows x 128 columns of a row-major matrix (columns contiguous), to be
// stored transposed (column-major in k) in LDS. Each thread owns 4 k-rows x 8
// columns.
__device__ __forceinline__ Stage4 load_nn(const uint16_t* base, int ld, int k0) {
  const int kq = threadIdx.x & 15, nc = threadIdx.x >> 4;
  const uint16_t* p = base + (int64_t)(k0 + kq * 4) * ld + nc * 8;
  Stage4 r;
  r.v0 = gload16(p);
  r.v1 = gload16(p + ld);
  r.v2 = gload16(p + 2 * ld);
  r.v3 = gload16(p + 3 * ld);
  return r;
}
__device__ __forceinline__ void store_nn(uint16_t* sm, const Stage4& r) {
  const int kq = threadIdx.x & 15, nc = threadIdx.x >> 4;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t a = r.v0[w], b = r.v1[w], c = r.v2[w], d = r.v3[w];
    // columns 2w and 2w+1 of the four k-rows
    u32x2 lo, hi;
    lo.x = __builtin_amdgcn_perm(b, a, 0x05040100u);   // (a.lo, b.lo)
    lo.y = __builtin_amdgcn_perm(d, c, 0x05040100u);   // (c.lo, d.lo)
    hi.x = __builtin_amdgcn_perm(b, a, 0x07060302u);   // (a.hi, b.hi)
    hi.y = __builtin_amdgcn_perm(d, c, 0x07060302u);   // (c.hi, d.hi)
    *reinterpret_cast<u32x2*>(sm + (nc * 8 + 2 * w) * LDA + kq * 4) = lo;
    *reinterpret_cast<u32x2*>(sm + (nc * 8 + 2 * w + 1) * LDA + kq * 4) = hi;
  }
}

typedef __attribute__((address_space(1))) u32x4 g_u32x4_w;
__device__ __forceinline__ void gstore16(uint16_t* p, u32x4 v) { *(g_u32x4_w*)(p) = v; }

__device__ __forceinline__ void unpack8(const u32x4& v, float* f) {
  f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
  f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
  f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
  f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
}
__device__ __forceinline__ u32x4 pack8(const float* f) {
  u32x4 v;
  v.x = pack_bf16x2(f[0], f[1]);
  v.y = pack_bf16x2(f[2], f[3]);
  v.z = pack_bf16x2(f[4], f[5]);
  v.w = pack_bf16x2(f[6], f[7]);
  return v;
}

template <int OP>
__global__ __launch_bounds__(256, 2) void ns_mfma_kernel(NsArgs args) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * 2 * OPS];

  const int blk = blockIdx.x;
  const int e = find_entry(args.tm, blk);
  const MatDesc& d = args.mats[args.tm.perm[e]];
  const int t = blk - args.tm.start[e];
  int ti, tj;
  if (OP == OP_APPLY) {
    const int ntc = d.cp / BN;
    ti = t / ntc;
    tj = t % ntc;
  } else {
    tri_decode(t, ti, tj);
  }
  const uint16_t* Xin = static_cast<const uint16_t*>(args.src ? d.x1 : d.x0);
  const int rp = d.rp, cp = d.cp;

  const uint16_t* Aop;   // rows ti*BM.., contraction contiguous
  const uint16_t* Bop;   // NT: rows tj*BN..; NN: columns tj*BN..
  int lda, ldb, K;
  if (OP == OP_GRAM) {
    Aop = Xin + (int64_t)ti * BM * cp; Bop = Xin + (int64_t)tj * BN * cp; lda = ldb = cp; K = cp;
  } else if (OP == OP_SQUARE) {
    const uint16_t* A = static_cast<const uint16_t*>(d.a);
    Aop = A + (int64_t)ti * BM * rp; Bop = A + (int64_t)tj * BN * rp; lda = ldb = rp; K = rp;
  } else {
    const uint16_t* B = static_cast<const uint16_t*>(d.b);
    Aop = B + (int64_t)ti * BM * rp; lda = rp;
    Bop = Xin + tj * BN; ldb = cp; K = rp;
  }

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wr = w >> 1, wc = w & 1;
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  Stage4 ra = load_nt(Aop, lda, 0);
  Stage4 rb = (OP == OP_APPLY) ? load_nn(Bop, ldb, 0) : load_nt(Bop, ldb, 0);
  store_nt(smem, ra);
  if (OP == OP_APPLY) store_nn(smem + OPS, rb); else store_nt(smem + OPS, rb);
  __syncthreads();

  const int nk = K / BK;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      ra = load_nt(Aop, lda, (kt + 1) * BK);
      rb = (OP == OP_APPLY) ? load_nn(Bop, ldb, (kt + 1) * BK) : load_nt(Bop, ldb, (kt + 1) * BK);
    }
    const uint16_t* As = smem + cur * 2 * OPS;
    const uint16_t* Bs = As + OPS;
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[2], bfv[2];
      const int koff = ks * 16 + (lane >> 5) * 8;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const bf16x8*>(As + (wr * 64 + i * 32 + (lane & 31)) * LDA + koff);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bfv[j] = *reinterpret_cast<const bf16x8*>(Bs + (wc * 64 + j * 32 + (lane & 31)) * LDA + koff);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfv[j], acc[i][j], 0, 0, 0);
    }
    if (more) {
      uint16_t* nxt = smem + (cur ^ 1) * 2 * OPS;
      store_nt(nxt, ra);
      if (OP == OP_APPLY) store_nn(nxt + OPS, rb); else store_nt(nxt + OPS, rb);
    }
    __syncthreads();
  }

  // Epilogue: accumulators -> LDS (fp32), then 16-byte rows out.
  float* Cs = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = wr * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int col = wc * 64 + j * 32 + (lane & 31);
        Cs[row * CP + col] = acc[i][j][v];
      }
  __syncthreads();

  float alpha = 1.f;
  if (args.first) {
    const float sg = d.stat[0];
    alpha = (OP == OP_GRAM) ? sg * sg : (OP == OP_APPLY ? sg : 1.f);
  }
  uint16_t* out;
  int ldo;
  const uint16_t* extra = nullptr;
  if (OP == OP_GRAM) { out = static_cast<uint16_t*>(d.a); ldo = rp; }
  else if (OP == OP_SQUARE) { out = static_cast<uint16_t*>(d.b); ldo = rp; extra = static_cast<const uint16_t*>(d.a); }
  else { out = static_cast<uint16_t*>(args.src ? d.x0 : d.x1); ldo = cp; extra = Xin; }

#pragma unroll 2
  for (int p = 0; p < 8; ++p) {
    const int q = threadIdx.x + 256 * p, row = q >> 4, cc = (q & 15) * 8;
    float v[8];
    const float4 c0 = *reinterpret_cast<const float4*>(Cs + row * CP + cc);
    const float4 c1 = *reinterpret_cast<const float4*>(Cs + row * CP + cc + 4);
    v[0] = c0.x; v[1] = c0.y; v[2] = c0.z; v[3] = c0.w;
    v[4] = c1.x; v[5] = c1.y; v[6] = c1.z; v[7] = c1.w;
    const int64_t go = (int64_t)(ti * BM + row) * ldo + tj * BN + cc;
    if (OP == OP_GRAM) {
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] *= alpha;
    } else {
      float x[8];
      unpack8(gload16(extra + go), x);
      if (OP == OP_SQUARE) {
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = args.b * x[u] + args.c * v[u];
      } else {
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = alpha * (args.a * x[u] + v[u]);
      }
    }
    gstore16(out + go, pack8(v));
  }
  if (OP != OP_APPLY && ti != tj) {
    // mirrored tile (tj, ti): element (r', c') = C(c', r')
#pragma unroll 2
    for (int p = 0; p < 8; ++p) {
      const int q = threadIdx.x + 256 * p, row = q >> 4, cc = (q & 15) * 8;
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = Cs[(cc + u) * CP + row];
      const int64_t go = (int64_t)(tj * BN + row) * ldo + ti * BM + cc;
      if (OP == OP_GRAM) {
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] *= alpha;
      } else {
        float x[8];
        unpack8(gload16(extra + go), x);
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = args.b * x[u] + args.c * v[u];
      }
      gstore16(out + go, pack8(v));
    }
  }
}

}  // namespace

void launch_ns_bf16(int op, const MatDesc* mats, TileMap tm, int src, int first, float a, float b, float c,
                    hipStream_t s) {
  if (tm.total == 0) return;
  NsArgs g{mats, tm, src, first, a, b, c};
  if (op == NS_GRAM)
    hipLaunchKernelGGL(ns_mfma_kernel<OP_GRAM>, dim3(tm.total), dim3(256), 0, s, g);
  else if (op == NS_SQUARE)
    hipLaunchKernelGGL(ns_mfma_kernel<OP_SQUARE>, dim3(tm.total), dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL(ns_mfma_kernel<OP_APPLY>, dim3(tm.total), dim3(256), 0, s, g);
}

}  // namespace ma
