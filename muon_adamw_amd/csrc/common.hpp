// Shared host/device definitions of the Muon + AdamW library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ma {

enum : int32_t { DT_F32 = 0, DT_BF16 = 1 };
enum : int32_t { CAUT_NONE = 0, CAUT_WD_MASK = 1, CAUT_WRAPPER = 2 };

// Canonical buffers are padded to multiples of this many rows and columns, so
// every Newton-Schulz GEMM tile is full. Zero padding is exact: zero rows and
// columns stay zero through X X^T, A^2 and B X.
constexpr int kPad = 128;
// Element tile of the momentum pass, the reductions and the apply pass.
constexpr int kEw = 64;
// Output tile edge of the Newton-Schulz GEMMs (bf16 matrix-core / fp32 paths).
// The bf16 tile may overhang a 128-padded matrix; its loads clamp and its
// stores are masked.
constexpr int kNsTileBf16 = 256;
constexpr int kNsTileF32 = 64;

// One matrix: one view of one batch entry of one Muon tensor, plus its
// workspace buffers. Built on the host, read by every Muon kernel.
struct MatDesc {
  // stored view (row-major m x n, leading dimension n)
  void* param;        // first element of the view
  const void* grad;   // first element of the view
  float* mom;         // first element of the view; null: Newton-Schulz only
  float* row_v;       // NorMuon second moment of the view's m rows, or null
  int32_t m, n;       // stored shape
  int32_t r, c;       // canonical shape (min, max)
  int32_t rp, cp;     // padded canonical shape
  int32_t tall;       // m > n: canonical = stored transposed
  int32_t pdt, gdt;   // param / grad dtype
  int32_t vec;        // stored rows may use 16-byte accesses
  float decay;        // 1 - lr*wd
  float lrwd;         // lr*wd
  float step;         // lr*scale
  float scale;        // sqrt(max(1, m/n))
  // workspace
  void* x0;           // canonical rp x cp, ns dtype: Q, then X2, X4
  void* x1;           // canonical rp x cp, ns dtype: X1, X3, X5
  void* a;            // rp x rp Gram
  void* b;            // rp x rp  b*A + c*A^2
  double* part;       // sum-of-squares partial per momentum-pass tile (fp64: no overflow)
  float* stat;        // [0] sigma = 1/(||Q||_F + eps) of X0; [1] the power of two X0 was
                      // scaled by against an overflow of the first Gram (1: not scaled)
  float* csum_r;      // canonical row sums of squares, rp entries
  float* csum_c;      // canonical column sums of squares, cp entries
  float* rfac;        // per stored row factor, m entries
  float* cfac;        // per stored column factor, n entries
  // global-norm clip state of the step (ma_global_grad_norm: [1] the factor
  // the gradient is read with, [2] nonzero: skip every update), or null
  const float* clip;
  int32_t ntile_ew;   // number of momentum-pass tiles (= partial count)
  int32_t kmajor;     // SQUARE and APPLY read both operands k-major (else row-wise)
};


// Maps a flat block index to (matrix, local tile) for one launch: matrices
// are visited in `perm` order; entry k owns tiles [start[k], start[k+1]).
//
// With `xcd` set the launch is XCD-aware: the hardware hands workgroup b to
// XCD b % 8, so tile lists are laid out XCD-major (all tiles of a matrix on
// one XCD, sharing its L2) and block b takes tile xbase[b % 8] + b / 8 of its
// XCD's list, or exits if that list is shorter.
struct TileMap {
  const int32_t* start;  // nmat + 1 prefix sums
  const int32_t* perm;   // nmat matrix indices
  int32_t nmat;
  int32_t total;         // tiles (= start[nmat])
  int32_t grid;          // blocks to launch
  int32_t xcd;           // 1: XCD-aware decode below
  int32_t xbase[8];
  int32_t xcnt[8];
};

// Task queues of the persistent Newton-Schulz launch: one per XCD.
// segs[seg_off[x] .. seg_off[x] + nseg[x]] are XCD x's segments {matrix,
// iteration * 4 + product, first task index, tiles of the matrix that must
// be complete first}, followed by a sentinel whose .z is the queue length.
// qhead (8 counters, 32 ints apart), err (1 int, then padding) and count
// (one counter per matrix, 32 ints apart) are contiguous in that order and
// zeroed by the launcher.
constexpr int kPersistBlocksPerXcd = 32;   // one block per CU
struct NsQueue {
  const int4* segs;
  int* qhead;
  int* err;
  int* count;
  int* status;          // the step's status word (first int of the workspace)
  const float* coefs;   // (a, b, c) of each iteration, 3 floats per iteration
  const float* clip;    // the step's clip state or null: a skipped step runs no tile
  int32_t seg_off[8];
  int32_t nseg[8];
};

__device__ __forceinline__ int find_entry(const TileMap& tm, int tile) {
  int lo = 0, hi = tm.nmat - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (tm.start[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Block -> tile index of the launch, or -1 for an idle block.
__device__ __forceinline__ int block_tile(const TileMap& tm, int blk) {
  if (!tm.xcd) return blk;
  const int x = blk & 7, s = blk >> 3;
  return s < tm.xcnt[x] ? tm.xbase[x] + s : -1;
}

// bf16 <-> fp32. Stores round to nearest even with the hardware conversion
// (v_cvt_pk_bf16_f32, two values per instruction, no branches).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t h = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, h);
}

// Global-memory view of a generic pointer (one read from a descriptor, say):
// accesses through it compile to global_* instructions instead of FLAT ones,
// which also count in lgkmcnt and cost more to issue.
// (clang vector types: HIP's float4 and friends are classes whose members
// cannot be used through an address-space-qualified pointer)
typedef float gf4 __attribute__((ext_vector_type(4)));
typedef uint32_t gu2 __attribute__((ext_vector_type(2)));
template <typename T>
__device__ __forceinline__ __attribute__((address_space(1))) T* gmem(T* p) {
  return (__attribute__((address_space(1))) T*)(p);
}

__device__ __forceinline__ float load_elem(const void* p, int64_t i, int dt) {
  return dt == DT_BF16 ? bf16_to_f32(gmem(static_cast<const uint16_t*>(p))[i])
                       : gmem(static_cast<const float*>(p))[i];
}
__device__ __forceinline__ void store_elem(void* p, int64_t i, int dt, float v) {
  if (dt == DT_BF16) gmem(static_cast<uint16_t*>(p))[i] = f32_to_bf16(v);
  else gmem(static_cast<float*>(p))[i] = v;
}

// Wave64 sum in a fixed butterfly order (deterministic).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// The step is skipped (clip state says so): nothing may be written.
__device__ __forceinline__ bool step_skipped(const float* clip) {
  return clip != nullptr && __builtin_amdgcn_readfirstlane(__float_as_uint(gmem(clip)[2])) != 0u;
}
__device__ __forceinline__ float clip_factor(const float* clip) {
  return clip != nullptr ? __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(gmem(clip)[1]))) : 1.0f;
}

}  // namespace ma
