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
//   APPLY   X' = s1 * (a X + B X)    contraction over r, X read k-major
// Storage is row-major bf16 everywhere.
//
// Block: 256 x 256 outputs, 512 threads = 8 wave64s in a 2 x 4 grid, each
// wave 128 x 64 outputs = 4 x 2 tiles of v_mfma_f32_32x32x16_bf16 (128 fp32
// accumulators per lane). The contraction advances 32 per stage. Both
// operands go straight from HBM into LDS with global_load_lds_dwordx4 (no
// staging registers), four stages deep (4 x 32 KB).
//   * operands contiguous along the contraction (all of GRAM and SQUARE, B in
//     APPLY) land as 64-byte rows, the four 16-byte chunks XOR-swizzled by row
//     so that fragment reads of 8 or 16 consecutive rows hit distinct banks;
//   * APPLY's X lands as it is stored (32 k-rows of 512 B), chunks swizzled
//     by k, and its MFMA fragments are read with ds_read_b64_tr_b16: lane j of
//     each 16-lane group addresses (k0 + j/4, n0 + 4 (j%4)) and lane i then
//     holds k0..k0+3 of column n0 + i, the matrix-core operand layout.
// The direct loads place the swizzle by choosing each lane's source chunk.
// Each stage is split into two k-substeps of 16 whose fragments are double
// buffered in registers, so the LDS reads of one substep overlap the matrix
// multiplies of the other. All waits are explicit (s_waitcnt in inline
// assembly, a plain s_barrier): the compiler would otherwise wait for all
// memory traffic at every barrier and LDS read. The tail re-loads the last
// stage so the wait counts stay constant. Workgroups are dealt to XCDs so
// that all tiles of a matrix share one L2. Edge tiles (dimensions that are
// multiples of 128 but not of 256) clamp their loads and mask their stores.
//
// Epilogue: the direct tile goes through LDS in four passes of 64 fp32 rows
// and leaves as rows of 8-byte stores (one float4 of LDS per lane); the mirrored tile of the symmetric products
// leaves straight from the accumulators, whose layout already gives each lane
// four consecutive elements of a mirror row. The combine terms (b A + c A^2,
// a X + B X) and the first iteration's normalisation sigma = 1/(||Q||_F + eps)
// are applied in fp32 on the way out.
#include <type_traits>

#include "kernels.hpp"

namespace ma {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) const u32x4 g_u32x4;
typedef __attribute__((address_space(1))) u32x4 g_u32x4_w;
typedef __attribute__((address_space(1))) const u32x2 g_u32x2;
typedef __attribute__((address_space(1))) u32x2 g_u32x2_w;

constexpr int BM = 256;
constexpr int BN = 256;
constexpr int BK = 32;
constexpr int NTHR = 512;
constexpr int RB = BK * 2;               // bytes per LDS row of a contraction-contiguous operand
constexpr int XR = BN * 2;               // bytes per LDS row of APPLY's k-major X (512)
constexpr int OPB = BM * RB;             // bytes per operand per stage (16 KB; X: 32 x 512)
constexpr int NSTAGE = 4;                // direct-load pipeline depth
constexpr int SMEM = NSTAGE * 2 * OPB;   // 128 KB
constexpr int EPR = 64;                  // accumulator rows per epilogue pass
constexpr int EPP = BN + 8;              // fp32 pitch of the staged rows
static_assert(EPR * EPP * 4 <= SMEM, "epilogue staging must fit");

enum { OP_GRAM = 0, OP_SQUARE = 1, OP_APPLY = 2 };

struct NsArgs {
  const MatDesc* mats;
  TileMap tm;
  int src;     // which ping-pong buffer holds the current X
  int first;   // first iteration: fold sigma in
  float a, b, c;
};

__device__ __forceinline__ u32x4 gload16(const uint16_t* p) { return *(g_u32x4*)(p); }
__device__ __forceinline__ void gstore16(uint16_t* p, u32x4 v) { *(g_u32x4_w*)(p) = v; }
__device__ __forceinline__ u32x2 gload8(const uint16_t* p) { return *(g_u32x2*)(p); }
__device__ __forceinline__ void gstore8(uint16_t* p, u32x2 v) { *(g_u32x2_w*)(p) = v; }

// 16 bytes per lane from global memory straight into LDS: lane l's data lands
// at lds + 16 * l (lds is the wave's LDS byte address, uniform). Issued as
// inline assembly so that the compiler does not see a load into LDS: it would
// then wait for every such load (vmcnt(0)) in front of LDS reads it cannot
// prove disjoint. The hardware counts these loads in vmcnt only, never in
// lgkmcnt, so the compiler's own waits for LDS reads stay exact; the waits
// for the loads themselves are explicit (MA_WAIT_VM). M0 holds the LDS
// address; one wait state (the s_nop) separates its write from the load.
__device__ __forceinline__ void dma16(const uint16_t* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(g), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}
#define MA_WAIT_VM(n) asm volatile("s_waitcnt vmcnt(" #n ")" ::: "memory")

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
}

// Contraction-contiguous operand rows (64 B): the 16-byte chunks are XORed
// with (row / 4) mod 4. A fragment read (32 consecutive rows, one chunk each
// half-wave) then spreads every 16-lane quarter over all 16 bank groups of
// the 256-byte bank line: measured conflict-free on gfx950, where the row
// parity mixes of other swizzles cost 25% more cycles.
__device__ __forceinline__ int swz(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int lds_off(int row, int chunk) { return row * RB + ((chunk ^ swz(row)) << 4); }
// APPLY's X rows (512 B, indexed by k): chunk XOR 4 (k mod 4), so the four
// k-rows of one transposing read land in distinct 64-byte quarters of the
// 256-byte bank line (measured conflict-free; unswizzled rows cost 1.5x).
__device__ __forceinline__ int xswz(int k) { return (k & 3) << 2; }
__device__ __forceinline__ int xoff(int k, int chunk) { return k * XR + ((chunk ^ xswz(k)) << 4); }

__device__ __forceinline__ void tri_decode(int k, int& ti, int& tj) {
  int i = static_cast<int>((sqrtf(8.0f * k + 1.0f) - 1.0f) * 0.5f);
  while ((i + 1) * (i + 2) / 2 <= k) ++i;
  while (i * (i + 1) / 2 > k) --i;
  ti = i;
  tj = k - i * (i + 1) / 2;
}

// Tile orders. The tiles of one matrix run on one XCD, about 32 at a time,
// so consecutive tiles should cover a compact area of the output and share
// operand panels in that XCD's L2.
// Symmetric products (lower triangle, ntr block rows): groups of kTriGroup
// block rows in order; inside a group, column by column with the rows of the
// group fastest. A group spans the same positions as in plain row-major
// order, so the group of position t is the row-major row of t over kTriGroup.
constexpr int kTriGroup = 4;
__device__ __forceinline__ void tri_decode_grouped(int t, int ntr, int& ti, int& tj) {
  int i, j;
  tri_decode(t, i, j);
  const int r0 = (i / kTriGroup) * kTriGroup, gsz = min(kTriGroup, ntr - r0);
  int u = t - r0 * (r0 + 1) / 2;
  if (u < r0 * gsz) {            // columns left of the group's diagonal block: full height
    tj = u / gsz;
    ti = r0 + u % gsz;
    return;
  }
  u -= r0 * gsz;                 // the diagonal block: column c has gsz - c rows
  int c = 0;
  while (u >= gsz - c) {
    u -= gsz - c;
    ++c;
  }
  tj = r0 + c;
  ti = r0 + c + u;
}
// APPLY (ntr x ntc tiles): groups of kApplyGroup block rows; inside a group
// the rows are fastest, so about 32 consecutive tiles cover 8 rows x 4
// columns. With ntr <= kApplyGroup this is plain column-major order, in which
// all of B (r x r) serves every column block from L2.
constexpr int kApplyGroup = 8;
__device__ __forceinline__ void apply_decode(int t, int ntr, int ntc, int& ti, int& tj) {
  const int r0 = (t / (kApplyGroup * ntc)) * kApplyGroup, gsz = min(kApplyGroup, ntr - r0);
  const int u = t - r0 * ntc;
  ti = r0 + u % gsz;
  tj = u / gsz;
}

// b A + c A^2 for one element, in one fixed rounding order. The direct and
// the mirrored tile of SQUARE both use it, so B is symmetric bit for bit
// (left to the compiler, the two paths fused different products).
__device__ __forceinline__ float square_combine(float a, float a2, float b, float c) {
  return __builtin_fmaf(c, a2, b * a);
}

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

// One 256 x 256 output tile `t` of product OP for matrix d. `src` is the
// ping-pong buffer holding the current X, `first` folds in sigma. Every
// thread of the block calls it; it ends with a barrier, after which LDS is
// free again.
template <int OP, bool KM>
__device__ __forceinline__ void ns_tile(const MatDesc& d, int t, int src, int first, float coef_a, float coef_b,
                                        float coef_c,
                                        char* smem) {
  static_assert(!(OP == OP_GRAM && KM), "GRAM reads rows of X");
  const int rp = d.rp, cp = d.cp;
  int ti, tj;
  const int ntr = (rp + BM - 1) / BM;
  if (OP == OP_APPLY)
    apply_decode(t, ntr, (cp + BN - 1) / BN, ti, tj);
  else
    tri_decode_grouped(t, ntr, ti, tj);
  const uint16_t* Xin = static_cast<const uint16_t*>(src ? d.x1 : d.x0);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  // Operand geometry.
  const uint16_t* Abase;
  const uint16_t* Bbase;
  int lda, ldb, K, limA, limB;
  if (OP == OP_GRAM) {
    Abase = Xin; Bbase = Xin; lda = ldb = cp; K = cp; limA = limB = rp;
  } else if (OP == OP_SQUARE) {
    Abase = Bbase = static_cast<const uint16_t*>(d.a); lda = ldb = rp; K = rp; limA = limB = rp;
  } else {
    Abase = static_cast<const uint16_t*>(d.b); lda = rp; limA = rp;
    Bbase = Xin; ldb = cp; limB = cp; K = rp;
  }
  const int nk = K / BK;

  // Operand layout in LDS. Row-wise (KM false): each operand's tile rows
  // are read along the contraction, 64-byte rows per stage; APPLY's X is
  // k-major regardless, since it is stored that way. k-major (KM, SQUARE and
  // APPLY): both operands as 512-byte k-rows per stage. The first operand
  // is a symmetric matrix (A, B) whose two triangles are stored bit for bit
  // equal, so its tile rows are read as columns of its k-rows and every
  // element read is the same value as in the row-wise reading. On gfx950
  // direct loads of 512-byte row pieces stream from L2 about 1.7x faster
  // than 64-byte pieces, but the transposing LDS reads take twice the
  // instructions of 16-byte row reads; the planner picks k-major for small
  // matrices, where the operand stream limits (768 rows: 3% faster), and
  // row-wise for large ones, where the chip runs power-limited and the extra
  // LDS instructions cost clock (8192 rows: 6% slower k-major).
  const uint16_t *ga0, *ga1, *gb0, *gb1;
  if (!KM) {
    // wave w fills tile rows [32w, 32w+32) with two 16-row instructions;
    // lane l takes LDS slot (row 16i + l/4, slot l%4) and loads the chunk
    // the swizzle places there
    const int drow0 = 32 * w + (lane >> 2), drow1 = drow0 + 16;
    const int dch0 = (lane & 3) ^ swz(drow0), dch1 = (lane & 3) ^ swz(drow1);
    ga0 = Abase + (int64_t)min(ti * BM + drow0, limA - 1) * lda + dch0 * 8;
    ga1 = Abase + (int64_t)min(ti * BM + drow1, limA - 1) * lda + dch1 * 8;
    if (OP != OP_APPLY) {
      gb0 = Bbase + (int64_t)min(tj * BN + drow0, limB - 1) * ldb + dch0 * 8;
      gb1 = Bbase + (int64_t)min(tj * BN + drow1, limB - 1) * ldb + dch1 * 8;
    } else {
      const int xr0 = 4 * w + (lane >> 5), xr1 = xr0 + 2;
      const int xc0 = (lane & 31) ^ xswz(xr0), xc1 = (lane & 31) ^ xswz(xr1);
      gb0 = Bbase + (int64_t)xr0 * ldb + min(tj * BN + xc0 * 8, limB - 8);
      gb1 = Bbase + (int64_t)xr1 * ldb + min(tj * BN + xc1 * 8, limB - 8);
    }
  } else {
    // wave w fills k-rows 4w..4w+3, two rows (2 x 512 B) per instruction;
    // lane l takes row 4w + 2i + l/32, slot l%32
    const int xr0 = 4 * w + (lane >> 5), xr1 = xr0 + 2;
    const int xc0 = (lane & 31) ^ xswz(xr0), xc1 = (lane & 31) ^ xswz(xr1);
    ga0 = Abase + (int64_t)xr0 * lda + min(ti * BM + xc0 * 8, limA - 8);
    ga1 = Abase + (int64_t)xr1 * lda + min(ti * BM + xc1 * 8, limA - 8);
    gb0 = Bbase + (int64_t)xr0 * ldb + min(tj * BN + xc0 * 8, limB - 8);
    gb1 = Bbase + (int64_t)xr1 * ldb + min(tj * BN + xc1 * 8, limB - 8);
  }
  const int dlds = w * 32 * RB;   // == 4 * w * XR: the wave's first LDS byte in a stage
  char* const Abuf = smem;                         // NSTAGE x OPB
  char* const Bbuf = smem + NSTAGE * OPB;          // NSTAGE x OPB
  const uint32_t a_lds = lds_addr(Abuf) + dlds, b_lds = lds_addr(Bbuf) + dlds;

  // Direct loads of stage `stage` into LDS buffer `buf` (4 instructions per
  // wave). Stages past the end re-load the last one, so the wait counts below
  // stay constant.
  auto issue = [&](int stage, int buf) {
    const int ks = min(stage, nk - 1);
    const int64_t koffA = (int64_t)ks * BK;
    const uint32_t a = a_lds + buf * OPB, b = b_lds + buf * OPB;
    if (!KM) {
      dma16(ga0 + koffA, a);
      dma16(ga1 + koffA, a + 16 * RB);
      if (OP != OP_APPLY) {
        dma16(gb0 + koffA, b);
        dma16(gb1 + koffA, b + 16 * RB);
      } else {
        dma16(gb0 + koffA * ldb, b);
        dma16(gb1 + koffA * ldb, b + 2 * XR);
      }
    } else {
      dma16(ga0 + koffA * lda, a);
      dma16(ga1 + koffA * lda, a + 2 * XR);
      dma16(gb0 + koffA * ldb, b);
      dma16(gb1 + koffA * ldb, b + 2 * XR);
    }
  };

  const int wr = w >> 2, wc = w & 3, khalf = lane >> 5;
  // Per-lane LDS offsets of the fragments. Row-wise operands, [k-substep]:
  // A rows, NT B rows. k-major operands: the k-row and column a lane's
  // transposing read starts at (k0 = 0); the other reads of a stage are
  // whole-row shifts of it, because the swizzle depends on k mod 4 only.
  int aoff[4][2] = {}, boff[2][2] = {}, akm[4] = {}, bkm[2] = {};
  constexpr bool BKM = KM || OP == OP_APPLY;   // second operand k-major
  {
    const int q16 = lane >> 4, i16 = lane & 15;
    const int k = 8 * (q16 >> 1) + (i16 >> 2);
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!KM) aoff[i][q] = lds_off(wr * 128 + i * 32 + (lane & 31), q * 2 + khalf);
        if (!BKM && i < 2) boff[i][q] = lds_off(wc * 64 + i * 32 + (lane & 31), q * 2 + khalf);
      }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int mm = wr * 128 + i * 32 + 16 * (q16 & 1) + 4 * (i16 & 3);
      if (KM) akm[i] = xoff(k, mm >> 3) + (mm & 7) * 2;
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = wc * 64 + j * 32 + 16 * (q16 & 1) + 4 * (i16 & 3);
      if (BKM) bkm[j] = xoff(k, n >> 3) + (n & 7) * 2;
    }
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  // Fragment double buffer: while the matrix cores work through one
  // k-substep the LDS reads of the next are in flight (the compiler places
  // the LDS waits; scheduling barriers keep each read batch ahead of the
  // multiplies it overlaps).
  struct Frag {
    bf16x8 a[4];
    bf16x8 b[2];
  };
  Frag F0, F1;

  // a k-major fragment: two transposing reads of four k-rows each
  auto tr8 = [](const char* p) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(p + 4 * XR));
    const short __attribute__((ext_vector_type(8))) v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  };
  auto read = [&](Frag& f, int soff, auto Q_) {   // soff: byte offset of the stage's buffer
    constexpr int Q = decltype(Q_)::value;
    const char* As = Abuf + soff;
    const char* Bs = Bbuf + soff;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      f.b[j] = BKM ? tr8(Bs + bkm[j] + Q * 16 * XR) : *reinterpret_cast<const bf16x8*>(Bs + boff[j][Q]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      f.a[i] = KM ? tr8(As + akm[i] + Q * 16 * XR) : *reinterpret_cast<const bf16x8*>(As + aoff[i][Q]);
  };
  auto mma = [&](const Frag& f) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  // One stage kt (LDS buffer S = kt mod 4), entered with F0 = (kt, substep
  // 0) in flight: read (kt, 1) into F1 and multiply F0; then wait for stage
  // kt+1 (own loads, then the barrier for everybody's), refill the buffer
  // read in stage kt-1 with stage kt+3, read (kt+1, 0) into F0 and multiply
  // F1. Every wave's reads of stage kt-1 completed before its last multiply
  // of that stage, so the refill after the barrier overwrites nothing live.
  // The buffer index is a compile-time constant (the loop is unrolled by
  // four), so LDS offsets fold into the instructions.
  auto stage = [&](int kt, auto S_) {
    constexpr int S = decltype(S_)::value;
    read(F1, S * OPB, I1{});
    __builtin_amdgcn_sched_barrier(0);   // keep the reads ahead of the multiplies
    mma(F0);
    __builtin_amdgcn_sched_barrier(0);
    MA_WAIT_VM(4);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue(kt + 3, (S + 3) % NSTAGE);
    read(F0, ((S + 1) % NSTAGE) * OPB, I0{});
    __builtin_amdgcn_sched_barrier(0);
    mma(F1);
    __builtin_amdgcn_sched_barrier(0);
  };

  issue(0, 0);
  issue(1, 1);
  issue(2, 2);
  MA_WAIT_VM(8);
  __builtin_amdgcn_s_barrier();
  read(F0, 0, I0{});
  for (int kt = 0; kt < nk; kt += NSTAGE) {   // nk is a multiple of 4
    stage(kt, std::integral_constant<int, 0>{});
    stage(kt + 1, std::integral_constant<int, 1>{});
    stage(kt + 2, std::integral_constant<int, 2>{});
    stage(kt + 3, std::integral_constant<int, 3>{});
  }
  // drain the trailing re-loads before the epilogue reuses LDS
  MA_WAIT_VM(0);
  __syncthreads();

  // ---------------------------------------------------------------- epilogue
  float alpha = 1.f;
  if (first) {
    const float sg = gmem(d.stat)[0];
    alpha = (OP == OP_GRAM) ? sg * sg : (OP == OP_APPLY ? sg : 1.f);
  }
  uint16_t* out;
  int ldo, limR, limC;
  const uint16_t* extra = nullptr;
  if (OP == OP_GRAM) {
    out = static_cast<uint16_t*>(d.a); ldo = rp; limR = rp; limC = rp;
  } else if (OP == OP_SQUARE) {
    out = static_cast<uint16_t*>(d.b); ldo = rp; limR = rp; limC = rp; extra = static_cast<const uint16_t*>(d.a);
  } else {
    out = static_cast<uint16_t*>(src ? d.x0 : d.x1); ldo = cp; limR = rp; limC = cp; extra = Xin;
  }

  // Every load of the combine term reads a clamped, always valid address, so
  // a batch of them issues back to back; only the stores are predicated
  // (edge tiles of a 128-padded matrix). Extents are multiples of 4, so the
  // four elements of a store are all in or all out.
  auto unpack4 = [](u32x2 xx, float* x) {
    x[0] = __uint_as_float(xx.x << 16); x[1] = __uint_as_float(xx.x & 0xffff0000u);
    x[2] = __uint_as_float(xx.y << 16); x[3] = __uint_as_float(xx.y & 0xffff0000u);
  };
  auto store4 = [&](int64_t go, const float* v) {
    u32x2 o;
    o.x = pack_bf16x2(v[0], v[1]);
    o.y = pack_bf16x2(v[2], v[3]);
    gstore8(out + go, o);
  };

  if (OP != OP_APPLY && ti != tj) {
    // mirrored tile (tj, ti) straight from the accumulators: lane holds rows
    // r0..r0+3 of tile column c, i.e. four consecutive entries of mirror row c
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      u32x2 xx[2][4];
      int64_t go[2][4];
      bool ok[2][4];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int gr = tj * BN + wc * 64 + j * 32 + (lane & 31);
          const int gc = ti * BM + wr * 128 + i * 32 + 8 * g + 4 * (lane >> 5);
          ok[j][g] = gr < limR && gc < limC;
          go[j][g] = (int64_t)min(gr, limR - 1) * ldo + min(gc, limC - 4);
          if (OP == OP_SQUARE) xx[j][g] = gload8(extra + go[j][g]);
        }
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float v[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] = acc[i][j][4 * g + u];
          if (OP == OP_GRAM) {
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] *= alpha;
          } else {
            float x[4];
            unpack4(xx[j][g], x);
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = square_combine(x[u], v[u], coef_b, coef_c);
          }
          if (ok[j][g]) store4(go[j][g], v);
        }
    }
  }

  // Direct tile through LDS, 64 accumulator rows per pass; the pass's
  // combine-term loads are issued before the staging so their latency
  // overlaps it.
  float* Cs = reinterpret_cast<float*>(smem);
  constexpr int PER = (EPR * BN / 4) / NTHR;   // float4 groups per lane and pass
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    u32x2 xx[PER];
    int64_t go[PER];
    bool ok[PER];
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      // one float4 per lane: consecutive lanes read consecutive 16 bytes
      const int q = tid + NTHR * it, sr = q >> 6, cc = (q & 63) * 4;
      const int gr = ti * BM + (sr >> 5) * 128 + p * 32 + (sr & 31);
      const int gc = tj * BN + cc;
      ok[it] = gr < limR && gc < limC;
      go[it] = (int64_t)min(gr, limR - 1) * ldo + min(gc, limC - 4);
      if (OP != OP_GRAM) xx[it] = gload8(extra + go[it]);
    }
    // staged row sr = wr*32 + r  <->  tile row wr*128 + p*32 + r
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int sr = wr * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int col = wc * 64 + j * 32 + (lane & 31);
        Cs[sr * EPP + col] = acc[p][j][v];
      }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int q = tid + NTHR * it, sr = q >> 6, cc = (q & 63) * 4;
      const f32x4 c4 = *reinterpret_cast<const f32x4*>(Cs + sr * EPP + cc);
      float v[4] = {c4.x, c4.y, c4.z, c4.w};
      if (OP == OP_GRAM) {
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] *= alpha;
      } else {
        float x[4];
        unpack4(xx[it], x);
        if (OP == OP_SQUARE) {
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] = square_combine(x[u], v[u], coef_b, coef_c);
        } else {
#pragma unroll
          for (int u = 0; u < 4; ++u) v[u] = alpha * (coef_a * x[u] + v[u]);
        }
      }
      if (ok[it]) store4(go[it], v);
    }
    __syncthreads();
  }
}

// The operand layout is chosen per matrix (MatDesc::kmajor, uniform).
template <int OP>
__device__ __forceinline__ void ns_tile_any(const MatDesc& d, int t, int src, int first, float coef_a,
                                            float coef_b, float coef_c, char* smem) {
  if constexpr (OP == OP_GRAM) {
    ns_tile<OP, false>(d, t, src, first, coef_a, coef_b, coef_c, smem);
  } else {
    if (__builtin_amdgcn_readfirstlane(d.kmajor))
      ns_tile<OP, true>(d, t, src, first, coef_a, coef_b, coef_c, smem);
    else
      ns_tile<OP, false>(d, t, src, first, coef_a, coef_b, coef_c, smem);
  }
}

template <int OP>
__global__ __launch_bounds__(NTHR, 1) void ns_mfma_kernel(NsArgs args) {
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  const int t_all = block_tile(args.tm, blockIdx.x);
  if (t_all < 0) return;
  const int e = find_entry(args.tm, t_all);
  ns_tile_any<OP>(args.mats[args.tm.perm[e]], t_all - args.tm.start[e], args.src, args.first, args.a, args.b,
                  args.c, smem);
}

// All Newton-Schulz iterations of a step in one launch. Each XCD serves its
// own queue (the workgroup reads the XCD it runs on from the XCC_ID
// register): the matrices of a queue never leave that XCD, so everything a
// tile reads was written through the same L2. A queue is a list of segments
// {matrix, iteration*4 + product, first task, tiles of the matrix done
// before}, in (iteration, product, matrix) order; a block takes the next
// task, waits until the matrix's completion counter reaches the segment's
// requirement (every earlier product of that matrix complete), runs the
// tile and counts it. Tasks are taken in queue order, so a wait only ever
// depends on tasks that running blocks already hold: the schedule cannot
// deadlock. Each wait is still bounded (kMaxPolls, about a second); one that
// runs out sets the error word, after which no wait blocks again, and the
// block goes on: every wave always exits, and a broken schedule costs at
// most one timeout.
//
// Visibility: a producer waits for its own stores (vmcnt(0)) before the
// block's counter increment, so its tile is in L2 before the count moves;
// a consumer invalidates its CU's L1 (buffer_inv at agent scope) after the
// wait and before reading, since the CU may hold lines of the same matrix
// from an earlier task. L2 is shared by producer and consumer (same XCD), so
// nothing is written back. Counters are agent-scope atomics.
constexpr int kMaxPolls = 1 << 20;

__global__ __launch_bounds__(NTHR, 1) void ns_persistent_kernel(const MatDesc* __restrict__ mats, NsQueue q) {
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  __shared__ int task[4];
  // a skipped step (global-norm clip state) runs no tile; every block leaves
  // before touching the queue, so nothing waits on it
  if (step_skipped(q.clip)) return;
  const int x = __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20) & 7;   // hwreg(HW_REG_XCC_ID, 0, 4)
  const int4* segs = q.segs + q.seg_off[x];
  const int nseg = q.nseg[x];
  const int total = nseg ? segs[nseg].z : 0;   // sentinel segment holds the queue length
  // Wave 0 fetches and waits; the branch on it is wave-uniform (a scalar
  // branch), and every value it computes is made uniform with
  // readfirstlane, so the task loop stays one loop for all lanes. (With a
  // thread-0-only fetch the compiler split the loop per lane: the other
  // lanes looped back to the barrier without ever fetching again.)
  const bool wave0 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0;
  for (;;) {
    if (wave0) {
      int t = 0;
      if (threadIdx.x == 0)
        t = __hip_atomic_fetch_add(q.qhead + 32 * x, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      t = __builtin_amdgcn_readfirstlane(t);
      int m = -1, itop = 0, tile = 0;
      if (t < total) {
        int lo = 0, hi = nseg - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (__builtin_amdgcn_readfirstlane(segs[mid].z) <= t) lo = mid; else hi = mid - 1;
        }
        const int4 sg = segs[lo];
        m = __builtin_amdgcn_readfirstlane(sg.x);
        itop = __builtin_amdgcn_readfirstlane(sg.y);
        tile = t - __builtin_amdgcn_readfirstlane(sg.z);
        const int need = __builtin_amdgcn_readfirstlane(sg.w);
        for (int polls = 0;; ++polls) {
          const int done = __builtin_amdgcn_readfirstlane(
              __hip_atomic_load(q.count + 32 * m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
          if (done >= need) break;
          // after one wait has run out, no wait anywhere blocks again
          const int failed = __builtin_amdgcn_readfirstlane(
              __hip_atomic_load(q.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
          if (failed || polls >= kMaxPolls) {
            if (threadIdx.x == 0) __hip_atomic_store(q.err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          __builtin_amdgcn_s_sleep(4);
        }
        // agent scope (sc1): the workgroup-scope form does not touch the L1
        // outside thread-group-split mode, and this CU may hold lines of the
        // matrix from an earlier task
        asm volatile("buffer_inv sc1\n\ts_waitcnt vmcnt(0)" ::: "memory");
      }
      if (threadIdx.x == 0) {
        task[0] = m;
        task[1] = itop;
        task[2] = tile;
      }
    }
    __syncthreads();
    const int m = __builtin_amdgcn_readfirstlane(task[0]);
    const int itop = __builtin_amdgcn_readfirstlane(task[1]);
    const int tile = __builtin_amdgcn_readfirstlane(task[2]);
    if (m < 0) break;
    const MatDesc& d = mats[m];
    const int it = itop >> 2, op = itop & 3;
    // this iteration's (a, b, c)
    const float coef_a = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(gmem(q.coefs)[3 * it])));
    const float coef_b = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(gmem(q.coefs)[3 * it + 1])));
    const float coef_c = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(gmem(q.coefs)[3 * it + 2])));
    if (op == OP_GRAM)
      ns_tile_any<OP_GRAM>(d, tile, it & 1, it == 0, coef_a, coef_b, coef_c, smem);
    else if (op == OP_SQUARE)
      ns_tile_any<OP_SQUARE>(d, tile, it & 1, it == 0, coef_a, coef_b, coef_c, smem);
    else
      ns_tile_any<OP_APPLY>(d, tile, it & 1, it == 0, coef_a, coef_b, coef_c, smem);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this thread's stores are in L2
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_fetch_add(q.count + 32 * m, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// The outcome of the persistent launch, in the step's status word: bit 0 a
// bounded wait ran out (a tile may then have read operands before they were
// complete), bit 1 an XCD's queue was not handed out to its end (no block
// ran on that XCD, so its matrices were left unfinished). A skipped step ran
// no tile and reports 0. One thread; runs after the launch on its stream, so
// the counters it reads are final.
__global__ void ns_status_kernel(NsQueue q) {
  if (threadIdx.x != 0) return;
  int st = 0;
  if (!step_skipped(q.clip)) {
    if (gmem(q.err)[0] != 0) st |= NS_STATUS_WAIT_TIMEOUT;
    for (int x = 0; x < 8; ++x) {
      const int total = q.nseg[x] ? q.segs[q.seg_off[x] + q.nseg[x]].z : 0;
      if (gmem(q.qhead)[32 * x] < total) st |= NS_STATUS_QUEUE_UNDRAINED;
    }
  }
  gmem(q.status)[0] = st;
}

__global__ void zero_ints_kernel(int* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) gmem(p)[i] = 0;
}

}  // namespace

void launch_ns_persistent(const MatDesc* mats, const NsQueue& q, int zero_ints, hipStream_t s) {
  hipLaunchKernelGGL(zero_ints_kernel, dim3(16), dim3(256), 0, s, q.qhead, zero_ints);
  hipLaunchKernelGGL(ns_persistent_kernel, dim3(8 * kPersistBlocksPerXcd), dim3(NTHR), 0, s, mats, q);
}

void launch_ns_status(const NsQueue& q, hipStream_t s) {
  hipLaunchKernelGGL(ns_status_kernel, dim3(1), dim3(64), 0, s, q);
}

void launch_ns_bf16(int op, const MatDesc* mats, TileMap tm, int src, int first, float a, float b, float c,
                    hipStream_t s) {
  if (tm.total == 0) return;
  NsArgs g{mats, tm, src, first, a, b, c};
  if (op == NS_GRAM)
    hipLaunchKernelGGL(ns_mfma_kernel<OP_GRAM>, dim3(tm.grid), dim3(NTHR), 0, s, g);
  else if (op == NS_SQUARE)
    hipLaunchKernelGGL(ns_mfma_kernel<OP_SQUARE>, dim3(tm.grid), dim3(NTHR), 0, s, g);
  else
    hipLaunchKernelGGL(ns_mfma_kernel<OP_APPLY>, dim3(tm.grid), dim3(NTHR), 0, s, g);
}

}  // namespace ma
