// Host-side launchers of the Muon / AdamW kernels. Each enqueues on `s`.
#pragma once

#include "common.hpp"

namespace ma {

// Momentum EMA + Nesterov lerp + canonical-orientation Q write + per-tile
// Frobenius partials (speedtronic "Muon update", first two lines).
void launch_momentum(const MatDesc* mats, TileMap tm, int ns_dt, float beta, float one_minus_beta,
                     int nesterov, hipStream_t s);
// sigma = 1 / (sqrt(sum of partials) * scale + eps), one block per matrix, fixed
// order in fp64. A matrix whose norm could overflow the fp32 sums of the first
// Gram has its X0 scaled by a power of two there, and sigma compensates.
void launch_norm_finalize(const MatDesc* mats, TileMap tm, int ns_dt, float eps, float scale, hipStream_t s);

// One product of a Newton-Schulz iteration over every matrix (op 0: Gram
// A = s2 * X X^T, lower-triangle tiles mirrored; op 1: B = b A + c A A^T, A
// symmetric; op 2: X' = s1 * (a X + B X)). On the first iteration s2 = sigma^2
// and s1 = sigma (the normalisation folded in); otherwise both are 1.
enum : int { NS_GRAM = 0, NS_SQUARE = 1, NS_APPLY = 2 };
void launch_ns_bf16(int op, const MatDesc* mats, TileMap tm, int src, int first, float a, float b, float c,
                    hipStream_t s);
void launch_ns_f32(int op, const MatDesc* mats, TileMap tm, int src, int first, float a, float b, float c,
                   hipStream_t s);
// Every iteration of the bf16 Newton-Schulz chain in one persistent launch
// (after zeroing the first `zero_ints` ints at q.qhead: the queue heads, the
// error word and the completion counters).
// The coefficients of iteration it are q.coefs[3 it .. 3 it + 2].
void launch_ns_persistent(const MatDesc* mats, const NsQueue& q, int zero_ints, hipStream_t s);
// After the persistent launch: writes q.status (bit 0: a bounded wait ran out,
// bit 1: a queue was not handed out to its end; 0 on a skipped step).
enum : int { NS_STATUS_WAIT_TIMEOUT = 1, NS_STATUS_QUEUE_UNDRAINED = 2 };
void launch_ns_status(const NsQueue& q, hipStream_t s);

// Sums of squares of the final Newton-Schulz output along canonical rows
// (csum_r) or canonical columns (csum_c), optionally weighted by the square
// of the stored-row factor (Muon+ second stage).
void launch_canon_rowsum(const MatDesc* mats, TileMap tm, int ns_dt, int src, int weighted,
                         hipStream_t s);
void launch_canon_colsum(const MatDesc* mats, TileMap tm, int ns_dt, int src, int weighted,
                         hipStream_t s);
// NorMuon: V update and per-stored-row factor d_i * kappa (one block / matrix).
void launch_finalize_normuon(const MatDesc* mats, TileMap tm, float one_minus_beta2, hipStream_t s);
// Muon+: stage 1 row factors 1/sqrt(r_i + eps), stage 2 column factors.
void launch_finalize_muon_plus(const MatDesc* mats, TileMap tm, int stage, float eps, hipStream_t s);

// Scale + decoupled decay + apply in the stored orientation, with the cautious
// masks; mode 1 copies U out instead (Newton-Schulz-only entry).
enum : int { APPLY_UPDATE = 0, APPLY_COPY = 1 };
void launch_apply(const MatDesc* mats, TileMap tm, int ns_dt, int src, int mode, int cautious,
                  int use_rfac, int use_cfac, hipStream_t s);

// Multi-tensor AdamW.
struct AdamTensorArg {
  void* p;
  const void* g;
  void* m;            // fp32, or bf16 stored by stochastic rounding
  void* v;
  int64_t numel;
  int64_t index0;     // tensor-flat index of element 0 (the rounding counter)
  uint64_t key_m;     // stochastic-rounding keys of the two moments
  uint64_t key_v;
  int32_t pdt, gdt, mdt;
  float lr, wd;
};
constexpr int kMaxAdamTensors = 32;
constexpr int kAdamChunk = 2048;  // elements per block
struct AdamLaunch {
  AdamTensorArg t[kMaxAdamTensors];
  int32_t block_start[kMaxAdamTensors + 1];
  int32_t nt;
  int32_t cautious;   // keep an entry's update only where update * grad > 0
  float b1, omb1, b2, omb2, eps, inv_bc1, inv_sqrt_bc2;
  const float* clip;  // global-norm clip state or null
};
static_assert(sizeof(AdamLaunch) <= 4000, "kernel argument size");
// SplitMix64's output function (Steele, Lea and Flood, "Fast splittable
// pseudorandom number generators", OOPSLA 2014) and its state increment.
constexpr uint64_t kSplitMixGamma = 0x9E3779B97F4A7C15ull;
__host__ __device__ inline uint64_t splitmix64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
void launch_adamw(const AdamLaunch& L, int nblocks, hipStream_t s);

// Global gradient norm: per-chunk fp64 partial sums of g^2 (an fp32 square
// overflows above |g| ~ 1.8e19), then one block that adds them in fp64 in a
// fixed order and writes the clip state.
struct GradNormArg {
  const void* g;
  int64_t numel;
  int32_t dt;
  int32_t pad_;
};
constexpr int kMaxGradNormTensors = 64;
constexpr int kGradNormChunk = 8192;   // elements per block
struct GradNormLaunch {
  GradNormArg t[kMaxGradNormTensors];
  int32_t block_start[kMaxGradNormTensors + 1];
  int32_t nt;
  double* partial;     // one fp64 per block of all launches
  int32_t partial_off; // this launch's first partial
};
void launch_grad_sumsq(const GradNormLaunch& L, int nblocks, hipStream_t s);
void launch_grad_norm_finalize(const double* partial, int n, float max_norm, float* state, hipStream_t s);

// Measured bf16 matrix-core ceiling: `blocks` workgroups of 4 waves, each
// wave `iters` x 8 v_mfma_f32_32x32x16_bf16 on registers only (32768 flops
// each); one float per block to `sink`.
void launch_mfma_ceiling(float* sink, int blocks, int iters, hipStream_t s);

}  // namespace ma
