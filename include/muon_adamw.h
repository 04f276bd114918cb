/*
 * muon_adamw.h -- C ABI of the MI355X (gfx950) hybrid Muon + AdamW step.
 *
 * Everything here is plain C: pointers, sizes and small structs. Device
 * pointers address HBM on the GPU that is current when the call is made;
 * host pointers are marked as such. No call allocates device memory: the
 * caller owns every device buffer, including the Muon workspace. The library
 * owns only small pinned host staging buffers for its launch tables.
 *
 * Errors: every entry point validates all of its arguments before it enqueues
 * anything, so a non-OK status leaves every buffer untouched (the hybrid step
 * is all-or-nothing: the kimi-k3 "Optimization" chapter has an FP16 overflow
 * skip the update of both optimizers together). ma_last_error() returns a
 * thread-local message for the last non-OK status; the pointer stays valid
 * until this thread's next call that fails, so read it after the call returns
 * and copy it to keep it. Kernel faults are
 * asynchronous and surface at the caller's next synchronisation; a launch
 * failure seen right after enqueueing returns MA_E_HIP.
 *
 * Streams: `stream` is a hipStream_t (NULL = the legacy default stream). All
 * work of one call is enqueued on that stream in order. No call synchronises
 * the host with the device, except ma_muon_step_status() and, when the host
 * runs 64 calls ahead of the device, the reuse of a pinned staging buffer.
 * Calls that share a workspace must be ordered on one stream.
 *
 * Plans: muon_step keeps the plan of a tensor list (its matrices, shape
 * buckets, launch tables and workspace layout) keyed by the list's structure
 * (which tensors have gradients, their batch, rows, cols and views), the
 * Newton-Schulz dtype, step count and coefficients. A later call with the same
 * structure skips the planning; arguments are still validated on every call.
 */
#ifndef MUON_ADAMW_H
#define MUON_ADAMW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MA_OK = 0,
  MA_E_INVALID = 1,      /* bad pointer, shape, flag or hyperparameter       */
  MA_E_DTYPE = 2,        /* dtype outside {f32, bf16} (complex included)      */
  MA_E_ALIAS = 3,        /* two tensors' parameter or state ranges overlap    */
  MA_E_WORKSPACE = 4,    /* workspace missing or smaller than required        */
  MA_E_UNSUPPORTED = 5,  /* a combination this library does not define        */
  MA_E_HIP = 6           /* the HIP runtime reported an error                 */
} ma_status;

typedef enum { MA_F32 = 0, MA_BF16 = 1 } ma_dtype;

typedef enum {
  MA_CAUTIOUS_NONE = 0,
  /* flaxchat "Optimizer" page, "Muon Algorithm" step 4: weight decay only
   * where (update * param) >= 0; the orthogonalised update always applies. */
  MA_CAUTIOUS_WD_MASK = 1,
  /* speedtronic "v2 optimizers" page, "Cautious updates": keep an entry's
   * whole observed update (decay included) only where update * grad > 0,
   * otherwise leave the parameter unchanged. */
  MA_CAUTIOUS_WRAPPER = 2
} ma_cautious;

/*
 * One parameter tensor stepped by Muon (speedtronic "v2 optimizers" page,
 * "Muon update"; kimi-k3 "Optimization", matrix views).
 *
 * param     device, batch*rows*cols elements of param_dtype, row-major and
 *           contiguous: entry b is a rows x cols matrix (rows = output
 *           features, cols = input features). Updated in place.
 * grad      device, same shape, grad_dtype, read only. NULL means the tensor
 *           has no gradient this step: nothing about it is read or written
 *           (an inactive expert is neither moved nor decayed).
 * momentum  device, fp32, same shape as param, updated in place. It belongs to
 *           the packed parent: views share it, nothing is duplicated.
 * row_v     device, fp32, batch*rows entries (one per stored row of each view),
 *           updated in place; the NorMuon second moment (flaxchat "Muon
 *           Algorithm" step 3). Required iff hparams.normuon, else ignored.
 * views     rows are split into `views` equal blocks of rows/views rows; each
 *           block of each batch entry is one independent matrix (a packed
 *           gate/up is registered as (2, rows, columns)). rows % views == 0.
 * lr, weight_decay  this tensor's learning rate and decoupled decay.
 *
 * Tied weights must be passed once: overlapping param or momentum ranges are
 * rejected with MA_E_ALIAS.
 */
typedef struct {
  void* param;
  const void* grad;
  float* momentum;
  float* row_v;
  int64_t batch;
  int64_t rows;
  int64_t cols;
  int32_t views;
  int32_t param_dtype;   /* ma_dtype */
  int32_t grad_dtype;    /* ma_dtype */
  float lr;
  float weight_decay;
} ma_muon_tensor;

/*
 * Hyperparameters shared by every Muon tensor of one call.
 *
 * beta, nesterov   B <- beta*B + (1-beta)*G; Q <- lerp(G, B, beta) if nesterov,
 *                  else Q <- B (speedtronic "Muon update"; flaxchat step 1).
 * ns_steps, ns_a, ns_b, ns_c, ns_eps
 *                  X <- Q/(||Q||_F + ns_eps), then ns_steps times
 *                  A = X X^T; X <- a X + (b A + c A^2) X, with a matrix that has
 *                  more rows than columns transposed first and back after
 *                  (speedtronic "Newton-Schulz": 5 steps, (3.4445, -4.7750,
 *                  2.0315), eps 1e-7). 1 <= ns_steps <= 64.
 * ns_dtype         MA_BF16: bf16 operands on the MFMA matrix cores with fp32
 *                  accumulation; MA_F32: fp32 throughout.
 * normuon, normuon_beta2
 *                  NorMuon after Newton-Schulz: per stored row,
 *                  V <- V + (1-beta2)(mean_j U_ij^2 - V); U_i <- U_i / sqrt(V_i),
 *                  then rescaled to keep ||U||_F (flaxchat step 3).
 * muon_plus, muon_plus_eps
 *                  Muon+ row_col after Newton-Schulz: rows, then columns, to
 *                  unit L2 norm with eps inside each square root (speedtronic
 *                  "Muon+"). normuon and muon_plus together: MA_E_UNSUPPORTED.
 * cautious         ma_cautious.
 * ns_table         host array of ns_steps x 3 floats: iteration i uses
 *                  (a, b, c) = row i (flaxchat "Muon Algorithm" step 2 loops
 *                  over a list of coefficient triples); NULL uses (ns_a, ns_b,
 *                  ns_c) at every iteration. Read during the call only.
 * ns_norm_scale    X <- Q / (||Q||_F * ns_norm_scale + ns_eps); flaxchat's
 *                  step 2 divides by ||g|| * 1.01. 0 reads as 1.
 * clip             device, 16-byte aligned: the state ma_global_grad_norm
 *                  wrote for this step, or NULL. The gradient is read times
 *                  clip[1]; clip[2] != 0 skips the call's updates entirely
 *                  (parameters, momentum and V bitwise unchanged).
 * After these, W <- (1 - lr*wd) W - lr * sqrt(max(1, m/n)) * U with m x n the
 * view's stored shape, subject to the cautious mask.
 */
typedef struct {
  double beta;           /* doubles: the host forms 1 - beta exactly (beta2 = 0.999
                            as a float would put a 1.3e-5 error into 1 - beta2) */
  double normuon_beta2;
  float ns_a;
  float ns_b;
  float ns_c;
  float ns_eps;
  float muon_plus_eps;
  int32_t nesterov;
  int32_t ns_steps;
  int32_t ns_dtype;
  int32_t normuon;
  int32_t muon_plus;
  int32_t cautious;
  int32_t pad_;
  const float* ns_table;  /* host, ns_steps x 3, or NULL                      */
  const float* clip;      /* device clip state, or NULL                       */
  float ns_norm_scale;    /* 0 reads as 1                                      */
  int32_t pad2_;
} ma_muon_hparams;

/* Device bytes of workspace muon_step needs for this tensor list (host call,
 * no GPU work). Returns 0 and sets ma_last_error() if the arguments are
 * invalid. Also returns 0, with ma_last_error() untouched, when no tensor has a
 * gradient: muon_step then has nothing to do and needs no workspace (NULL is
 * accepted). */
size_t ma_muon_workspace_bytes(const ma_muon_tensor* tensors, int32_t n,
                               const ma_muon_hparams* hp);

/*
 * The Muon half of the hybrid step over `n` tensors (host array `tensors`,
 * host struct `hp`). `workspace` is a device buffer of at least
 * ma_muon_workspace_bytes() bytes, 256-byte aligned, owned by the caller and
 * free for the library's use until the enqueued work completes; its contents
 * on entry do not matter. Enqueues: the fused momentum/Nesterov/norm pass,
 * ns_steps x (Gram, A^2 -> bA + cA^2, aX + BX) batched over all matrices,
 * the optional NorMuon / Muon+ reductions, and the fused scale/decay/apply.
 * The first int32 of the workspace receives the call's device status (see
 * ma_muon_step_status).
 */
ma_status muon_step(const ma_muon_tensor* tensors, int32_t n, const ma_muon_hparams* hp,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Device status of the last muon_step or ma_newton_schulz that used
 * `workspace` (device, 256-byte aligned) and had at least one matrix to
 * step. Waits for `stream` (the stream of that call) and writes the status to
 * host `*status`: 0 when the step ran to completion. The bits come from the
 * persistent Newton-Schulz launch, which hands every XCD of the device a queue
 * of tiles and bounds each of its waits:
 *   MA_NS_WAIT_TIMEOUT     a wait for another tile ran out (about a second);
 *                          the launch went on, so some results may have been
 *                          computed from incomplete operands;
 *   MA_NS_QUEUE_UNDRAINED  an XCD's queue was not handed out to its end, so
 *                          some matrices were left unfinished.
 * Either means the step's results are not to be used. A step skipped by the
 * clip state reports 0. Returns MA_E_HIP if the read fails.
 */
enum { MA_NS_WAIT_TIMEOUT = 1, MA_NS_QUEUE_UNDRAINED = 2 };
ma_status ma_muon_step_status(const void* workspace, int32_t* status, void* stream);

/*
 * One tensor stepped by AdamW (dew.training.optim: optax.adamw; speedtronic
 * "v2 optimizers": torch AdamW). param (param_dtype), grad (grad_dtype), m and
 * v (moment_dtype) are device arrays of `numel` elements; param, m, v are
 * updated in place. grad == NULL skips the tensor.
 * moment_dtype MA_BF16 stores both moments in bf16 (dew.training.optim
 * "bf16_moments"): they are widened to fp32 for the update and written back
 * stochastically rounded ("stochastic_round_bf16": 16 uniform bits added below
 * the kept mantissa, then truncated; NaN stays NaN). The bits are the top 16 of
 * SplitMix64's output at state key + (i + 1) * 0x9E3779B97F4A7C15 for the
 * element's flat index i, with key = mix(seed ^ mix((step << 32) + (tensor
 * index << 1) + moment)), moment 0 for m and 1 for v, mix = SplitMix64's
 * output function (Steele, Lea and Flood, OOPSLA 2014).
 */
typedef struct {
  void* param;
  const void* grad;
  void* m;
  void* v;
  int64_t numel;
  int32_t param_dtype;
  int32_t grad_dtype;
  float lr;
  float weight_decay;
  int32_t moment_dtype;  /* ma_dtype; 0 = fp32 */
  int32_t pad_;
} ma_adamw_tensor;

/*
 * m <- beta1 m + (1-beta1) g; v <- beta2 v + (1-beta2) g^2;
 * p <- p - lr * ( (m/(1-beta1^step)) / (sqrt(v/(1-beta2^step)) + eps) + wd p ).
 * step >= 1 counts successful updates (the caller's host counter; a step the
 * clip state skipped is not one).
 * cautious   MA_CAUTIOUS_WRAPPER (speedtronic "Cautious updates": the wrapper
 *            applies to either base optimizer) keeps an entry's observed
 *            update, decay included, only where update * g > 0 and leaves the
 *            parameter as it was elsewhere; m and v are updated either way.
 *            MA_CAUTIOUS_WD_MASK is Muon's rule: MA_E_UNSUPPORTED.
 * seed       stochastic-rounding seed of bf16 moments.
 * clip       as in ma_muon_hparams: g is read times clip[1], clip[2] != 0
 *            skips every update of the call.
 */
typedef struct {
  double beta1;
  double beta2;
  double eps;
  int64_t step;
  int32_t cautious;      /* MA_CAUTIOUS_NONE or MA_CAUTIOUS_WRAPPER */
  int32_t pad_;
  uint64_t seed;
  const float* clip;     /* device clip state, or NULL */
} ma_adamw_hparams;

/* The AdamW half of the hybrid step over `n` tensors; no workspace. */
ma_status adamw_step(const ma_adamw_tensor* tensors, int32_t n, const ma_adamw_hparams* hp,
                     void* stream);

/*
 * Global gradient norm over every gradient of the hybrid step (dew.training.
 * optim "build_optimizer": the global-norm clip reads every gradient
 * together, before the parameter groups split them; kimi-k3 "Optimization":
 * with max_grad_norm > 0 the norm is clipped, with 0 it is only observed, and
 * an overflow skips the whole hybrid update).
 *
 * grads      host array of n gradient references (device arrays; grad NULL
 *            or numel 0 contributes nothing). Pass the Muon and the AdamW
 *            gradients of the step together.
 * state      device, 4 floats, 16-byte aligned, written on the stream:
 *            [0] ||g||_2 over all elements (fp64 sums of squares per 8192
 *            elements, added in fp64 in a fixed order: the same bits for the
 *            same inputs, and no overflow for any finite gradient), [1] the
 *            clip factor min(1, max_norm / ||g||) (1 when
 *            max_norm <= 0 or ||g|| <= max_norm), [2] 1 when ||g|| is not
 *            finite (the step is to be skipped), else 0, [3] 0.
 *            Hand `state` to muon_step and adamw_step (hparams.clip): they read
 *            it on the device, so nothing waits for the host. A caller that
 *            counts successful steps reads [2] back after the step.
 * workspace  device, ma_grad_norm_workspace_bytes() bytes, 256-byte aligned.
 */
typedef struct {
  const void* grad;
  int64_t numel;
  int32_t dtype;         /* ma_dtype */
  int32_t pad_;
} ma_grad_ref;

size_t ma_grad_norm_workspace_bytes(const ma_grad_ref* grads, int32_t n);
ma_status ma_global_grad_norm(const ma_grad_ref* grads, int32_t n, float max_norm, float* state,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Thread-local message for the last non-OK status of this thread. */
const char* ma_last_error(void);

/*
 * Newton-Schulz alone (speedtronic "Newton-Schulz": newton_schulz(matrix,
 * steps, eps)) on `batch` stored rows x cols matrices of `dtype` at device
 * `in`, written to device `out` (same shape and dtype; may equal `in`). Uses
 * hp's ns_* fields only. Workspace as for muon_step, sized by
 * ma_newton_schulz_workspace_bytes().
 */
size_t ma_newton_schulz_workspace_bytes(int64_t batch, int64_t rows, int64_t cols,
                                        int32_t dtype, const ma_muon_hparams* hp);
ma_status ma_newton_schulz(const void* in, void* out, int64_t batch, int64_t rows, int64_t cols,
                           int32_t dtype, const ma_muon_hparams* hp, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Host-only description of how muon_step lays out matrix `k` (0-based, in
 * tensor order, then batch entry, then view) of a tensor list. Tensors with a
 * NULL grad contribute no matrices. Used by tests and by callers that read the
 * orthogonalised update from the workspace after a step.
 */
typedef struct {
  int32_t tensor;        /* index into the tensor list                        */
  int32_t batch_index;
  int32_t view;
  int32_t m, n;          /* stored shape of the view                          */
  int32_t r, c;          /* canonical shape: min, max                         */
  int32_t rp, cp;        /* canonical shape padded to the GEMM tile           */
  int32_t transposed;    /* 1 iff m > n                                       */
  int32_t bucket;        /* index of its (r, c) shape bucket                  */
  float scale;           /* sqrt(max(1, m/n))                                 */
  int32_t pad_;
  uint64_t u_offset;     /* workspace byte offset of the final Newton-Schulz
                            output: rp x cp row-major, ns dtype, canonical
                            orientation, zero outside r x c                   */
  uint64_t a_offset;     /* workspace byte offset of the last iteration's
                            A = X X^T: rp x rp row-major, ns dtype, both
                            triangles stored (bit for bit equal)              */
  uint64_t b_offset;     /* the same for B = bA + cA^2                        */
} ma_matrix_info;

/* Number of matrices and shape buckets muon_step would form (host only). */
ma_status ma_muon_plan_counts(const ma_muon_tensor* tensors, int32_t n, const ma_muon_hparams* hp,
                              int32_t* n_matrices, int32_t* n_buckets);
ma_status ma_muon_matrix_info(const ma_muon_tensor* tensors, int32_t n, const ma_muon_hparams* hp,
                              int32_t k, ma_matrix_info* info);

/*
 * Plan introspection: the task queues of the persistent Newton-Schulz launch
 * (bf16 Newton-Schulz) for this tensor list, as the planner builds them.
 * nseg (host, 8 entries, one per XCD) receives the number of segments in XCD
 * x's queue, all 0 when the plan has none (fp32 Newton-Schulz, or no matrix).
 * `segs` (host) receives up to `max_segs` records of 4 int32 {matrix,
 * iteration * 4 + product (0 Gram, 1 square, 2 apply), index of the segment's
 * first task in its queue, tiles of that matrix that must be complete before
 * the segment's tiles start}, queue 0's first, in queue order. Host only:
 * nothing is dereferenced on the device. MA_E_INVALID when nseg is NULL,
 * max_segs < 0, or max_segs > 0 with segs NULL; otherwise the validation
 * statuses of muon_step.
 */
ma_status ma_muon_queue_info(const ma_muon_tensor* tensors, int32_t n, const ma_muon_hparams* hp,
                             int32_t* nseg, int32_t* segs, int32_t max_segs);

/*
 * Per-kernel timing with HIP events, a profiling aid (not needed for use).
 * Between ma_profile_begin() and ma_profile_end() on one host thread, every
 * kernel that muon_step, ma_newton_schulz or adamw_step enqueues is bracketed
 * by two events recorded on the same stream. ma_profile_end() waits for those
 * events, writes at most `max` entries (host array `out`, one per kernel name,
 * in first-launch order) and returns how many it wrote, or -1 on a HIP error.
 * Recording adds an event pair per launch, so time whole steps separately.
 */
typedef struct {
  char name[48];
  int64_t launches;
  double total_ms;
} ma_kernel_time;

ma_status ma_profile_begin(void);
int32_t ma_profile_end(ma_kernel_time* out, int32_t max);

/*
 * Measured ceiling of the bf16 matrix cores, a measurement aid beside the
 * nominal peak (not needed for use). Enqueues on `stream` an MFMA-only loop
 * with no memory traffic: `blocks` workgroups of 4 wave64s, each wave
 * running `iters` rounds of 8 independent v_mfma_f32_32x32x16_bf16, i.e.
 * blocks * 4 * iters * 8 * 32768 flops; the caller times it (events on the
 * same stream). `sink` is a device array of `blocks` floats, written with one
 * meaningless value per block. blocks in [1, 2^20], iters in [1, 2^24];
 * MA_E_INVALID otherwise, with nothing enqueued.
 */
ma_status ma_mfma_bf16_ceiling(float* sink, int32_t blocks, int32_t iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MUON_ADAMW_H */
