// CPU stand-in for the part of the HIP runtime and of the gfx950 device
// builtins that the library's sources use. With it those sources compile for
// the host as plain C++, and their kernels run on the CPU. Every block runs on
// one OS thread. Every lane of the block is a fiber on that thread, and the
// lanes switch only where lanes of a wave or of a block exchange data:
// barriers, cross-lane builtins, matrix-core products and the wait for direct
// loads into LDS.
//
// Test infrastructure only. The product library never loads it. It lets the
// tests run the kernels' own source against the oracle and catch
// out-of-bounds accesses (guard pages around every buffer) without a GPU.
// It says nothing of timing or caches. Lanes of a wave do not run in lockstep:
// a kernel that relies on implicit ordering inside a wave without a cross-lane
// builtin or barrier would give wrong results here.
#pragma once

#include <stddef.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <functional>
#include <tuple>
#include <type_traits>
#include <utility>

// ---- qualifiers -------------------------------------------------------------
#define __global__
#define __device__
#define __host__
#define __forceinline__ inline __attribute__((always_inline))
#define __launch_bounds__(...)
#define __align__(n) __attribute__((aligned(n)))
// LDS: one copy per OS thread, and a thread runs one block at a time.
#define __shared__ static thread_local

// ---- vector and index types --------------------------------------------------
struct dim3 {
  unsigned x, y, z;
  constexpr dim3(unsigned x_ = 1, unsigned y_ = 1, unsigned z_ = 1) : x(x_), y(y_), z(z_) {}
};
struct alignas(16) int4 { int x, y, z, w; };
struct alignas(8) int2 { int x, y; };
struct alignas(16) uint4 { unsigned x, y, z, w; };
struct alignas(8) uint2 { unsigned x, y; };
struct alignas(16) float4 { float x, y, z, w; };
struct alignas(8) float2 { float x, y; };

// ---- runtime API ---------------------------------------------------------------
typedef enum hipError_t {
  hipSuccess = 0,
  hipErrorInvalidValue = 1,
  hipErrorOutOfMemory = 2,
  hipErrorNotReady = 600,
  hipErrorLaunchFailure = 719,
  hipErrorUnknown = 999,
} hipError_t;
typedef enum hipMemcpyKind {
  hipMemcpyHostToHost = 0,
  hipMemcpyHostToDevice = 1,
  hipMemcpyDeviceToHost = 2,
  hipMemcpyDeviceToDevice = 3,
  hipMemcpyDefault = 4,
} hipMemcpyKind;
typedef enum hipDeviceAttribute_t {
  hipDeviceAttributeMultiprocessorCount = 1,
  hipDeviceAttributeNumberOfXccs = 2,
} hipDeviceAttribute_t;
typedef struct ihipStream_t* hipStream_t;
typedef struct ihipEvent_t* hipEvent_t;
#define hipHostMallocDefault 0u
#define hipEventDefault 0u
#define hipEventDisableTiming 2u

hipError_t hipGetDevice(int* dev);
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int dev);
hipError_t hipGetLastError();
hipError_t hipPeekAtLastError();
const char* hipGetErrorString(hipError_t e);
hipError_t hipEventCreate(hipEvent_t* e);
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned flags);
hipError_t hipEventDestroy(hipEvent_t e);
hipError_t hipEventRecord(hipEvent_t e, hipStream_t s);
hipError_t hipEventQuery(hipEvent_t e);
hipError_t hipEventSynchronize(hipEvent_t e);
hipError_t hipEventElapsedTime(float* ms, hipEvent_t a, hipEvent_t b);
hipError_t hipHostMalloc(void** p, size_t bytes, unsigned flags);
hipError_t hipHostFree(void* p);
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind kind, hipStream_t s);
hipError_t hipStreamSynchronize(hipStream_t s);
// __device__ variables are ordinary host variables here: their address is the symbol's
#define HIP_SYMBOL(x) (reinterpret_cast<const void*>(&(x)))
hipError_t hipGetSymbolAddress(void** p, const void* symbol);

// ---- device math ---------------------------------------------------------------
using std::isfinite;
using std::isinf;
using std::isnan;
template <typename A, typename B>
inline auto min(A a, B b) -> typename std::common_type<A, B>::type {
  return b < a ? b : a;
}
template <typename A, typename B>
inline auto max(A a, B b) -> typename std::common_type<A, B>::type {
  return a < b ? b : a;
}
inline float __uint_as_float(uint32_t u) { return __builtin_bit_cast(float, u); }
inline uint32_t __float_as_uint(float f) { return __builtin_bit_cast(uint32_t, f); }
inline float __int_as_float(int32_t u) { return __builtin_bit_cast(float, u); }
inline int32_t __float_as_int(float f) { return __builtin_bit_cast(int32_t, f); }

// ---- the simulator -------------------------------------------------------------
namespace hipsim {

struct Idx3 {
  unsigned x, y, z;
};
struct Block;

// One lane: its index and the data it hands to a cross-lane operation.
struct Lane {
  Idx3 tid;
  Block* blk;
  int wave;               // wave of the block
  int lid;                // lane in the wave
  alignas(64) unsigned char xin[128];
  alignas(64) unsigned char xout[128];
  void* impl;             // scheduler state
};
struct Block {
  Idx3 bid, bdim, gdim;
  void* impl;
};

extern thread_local Lane* t_lane;

// Cross-lane operation of one wave: every active lane has written its operand
// to xin; the resolver fills xout of the active lanes (act[l] nonzero).
typedef void (*Resolver)(Lane* const* lanes, const unsigned char* act);
// Blocks the lane until all active lanes of its wave reached the same call
// site; lanes of the wave that wait at a block barrier (or have returned) are
// inactive for it. Two different call sites pending in one wave are an error.
void wave_op(int site, Resolver r);
void syncthreads(int site);
void sleep_cycles(int n);
// A fault found by the simulator: the block stops, the launch fails, and the
// message is kept for the test (hipsim_fault()).
[[noreturn]] void fault(const char* fmt, ...);

void run_grid(dim3 grid, dim3 block, const std::function<void()>& body);

template <typename... P, typename... A>
void launch(void (*k)(P...), dim3 grid, dim3 block, size_t shmem, A&&... a) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  (void)shmem;
  std::tuple<typename std::decay<P>::type...> params{static_cast<typename std::decay<P>::type>(a)...};
  run_grid(grid, block, [&]() { std::apply(k, params); });
}

template <typename T>
void resolve_first(Lane* const* lanes, const unsigned char* act) {
  int f = 0;
  while (!act[f]) ++f;
  for (int l = 0; l < 64; ++l)
    if (act[l]) memcpy(lanes[l]->xout, lanes[f]->xin, sizeof(T));
}
template <typename T>
T readfirstlane(T v, int site) {
  static_assert(sizeof(T) <= 8, "readfirstlane operand");
  memcpy(t_lane->xin, &v, sizeof(T));
  wave_op(site, resolve_first<T>);
  T r;
  memcpy(&r, t_lane->xout, sizeof(T));
  return r;
}

template <typename T>
void resolve_xor(Lane* const* lanes, const unsigned char* act) {
  for (int l = 0; l < 64; ++l) {
    if (!act[l]) continue;
    int mask, width;
    memcpy(&mask, lanes[l]->xin + 16, 4);
    memcpy(&width, lanes[l]->xin + 20, 4);
    const int src = (l & ~(width - 1)) | ((l ^ mask) & (width - 1));
    if (!act[src]) fault("__shfl_xor reads inactive lane %d (lane %d, mask %d)", src, l, mask);
    memcpy(lanes[l]->xout, lanes[src]->xin, sizeof(T));
  }
}
template <typename T>
T shfl_xor(T v, int mask, int width, int site) {
  static_assert(sizeof(T) <= 16, "shuffle operand");
  memcpy(t_lane->xin, &v, sizeof(T));
  memcpy(t_lane->xin + 16, &mask, 4);
  memcpy(t_lane->xin + 20, &width, 4);
  wave_op(site, resolve_xor<T>);
  T r;
  memcpy(&r, t_lane->xout, sizeof(T));
  return r;
}

// v_mfma_f32_32x32x16_bf16: D = C + A B over one 32 x 32 output block. Lane
// l holds row l % 32 of A and column l % 32 of B, eight contraction elements
// each (the same eight for both operands: lanes 0-31 and 32-63 hold the two
// halves), and sixteen accumulators D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32].
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
f32x16_t mfma_32x32x16_bf16(bf16x8_t a, bf16x8_t b, f32x16_t c, int cbsz, int abid, int blgp, int site);

// ds_read_b64_tr_b16: every lane names 8 bytes (four 16-bit elements) of
// LDS; inside each group of 16 lanes, lane i receives element i % 4 of lanes
// 4 e + i / 4 (e = 0..3), so a 4 x 16 block addressed row-wise arrives
// column-wise.
typedef short i16x4_t __attribute__((ext_vector_type(4)));
i16x4_t ds_read_tr16_b64(const void* p, int site);

// global_load_lds_dwordx4: 16 bytes from each lane's address to LDS at
// m0 + 16 * (lane in wave); m0 is the wave's uniform LDS byte address.
// Completion is deferred to the wave's next s_waitcnt vmcnt(n) that covers
// it when deferral is on (hipsim_set_dma_deferred), else immediate.
void dma16(const void* g, uint32_t m0);
void wait_vm(int n);

uint32_t getreg(int imm);

// v_mov_b32 with DPP, quad_perm controls (0x00-0xFF) only: lane i of each
// group of four takes lane (ctrl >> 2 (i % 4)) & 3 of its group.
int mov_dpp(int v, int ctrl, int row_mask, int bank_mask, bool bound_ctrl, int site);

}  // namespace hipsim

#define threadIdx (::hipsim::t_lane->tid)
#define blockIdx (::hipsim::t_lane->blk->bid)
#define blockDim (::hipsim::t_lane->blk->bdim)
#define gridDim (::hipsim::t_lane->blk->gdim)

#define hipLaunchKernelGGL(k, g, b, sh, st, ...) ::hipsim::launch(k, dim3(g), dim3(b), (size_t)(sh), __VA_ARGS__)

#define __syncthreads() ::hipsim::syncthreads(__LINE__)
#define __shfl_xor(v, m, w) ::hipsim::shfl_xor((v), (m), (w), __LINE__)
#define __builtin_amdgcn_readfirstlane(v) ::hipsim::readfirstlane((v), __LINE__)
#define __builtin_amdgcn_s_barrier() ::hipsim::syncthreads(__LINE__)
#define __builtin_amdgcn_sched_barrier(m) ((void)(m))
#define __builtin_amdgcn_s_setprio(n) ((void)(n))
#define __builtin_amdgcn_mov_dpp(v, ctrl, rm, bm, bc) ::hipsim::mov_dpp((v), (ctrl), (rm), (bm), (bc), __LINE__)
#define __builtin_amdgcn_s_sleep(n) ::hipsim::sleep_cycles(n)
#define __builtin_amdgcn_s_getreg(imm) ::hipsim::getreg(imm)
#define __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, x, y, z) \
  ::hipsim::mfma_32x32x16_bf16((a), (b), (c), (x), (y), (z), __LINE__)
#define __builtin_amdgcn_ds_read_tr16_b64_v4i16(p) ::hipsim::ds_read_tr16_b64((const void*)(p), __LINE__)

#define __HIP_MEMORY_SCOPE_WAVEFRONT 2
#define __HIP_MEMORY_SCOPE_WORKGROUP 3
#define __HIP_MEMORY_SCOPE_AGENT 4
#define __HIP_MEMORY_SCOPE_SYSTEM 5
#define __hip_atomic_fetch_add(p, v, order, scope) __atomic_fetch_add((p), (v), (order))
#define __hip_atomic_load(p, order, scope) __atomic_load_n((p), (order))
#define __hip_atomic_store(p, v, order, scope) __atomic_store_n((p), (v), (order))
