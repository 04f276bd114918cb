// The CPU simulator behind tests/cpu_sim/include/hip/hip_runtime.h: block
// scheduling, lane fibers, cross-lane operations, direct loads into LDS, and
// the small runtime API the library calls. Test infrastructure only.
#include <hip/hip_runtime.h>

#include <sys/mman.h>
#include <unistd.h>

#include <atomic>
#include <chrono>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <deque>
#include <memory>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

namespace hipsim {

thread_local Lane* t_lane = nullptr;

namespace {

// Fiber switch for x86-64 (System V): saves the callee-saved registers on
// the current stack, stores the stack pointer to *save, continues on `next`
// (a stack saved the same way, or one prepared by fiber_stack). No system
// call, unlike swapcontext. The floating-point control state (MXCSR, x87
// control word) is the thread's and is not switched: no kernel changes it.
extern "C" void hipsim_switch(void** save, void* next);
extern "C" void hipsim_fiber_start();
asm(R"(
  .text
  .globl hipsim_switch
  .type hipsim_switch, @function
hipsim_switch:
  pushq %rbp
  pushq %rbx
  pushq %r12
  pushq %r13
  pushq %r14
  pushq %r15
  movq %rsp, (%rdi)
  movq %rsi, %rsp
  popq %r15
  popq %r14
  popq %r13
  popq %r12
  popq %rbx
  popq %rbp
  ret
  .size hipsim_switch, .-hipsim_switch

  .globl hipsim_fiber_start
  .type hipsim_fiber_start, @function
hipsim_fiber_start:
  andq $-16, %rsp
  call *%r12
  ud2
  .size hipsim_fiber_start, .-hipsim_fiber_start
)");

// A fresh fiber on the stack [lo, lo + size): the first switch to the
// returned pointer enters fn() through hipsim_fiber_start.
void* fiber_stack(char* lo, size_t size, void (*fn)()) {
  uint64_t* top = reinterpret_cast<uint64_t*>(reinterpret_cast<uintptr_t>(lo + size) & ~uintptr_t(15));
  uint64_t* sp = top - 8;
  sp[0] = 0;                                     // r15
  sp[1] = 0;                                     // r14
  sp[2] = 0;                                     // r13
  sp[3] = reinterpret_cast<uint64_t>(fn);        // r12: the fiber's function
  sp[4] = 0;                                     // rbx
  sp[5] = 0;                                     // rbp
  sp[6] = reinterpret_cast<uint64_t>(&hipsim_fiber_start);   // return address
  sp[7] = 0;
  return sp;
}

enum State { RUNNABLE, AT_WAVE, AT_BAR, SLEEPING, EXITED };

struct Pending {
  void* dst;
  const void* src;
};

struct LaneImpl {
  void* sp = nullptr;     // saved stack pointer of the suspended fiber
  State st = EXITED;
  int site = 0;
  Resolver res = nullptr;
  std::deque<Pending> dma;
};

constexpr size_t kStack = 256 << 10;
constexpr int kMaxLanes = 1024;

struct SimFault {};

// One OS thread that runs blocks: the lanes of its current block are fibers.
struct Worker {
  void* sched = nullptr;  // saved stack pointer of the scheduler
  Block blk;
  Lane lanes[kMaxLanes];
  LaneImpl impl[kMaxLanes];
  char* stacks = nullptr;
  size_t stack_bytes = 0;
  int nl = 0;
  const std::function<void()>* body = nullptr;
  bool faulted = false;
  Worker() {
    stack_bytes = (kStack + 4096) * kMaxLanes;
    void* p = mmap(nullptr, stack_bytes, PROT_READ | PROT_WRITE, MAP_PRIVATE | MAP_ANONYMOUS | MAP_NORESERVE, -1, 0);
    if (p == MAP_FAILED) {
      fprintf(stderr, "hipsim: cannot map lane stacks\n");
      abort();
    }
    stacks = static_cast<char*>(p);
    // a guard page below every stack: an overflow faults at once
    for (int l = 0; l < kMaxLanes; ++l) mprotect(stacks + l * (kStack + 4096), 4096, PROT_NONE);
  }
  ~Worker() { munmap(stacks, stack_bytes); }
  char* stack_of(int l) { return stacks + l * (kStack + 4096) + 4096; }
};

thread_local Worker* t_worker = nullptr;
thread_local bool t_in_lane = false;

std::mutex g_mu;
std::string g_fault;               // first fault since the last clear
std::atomic<bool> g_faulted{false};
std::atomic<int> g_workers{8};
std::atomic<bool> g_defer_dma{true};
// 0: every lane of the block to its next sync point, then resolve (lanes of
// all waves stay close together); 1 / 2: one wave at a time, as far as it
// can go before a block barrier, in ascending / descending wave order (the
// waves drift apart as far as the barriers allow)
std::atomic<int> g_schedule{0};
// XCDs that receive workgroups: the dispatcher hands workgroup b to XCD
// b mod this (8 on an MI355X; fewer stands for a device where some XCD gets
// no workgroup, which the persistent launch must report)
std::atomic<int> g_xcds{8};
std::atomic<long long> g_launches{0}, g_blocks{0}, g_wave_ops{0}, g_barriers{0}, g_dma{0}, g_mfma{0},
    g_skipped{0};
thread_local hipError_t t_last = hipSuccess;

void record_fault(const std::string& msg) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_faulted.load()) {
    g_fault = msg;
    g_faulted.store(true);
  }
}

LaneImpl& cur_impl() {
  Worker& W = *t_worker;
  return W.impl[t_lane - W.lanes];
}

void yield_to_sched() {
  Worker& W = *t_worker;
  LaneImpl& I = W.impl[t_lane - W.lanes];
  hipsim_switch(&I.sp, W.sched);
}

void complete_dma(LaneImpl& I, size_t keep) {
  while (I.dma.size() > keep) {
    const Pending p = I.dma.front();
    I.dma.pop_front();
    memcpy(p.dst, p.src, 16);
  }
}

void fiber_entry() {
  Worker& W = *t_worker;
  (*W.body)();
  LaneImpl& I = cur_impl();
  complete_dma(I, 0);
  I.st = EXITED;
  hipsim_switch(&I.sp, W.sched);
  abort();  // an exited lane is never resumed
}

const char* state_name(State s) {
  switch (s) {
    case RUNNABLE: return "runnable";
    case AT_WAVE: return "wave-op";
    case AT_BAR: return "barrier";
    case SLEEPING: return "sleeping";
    default: return "exited";
  }
}

// Runs block b of the grid on this thread. Returns false after a fault.
bool run_block(Worker& W, unsigned b, dim3 grid, dim3 block) {
  W.blk.bid = {b % grid.x, (b / grid.x) % grid.y, b / (grid.x * grid.y)};
  W.blk.bdim = {block.x, block.y, block.z};
  W.blk.gdim = {grid.x, grid.y, grid.z};
  const int n = static_cast<int>(block.x * block.y * block.z);
  W.nl = n;
  for (int l = 0; l < n; ++l) {
    Lane& L = W.lanes[l];
    L.tid = {l % block.x, (l / block.x) % block.y, l / (block.x * block.y)};
    L.blk = &W.blk;
    L.wave = l / 64;
    L.lid = l % 64;
    L.impl = &W.impl[l];
    LaneImpl& I = W.impl[l];
    I.st = RUNNABLE;
    I.dma.clear();
    I.sp = fiber_stack(W.stack_of(l), kStack, fiber_entry);
  }
  const int nwaves = (n + 63) / 64;
  const int policy = g_schedule.load();
  // Resolves wave w's pending cross-lane operation if every live lane of the
  // wave is blocked and those not at a barrier wait at one call site.
  // Returns true when lanes became runnable.
  auto resolve_wave = [&](int w, bool& sleeping) -> bool {
    Lane* wl[64];
    unsigned char act[64];
    int site = -1, other = -1, nat = 0, nbar = 0, nlive = 0;
    Resolver res = nullptr;
    for (int j = 0; j < 64; ++j) {
      const int l = w * 64 + j;
      if (l >= n || W.impl[l].st == EXITED) continue;
      ++nlive;
      const LaneImpl& I = W.impl[l];
      if (I.st == AT_WAVE) {
        ++nat;
        if (site < 0) {
          site = I.site;
          res = I.res;
        } else if (I.site != site || I.res != res) {
          other = I.site;
        }
      } else if (I.st == AT_BAR) {
        ++nbar;
      } else if (I.st == SLEEPING || I.st == RUNNABLE) {
        sleeping = true;
      }
    }
    if (nat == 0 || nat + nbar != nlive) return false;
    if (other >= 0)
      fault("divergent cross-lane operations in wave %d of block %u: lines %d and %d", w, b, site, other);
    for (int j = 0; j < 64; ++j) {
      const int l = w * 64 + j;
      wl[j] = l < n ? &W.lanes[l] : &W.lanes[w * 64];
      act[j] = l < n && W.impl[l].st == AT_WAVE;
    }
    g_wave_ops.fetch_add(1, std::memory_order_relaxed);
    Lane* const keep = t_lane;
    t_lane = nullptr;
    res(wl, act);
    t_lane = keep;
    for (int j = 0; j < 64; ++j)
      if (act[j]) W.impl[w * 64 + j].st = RUNNABLE;
    return true;
  };
  // Runs the runnable lanes of wave w once each. Returns true if any ran.
  auto run_wave = [&](int w, bool& slept) -> bool {
    bool ran = false;
    for (int j = 0; j < 64; ++j) {
      const int l = w * 64 + j;
      if (l >= n) break;
      LaneImpl& I = W.impl[l];
      if (I.st == RUNNABLE || I.st == SLEEPING) {
        I.st = RUNNABLE;
        t_lane = &W.lanes[l];
        t_in_lane = true;
        hipsim_switch(&W.sched, I.sp);
        t_in_lane = false;
        ran = true;
        if (W.impl[l].st == SLEEPING) slept = true;
        if (W.faulted) return ran;
      }
    }
    return ran;
  };
  try {
    for (;;) {
      bool progress = false, sleeping = false;
      if (policy == 0) {
        for (int w = 0; w < nwaves && !W.faulted; ++w) progress |= run_wave(w, sleeping);
        if (W.faulted) return false;
        for (int w = 0; w < nwaves; ++w) progress |= resolve_wave(w, sleeping);
      } else {
        for (int k = 0; k < nwaves; ++k) {
          const int w = policy == 1 ? k : nwaves - 1 - k;
          // this wave alone until it waits at a block barrier, exits or sleeps
          for (;;) {
            bool slept = false;
            const bool ran = run_wave(w, slept);
            if (W.faulted) return false;
            progress |= ran;
            if (slept) {
              sleeping = true;
              break;
            }
            bool dummy = false;
            if (!resolve_wave(w, dummy)) break;
            progress = true;
          }
        }
      }
      int live = 0;
      bool all_bar = true;
      for (int l = 0; l < n; ++l) {
        const State st = W.impl[l].st;
        if (st == EXITED) continue;
        ++live;
        if (st != AT_BAR) all_bar = false;
        if (st == SLEEPING || st == RUNNABLE) sleeping = true;
      }
      if (live == 0) return true;
      if (progress || sleeping) continue;
      if (all_bar) {
        g_barriers.fetch_add(1, std::memory_order_relaxed);
        for (int l = 0; l < n; ++l)
          if (W.impl[l].st == AT_BAR) W.impl[l].st = RUNNABLE;
        continue;
      }
      // nothing can move: describe the lanes and fail the launch
      std::string msg = "deadlock in block " + std::to_string(b) + ":";
      for (int w = 0; w < nwaves; ++w) {
        msg += " wave " + std::to_string(w) + " [";
        for (int j = 0; j < 64 && w * 64 + j < n; ++j) {
          const LaneImpl& I = W.impl[w * 64 + j];
          if (j == 0 || I.st != W.impl[w * 64 + j - 1].st || I.site != W.impl[w * 64 + j - 1].site)
            msg += std::string(j ? " " : "") + std::to_string(j) + ":" + state_name(I.st) + "@" + std::to_string(I.site);
        }
        msg += "]";
      }
      record_fault(msg);
      W.faulted = true;
      return false;
    }
  } catch (const SimFault&) {
    W.faulted = true;
    return false;
  }
}

void worker_loop(std::atomic<unsigned>* next, unsigned nblocks, dim3 grid, dim3 block,
                 const std::function<void()>* body) {
  // one per thread, kept for the thread's lifetime (its LDS lives in TLS too)
  static thread_local std::unique_ptr<Worker> mine;
  if (!mine) mine.reset(new Worker());
  Worker& W = *mine;
  t_worker = &W;
  W.body = body;
  W.faulted = false;
  for (;;) {
    if (g_faulted.load()) return;
    const unsigned b = next->fetch_add(1);
    if (b >= nblocks) return;
    g_blocks.fetch_add(1, std::memory_order_relaxed);
    if (!run_block(W, b, grid, block)) return;
  }
}

}  // namespace

void fault(const char* fmt, ...) {
  char buf[1024];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  std::string msg = buf;
  if (t_lane && t_lane->blk)
    msg += " (block " + std::to_string(t_lane->blk->bid.x) + ", thread " + std::to_string(t_lane->tid.x) + ")";
  record_fault(msg);
  if (t_in_lane) {
    t_worker->faulted = true;
    yield_to_sched();
    abort();
  }
  throw SimFault();
}

void wave_op(int site, Resolver r) {
  LaneImpl& I = cur_impl();
  I.st = AT_WAVE;
  I.site = site;
  I.res = r;
  yield_to_sched();
}

void syncthreads(int site) {
  LaneImpl& I = cur_impl();
  I.st = AT_BAR;
  I.site = site;
  yield_to_sched();
}

void sleep_cycles(int) {
  LaneImpl& I = cur_impl();
  // other blocks run on other threads: give them time
  if (g_workers.load() > 1) std::this_thread::sleep_for(std::chrono::microseconds(20));
  I.st = SLEEPING;
  yield_to_sched();
}

namespace {
void resolve_mfma(Lane* const* lanes, const unsigned char* act) {
  for (int l = 0; l < 64; ++l)
    if (!act[l]) fault("v_mfma_f32_32x32x16_bf16 with inactive lane %d", l);
  g_mfma.fetch_add(1, std::memory_order_relaxed);
  // A row i and B column j both come from lanes i (or j) and 32 + i
  // (bf16 bits are the top half of the fp32 pattern)
  double A[32][16], B[16][32];
  for (int l = 0; l < 64; ++l) {
    uint16_t a[8], b[8];
    memcpy(a, lanes[l]->xin, 16);
    memcpy(b, lanes[l]->xin + 16, 16);
    for (int j = 0; j < 8; ++j) {
      A[l % 32][8 * (l / 32) + j] = static_cast<double>(__builtin_bit_cast(float, uint32_t(a[j]) << 16));
      B[8 * (l / 32) + j][l % 32] = static_cast<double>(__builtin_bit_cast(float, uint32_t(b[j]) << 16));
    }
  }
  // Products of bf16 values are exact in double and their 16-term sums
  // nearly so. D = C + AB is rounded to fp32 once. Each output sums its
  // terms in k order; the inner loop runs over outputs, so it vectorises.
  double P[32][32] = {};
  for (int i = 0; i < 32; ++i)
    for (int k = 0; k < 16; ++k) {
      const double a = A[i][k];
      for (int j = 0; j < 32; ++j) P[i][j] += a * B[k][j];
    }
  for (int l = 0; l < 64; ++l) {
    f32x16_t c, d;
    memcpy(&c, lanes[l]->xin + 32, 64);
    for (int r = 0; r < 16; ++r) d[r] = static_cast<float>(c[r] + P[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32]);
    memcpy(lanes[l]->xout, &d, 64);
  }
}

void resolve_tr16(Lane* const* lanes, const unsigned char* act) {
  for (int g = 0; g < 4; ++g) {
    for (int i = 0; i < 16; ++i) {
      const int l = 16 * g + i;
      if (!act[l]) fault("ds_read_b64_tr_b16 with inactive lane %d", l);
      short out[4];
      for (int e = 0; e < 4; ++e) {
        const Lane* s = lanes[16 * g + 4 * e + i / 4];
        const short* p;
        memcpy(&p, s->xin, sizeof p);
        out[e] = p[i % 4];
      }
      memcpy(lanes[l]->xout, out, 8);
    }
  }
}
}  // namespace

f32x16_t mfma_32x32x16_bf16(bf16x8_t a, bf16x8_t b, f32x16_t c, int cbsz, int abid, int blgp, int site) {
  if (cbsz || abid || blgp) fault("v_mfma with broadcast modifiers is not simulated (line %d)", site);
  memcpy(t_lane->xin, &a, 16);
  memcpy(t_lane->xin + 16, &b, 16);
  memcpy(t_lane->xin + 32, &c, 64);
  wave_op(site, resolve_mfma);
  f32x16_t d;
  memcpy(&d, t_lane->xout, 64);
  return d;
}

i16x4_t ds_read_tr16_b64(const void* p, int site) {
  if (reinterpret_cast<uintptr_t>(p) & 7) fault("ds_read_b64_tr_b16 address not 8-byte aligned (line %d)", site);
  memcpy(t_lane->xin, &p, sizeof p);
  wave_op(site, resolve_tr16);
  i16x4_t r;
  memcpy(&r, t_lane->xout, 8);
  return r;
}

// LDS byte address -> pointer. __shared__ data is thread-local here, in the
// library's TLS block, like t_lane: the 32-bit address is completed with the
// high half of t_lane's address.
static char* lds_ptr(uint32_t a) {
  const uintptr_t anchor = reinterpret_cast<uintptr_t>(&t_lane);
  uintptr_t p = (anchor & ~uintptr_t(0xffffffffu)) | a;
  if (p > anchor + (uintptr_t(1) << 31)) p -= uintptr_t(1) << 32;
  else if (p + (uintptr_t(1) << 31) < anchor) p += uintptr_t(1) << 32;
  const uintptr_t d = p > anchor ? p - anchor : anchor - p;
  if (d > (uintptr_t(64) << 20)) fault("LDS address %#x does not resolve near the LDS block", a);
  return reinterpret_cast<char*>(p);
}

void dma16(const void* g, uint32_t m0) {
  if (reinterpret_cast<uintptr_t>(g) & 3) fault("global_load_lds_dwordx4 source not 4-byte aligned");
  char* dst = lds_ptr(m0) + 16 * t_lane->lid;
  g_dma.fetch_add(1, std::memory_order_relaxed);
  if (g_defer_dma.load()) cur_impl().dma.push_back({dst, g});
  else memcpy(dst, g, 16);
}

void wait_vm(int n) {
  if (n < 0) fault("s_waitcnt vmcnt(%d)", n);
  complete_dma(cur_impl(), static_cast<size_t>(n));
  __atomic_thread_fence(__ATOMIC_SEQ_CST);
}

namespace {
void resolve_quad_perm(Lane* const* lanes, const unsigned char* act) {
  for (int l = 0; l < 64; ++l) {
    if (!act[l]) continue;
    int ctrl;
    memcpy(&ctrl, lanes[l]->xin + 4, 4);
    const int src = (l & ~3) | ((ctrl >> (2 * (l & 3))) & 3);
    if (!act[src]) fault("DPP quad_perm reads inactive lane %d (lane %d)", src, l);
    memcpy(lanes[l]->xout, lanes[src]->xin, 4);
  }
}
}  // namespace

int mov_dpp(int v, int ctrl, int row_mask, int bank_mask, bool, int site) {
  if (ctrl < 0 || ctrl > 0xFF || row_mask != 0xF || bank_mask != 0xF)
    fault("DPP control %#x (row mask %#x, bank mask %#x) is not simulated (line %d)", ctrl, row_mask, bank_mask, site);
  memcpy(t_lane->xin, &v, 4);
  memcpy(t_lane->xin + 4, &ctrl, 4);
  wave_op(site, resolve_quad_perm);
  int r;
  memcpy(&r, t_lane->xout, 4);
  return r;
}

uint32_t getreg(int imm) {
  const int id = imm & 63, off = (imm >> 6) & 31, size = ((imm >> 11) & 31) + 1;
  if (id != 20) fault("s_getreg of hardware register %d is not simulated", id);
  const uint32_t v = t_lane->blk->bid.x % static_cast<uint32_t>(g_xcds.load());
  return (v >> off) & (size >= 32 ? ~0u : ((1u << size) - 1));
}

void run_grid(dim3 grid, dim3 block, const std::function<void()>& body) {
  const unsigned nblocks = grid.x * grid.y * grid.z;
  const unsigned nthr = block.x * block.y * block.z;
  if (g_faulted.load()) {
    g_skipped.fetch_add(1);
    t_last = hipErrorLaunchFailure;
    return;
  }
  if (nthr == 0 || nthr > kMaxLanes || nblocks == 0) {
    record_fault("launch with " + std::to_string(nblocks) + " blocks of " + std::to_string(nthr) + " threads");
    t_last = hipErrorInvalidValue;
    return;
  }
  g_launches.fetch_add(1);
  std::atomic<unsigned> next{0};
  const int nw = std::max(1, std::min<int>(g_workers.load(), static_cast<int>(nblocks)));
  if (nw == 1) {
    worker_loop(&next, nblocks, grid, block, &body);
  } else {
    std::vector<std::thread> th;
    for (int w = 0; w < nw; ++w) th.emplace_back(worker_loop, &next, nblocks, grid, block, &body);
    for (auto& t : th) t.join();
  }
  if (g_faulted.load()) t_last = hipErrorLaunchFailure;
}

}  // namespace hipsim

// ---- runtime API ---------------------------------------------------------------
struct ihipEvent_t {
  std::chrono::steady_clock::time_point t;
};

hipError_t hipGetDevice(int* dev) {
  *dev = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* value, hipDeviceAttribute_t attr, int) {
  if (attr == hipDeviceAttributeMultiprocessorCount) *value = 256;
  else if (attr == hipDeviceAttributeNumberOfXccs) *value = 8;
  else return hipErrorInvalidValue;
  return hipSuccess;
}
hipError_t hipGetLastError() {
  const hipError_t e = hipsim::t_last;
  hipsim::t_last = hipSuccess;
  return e;
}
hipError_t hipPeekAtLastError() { return hipsim::t_last; }
const char* hipGetErrorString(hipError_t e) {
  switch (e) {
    case hipSuccess: return "no error";
    case hipErrorLaunchFailure: return "simulated kernel failed";
    case hipErrorInvalidValue: return "invalid argument";
    case hipErrorNotReady: return "not ready";
    default: return "simulated runtime error";
  }
}
hipError_t hipEventCreate(hipEvent_t* e) {
  *e = new ihipEvent_t{std::chrono::steady_clock::now()};
  return hipSuccess;
}
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) { return hipEventCreate(e); }
hipError_t hipEventDestroy(hipEvent_t e) {
  delete e;
  return hipSuccess;
}
hipError_t hipEventRecord(hipEvent_t e, hipStream_t) {
  e->t = std::chrono::steady_clock::now();
  return hipSuccess;
}
hipError_t hipEventQuery(hipEvent_t) { return hipSuccess; }
hipError_t hipEventSynchronize(hipEvent_t) { return hipSuccess; }
hipError_t hipEventElapsedTime(float* ms, hipEvent_t a, hipEvent_t b) {
  *ms = std::chrono::duration<float, std::milli>(b->t - a->t).count();
  return hipSuccess;
}
hipError_t hipHostMalloc(void** p, size_t bytes, unsigned) {
  return posix_memalign(p, 4096, bytes ? bytes : 1) == 0 ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipHostFree(void* p) {
  free(p);
  return hipSuccess;
}
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind, hipStream_t) {
  memmove(dst, src, bytes);
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipGetSymbolAddress(void** p, const void* symbol) {
  *p = const_cast<void*>(symbol);
  return hipSuccess;
}

// ---- controls for the tests -------------------------------------------------------
extern "C" {
int hipsim_set_workers(int n) {
  const int old = hipsim::g_workers.load();
  hipsim::g_workers.store(n < 1 ? 1 : n);
  return old;
}
int hipsim_set_dma_deferred(int on) { return hipsim::g_defer_dma.exchange(on != 0) ? 1 : 0; }
int hipsim_set_xcds(int n) { return hipsim::g_xcds.exchange(n < 1 || n > 8 ? 8 : n); }
int hipsim_set_schedule(int policy) { return hipsim::g_schedule.exchange(policy < 0 || policy > 2 ? 0 : policy); }
// The first fault since the last clear ("" if none): a copy taken under the
// lock, valid until this thread's next call.
const char* hipsim_fault() {
  static thread_local std::string copy;
  std::lock_guard<std::mutex> lk(hipsim::g_mu);
  copy = hipsim::g_fault;
  return copy.c_str();
}
void hipsim_clear_fault() {
  std::lock_guard<std::mutex> lk(hipsim::g_mu);
  hipsim::g_fault.clear();
  hipsim::g_faulted.store(false);
}
long long hipsim_counter(int which) {
  switch (which) {
    case 0: return hipsim::g_launches.load();
    case 1: return hipsim::g_blocks.load();
    case 2: return hipsim::g_wave_ops.load();
    case 3: return hipsim::g_barriers.load();
    case 4: return hipsim::g_dma.load();
    case 5: return hipsim::g_mfma.load();
    case 6: return hipsim::g_skipped.load();
    default: return -1;
  }
}
}
