// C ABI of the hybrid Muon + AdamW step: argument validation, the
// shape-bucketing planner, the launch-table upload and the launch sequence.
//
// Planner: every Muon tensor is expanded into its matrices (batch entries x
// row views; kimi-k3 "Optimization", matrix views; dew.training.optim,
// BATCH_AXES), each matrix is put in canonical orientation (r = min(m, n)
// rows; speedtronic "Newton-Schulz": tall matrices are transposed), padded to
// the GEMM tile, grouped into (r, c) shape buckets, and given its workspace
// buffers. Each kernel launch then covers every matrix at once through a tile
// map whose order puts the buckets with the longest tiles first, so one launch
// per Newton-Schulz product serves the whole step.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <cstdlib>
#include <vector>

#include "muon_adamw.h"
#include "kernels.hpp"

using namespace ma;

static_assert(MA_NS_WAIT_TIMEOUT == NS_STATUS_WAIT_TIMEOUT && MA_NS_QUEUE_UNDRAINED == NS_STATUS_QUEUE_UNDRAINED,
              "status bits of the header and the kernels");

namespace {

thread_local std::string g_err;

ma_status fail(ma_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

constexpr size_t kAlign = 256;
// The first bytes of a Muon workspace: the status word of the call that last
// used it (int32 at offset 0), then padding.
constexpr size_t kHeaderBytes = 256;
size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }
int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
size_t dtype_size(int32_t dt) { return dt == MA_BF16 ? 2 : 4; }
bool dtype_ok(int32_t dt) { return dt == MA_F32 || dt == MA_BF16; }

// ---------------------------------------------------------------------------
// Plan
// ---------------------------------------------------------------------------
struct MatPlan {
  int tensor, bidx, view;
  int m, n, r, c, rp, cp, tall, bucket;
  float scale;
  int64_t elem_off;   // element offset of the view inside its tensor
  int64_t rowv_off;   // offset of the view's first row in row_v
  int ntile_ew;
  size_t off_x0, off_x1, off_a, off_b, off_part, off_stat, off_csr, off_csc, off_rf, off_cf;
};

struct MapRef {
  size_t start_off = 0, perm_off = 0;  // byte offsets inside the table region
  int nmat = 0, total = 0, grid = 0, xcd = 0;
  int xbase[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int xcnt[8] = {0, 0, 0, 0, 0, 0, 0, 0};
};

struct Plan {
  std::vector<MatPlan> mats;
  int nbuckets = 0;
  int ns_dt = MA_BF16;
  int gemm_tile = 128;
  std::vector<int32_t> ints;
  size_t desc_bytes = 0, table_bytes = 0, ws_bytes = 0;
  // persistent Newton-Schulz launch (bf16): per-XCD segment lists in `ints`
  // (int4 records from byte segs_off) and a zeroed counter region; built
  // whenever the launch could be used (a call still takes the per-launch
  // schedule on a device that cannot run it, or when asked to)
  bool persist = false;
  size_t coefs_off = 0;   // byte offset of the coefficient table within the int tables
  size_t segs_off = 0, off_counters = 0;
  int counter_ints = 0;
  int32_t seg_off[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  int32_t nseg[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  MapRef ew, gram, sq, app, rows_nt, cols_t, rows_t, cols_nt, fin_all, out;
};

struct Item {
  int mat;
  int tiles;
  int64_t key;  // per-tile work; larger first
};

constexpr int kXcds = 8;  // MI355X: 8 XCDs, workgroups dealt round-robin
// Steps with at most this many matrices run Newton-Schulz as one persistent
// launch; the counter region grows by 128 bytes per matrix. The environment
// variable MA_NS_SCHEDULE=launches selects three launches per iteration
// instead (same tiles, plain kernel boundaries between the products), and so
// does a device that is not one MI355X of 8 XCDs.
constexpr int kMaxPersistMats = 1 << 16;
// SQUARE and APPLY of matrices with at most this many (padded) rows read
// both operands k-major; larger ones read their symmetric operand row-wise.
// MA_NS_OPERANDS=kmajor or =rows forces one layout (the results are the same
// bits either way).
constexpr int kKmajorMaxRows = 2048;

// Lays out a launch's tile list. Plain maps keep one list ordered by
// decreasing per-tile work (the dispatcher then runs longest tiles first).
// XCD-aware maps deal whole matrices to the 8 XCDs by `xcd_of` (the same
// for all three Newton-Schulz launches, so a matrix's operands stay behind
// one L2), then order each XCD's list by decreasing per-tile work.
MapRef add_map(Plan& P, std::vector<Item> items, const std::vector<int>* xcd_of = nullptr) {
  const bool xcd_aware = xcd_of != nullptr;
  auto by_key = [](const Item& x, const Item& y) { return x.key > y.key; };
  std::stable_sort(items.begin(), items.end(), by_key);
  MapRef r;
  r.nmat = static_cast<int>(items.size());
  std::vector<Item> order;
  if (xcd_aware && !items.empty()) {
    std::vector<std::vector<Item>> bin(kXcds);
    for (const Item& it : items) bin[(*xcd_of)[it.mat]].push_back(it);
    int64_t base = 0, maxc = 0;
    for (int x = 0; x < kXcds; ++x) {
      std::stable_sort(bin[x].begin(), bin[x].end(), by_key);
      int64_t c = 0;
      for (const Item& it : bin[x]) {
        order.push_back(it);
        c += it.tiles;
      }
      r.xbase[x] = static_cast<int>(base);
      r.xcnt[x] = static_cast<int>(c);
      base += c;
      maxc = std::max(maxc, c);
    }
    r.xcd = 1;
    r.grid = static_cast<int>(maxc * kXcds);
  } else {
    order = items;
  }
  r.start_off = P.ints.size() * sizeof(int32_t);
  int64_t acc = 0;
  for (const Item& it : order) {
    P.ints.push_back(static_cast<int32_t>(acc));
    acc += it.tiles;
  }
  P.ints.push_back(static_cast<int32_t>(acc));
  r.perm_off = P.ints.size() * sizeof(int32_t);
  for (const Item& it : order) P.ints.push_back(it.mat);
  r.total = static_cast<int>(acc);
  if (!r.xcd) r.grid = r.total;
  return r;
}

ma_status validate_hparams(const ma_muon_hparams* hp) {
  if (!hp) return fail(MA_E_INVALID, "hparams is NULL");
  if (!(hp->beta >= 0.0 && hp->beta < 1.0)) return fail(MA_E_INVALID, "beta must be in [0, 1)");
  if (hp->nesterov != 0 && hp->nesterov != 1) return fail(MA_E_INVALID, "nesterov must be 0 or 1");
  if (hp->ns_steps < 1 || hp->ns_steps > 64) return fail(MA_E_INVALID, "ns_steps must be in [1, 64]");
  if (!std::isfinite(hp->ns_a) || !std::isfinite(hp->ns_b) || !std::isfinite(hp->ns_c))
    return fail(MA_E_INVALID, "Newton-Schulz coefficients must be finite");
  if (!(hp->ns_eps >= 0.f) || !std::isfinite(hp->ns_eps)) return fail(MA_E_INVALID, "ns_eps must be finite and >= 0");
  if (!dtype_ok(hp->ns_dtype)) return fail(MA_E_DTYPE, "ns_dtype must be MA_F32 or MA_BF16");
  if (hp->normuon != 0 && hp->normuon != 1) return fail(MA_E_INVALID, "normuon must be 0 or 1");
  if (hp->muon_plus != 0 && hp->muon_plus != 1) return fail(MA_E_INVALID, "muon_plus must be 0 or 1");
  if (hp->normuon && hp->muon_plus)
    return fail(MA_E_UNSUPPORTED, "NorMuon and Muon+ together are not defined; enable one");
  if (hp->normuon && !(hp->normuon_beta2 >= 0.0 && hp->normuon_beta2 <= 1.0))
    return fail(MA_E_INVALID, "normuon_beta2 must be in [0, 1]");
  if (hp->muon_plus && !(hp->muon_plus_eps >= 0.f && std::isfinite(hp->muon_plus_eps)))
    return fail(MA_E_INVALID, "muon_plus_eps must be finite and >= 0");
  if (hp->cautious < MA_CAUTIOUS_NONE || hp->cautious > MA_CAUTIOUS_WRAPPER)
    return fail(MA_E_INVALID, "cautious must be 0 (none), 1 (weight-decay mask) or 2 (wrapper)");
  if (hp->ns_table)
    for (int i = 0; i < 3 * hp->ns_steps; ++i)
      if (!std::isfinite(hp->ns_table[i])) return fail(MA_E_INVALID, "ns_table entries must be finite");
  if (!(hp->ns_norm_scale >= 0.f) || !std::isfinite(hp->ns_norm_scale))
    return fail(MA_E_INVALID, "ns_norm_scale must be finite and >= 0 (0 reads as 1)");
  if (reinterpret_cast<uintptr_t>(hp->clip) % 16) return fail(MA_E_INVALID, "clip state must be 16-byte aligned");
  return MA_OK;
}

// Coefficient k (0: a, 1: b, 2: c) of Newton-Schulz iteration `it`.
float ns_coef(const ma_muon_hparams* hp, int it, int k) {
  if (hp->ns_table) return hp->ns_table[3 * it + k];
  return k == 0 ? hp->ns_a : (k == 1 ? hp->ns_b : hp->ns_c);
}
float ns_norm_scale(const ma_muon_hparams* hp) { return hp->ns_norm_scale > 0.f ? hp->ns_norm_scale : 1.0f; }

struct Range {
  uintptr_t lo, hi;
  int tensor;
  const char* what;
};

ma_status check_overlaps(std::vector<Range>& rs) {
  std::sort(rs.begin(), rs.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  for (size_t i = 1; i < rs.size(); ++i) {
    if (rs[i].lo < rs[i - 1].hi)
      return fail(MA_E_ALIAS, std::string("overlapping buffers: ") + rs[i - 1].what + " of tensor " +
                                  std::to_string(rs[i - 1].tensor) + " and " + rs[i].what + " of tensor " +
                                  std::to_string(rs[i].tensor) + " (tied weights must be passed once)");
  }
  return MA_OK;
}

// Validates every argument that a call brings: pointers, alignment, dtypes,
// sizes, values and overlaps. Runs on every call. `ns_only`: the
// Newton-Schulz-only entry (no momentum, param = output).
ma_status validate_tensors(const ma_muon_tensor* t, int32_t n, const ma_muon_hparams* hp, bool ns_only) {
  ma_status st = validate_hparams(hp);
  if (st != MA_OK) return st;
  if (n < 0) return fail(MA_E_INVALID, "tensor count is negative");
  if (n > 0 && !t) return fail(MA_E_INVALID, "tensor array is NULL");
  std::vector<Range> ranges;
  for (int i = 0; i < n; ++i) {
    const ma_muon_tensor& x = t[i];
    const std::string who = "tensor " + std::to_string(i) + ": ";
    if (!dtype_ok(x.param_dtype) || !dtype_ok(x.grad_dtype))
      return fail(MA_E_DTYPE, who + "param/grad dtype must be MA_F32 or MA_BF16 (complex is not supported)");
    if (!x.param) return fail(MA_E_INVALID, who + "param is NULL");
    if (x.batch < 1 || x.rows < 1 || x.cols < 1) return fail(MA_E_INVALID, who + "batch, rows and cols must be >= 1");
    if (x.views < 1 || x.rows % x.views != 0) return fail(MA_E_INVALID, who + "views must be >= 1 and divide rows");
    if (x.rows / x.views > 65536 || x.cols > 65536)
      return fail(MA_E_UNSUPPORTED, who + "matrix dimensions above 65536 are not supported");
    if (x.batch * x.views > (1 << 20)) return fail(MA_E_UNSUPPORTED, who + "too many matrices");
    if (!std::isfinite(x.lr) || !std::isfinite(x.weight_decay))
      return fail(MA_E_INVALID, who + "lr and weight_decay must be finite");
    if (!x.grad) continue;
    if (!ns_only && !x.momentum) return fail(MA_E_INVALID, who + "momentum is NULL");
    if (hp->normuon && !x.row_v) return fail(MA_E_INVALID, who + "NorMuon needs row_v");
    const uintptr_t numel = static_cast<uintptr_t>(x.batch * x.rows * x.cols);
    const uintptr_t pb = reinterpret_cast<uintptr_t>(x.param);
    if (pb % dtype_size(x.param_dtype) || reinterpret_cast<uintptr_t>(x.grad) % dtype_size(x.grad_dtype))
      return fail(MA_E_INVALID, who + "param/grad not aligned to their element size");
    ranges.push_back({pb, pb + numel * dtype_size(x.param_dtype), i, "param"});
    if (!ns_only) {
      const uintptr_t mb = reinterpret_cast<uintptr_t>(x.momentum);
      if (mb % 4) return fail(MA_E_INVALID, who + "momentum not 4-byte aligned");
      ranges.push_back({mb, mb + numel * 4, i, "momentum"});
    }
    if (hp->normuon) {
      const uintptr_t vb = reinterpret_cast<uintptr_t>(x.row_v);
      if (vb % 4) return fail(MA_E_INVALID, who + "row_v not 4-byte aligned");
      ranges.push_back({vb, vb + static_cast<uintptr_t>(x.batch * x.rows) * 4, i, "row_v"});
    }
  }
  if (!ns_only) {
    st = check_overlaps(ranges);
    if (st != MA_OK) return st;
  }
  return MA_OK;
}

// Builds the plan of a validated list: the matrices, their buckets, the
// launch tables and the workspace layout. It depends only on the list's
// structure (which tensors have gradients, their shapes and views), the
// Newton-Schulz dtype and step count and the coefficients, which is what
// plan_key() below captures.
ma_status structure_plan(const ma_muon_tensor* t, int32_t n, const ma_muon_hparams* hp, Plan& P) {
  P = Plan();
  P.ns_dt = hp->ns_dtype;
  P.gemm_tile = hp->ns_dtype == MA_BF16 ? kNsTileBf16 : kNsTileF32;

  // Expand into matrices, canonicalise, bucket.
  std::map<std::pair<int, int>, int> buckets;
  for (int i = 0; i < n; ++i) {
    const ma_muon_tensor& x = t[i];
    if (!x.grad) continue;
    const int m = static_cast<int>(x.rows / x.views), nn = static_cast<int>(x.cols);
    for (int64_t b = 0; b < x.batch; ++b)
      for (int v = 0; v < x.views; ++v) {
        MatPlan mp{};
        mp.tensor = i;
        mp.bidx = static_cast<int>(b);
        mp.view = v;
        mp.m = m;
        mp.n = nn;
        mp.tall = m > nn;
        mp.r = std::min(m, nn);
        mp.c = std::max(m, nn);
        mp.rp = static_cast<int>(round_up(mp.r, kPad));
        mp.cp = static_cast<int>(round_up(mp.c, kPad));
        mp.scale = static_cast<float>(std::sqrt(std::max(1.0, static_cast<double>(m) / nn)));
        mp.elem_off = b * x.rows * x.cols + static_cast<int64_t>(v) * m * x.cols;
        mp.rowv_off = b * x.rows + static_cast<int64_t>(v) * m;
        mp.ntile_ew = (mp.rp / kEw) * (mp.cp / kEw);
        auto key = std::make_pair(mp.r, mp.c);
        auto it = buckets.find(key);
        if (it == buckets.end()) it = buckets.emplace(key, static_cast<int>(buckets.size())).first;
        mp.bucket = it->second;
        if (static_cast<int64_t>(mp.rp) * mp.cp > (int64_t(1) << 31) - 1)
          return fail(MA_E_UNSUPPORTED, "tensor " + std::to_string(i) + ": matrix too large");
        P.mats.push_back(mp);
      }
  }
  P.nbuckets = static_cast<int>(buckets.size());
  const int nm = static_cast<int>(P.mats.size());
  if (nm > (1 << 22)) return fail(MA_E_UNSUPPORTED, "too many matrices in one call");

  // Tile maps.
  const int T = P.gemm_tile;
  std::vector<Item> ew, fin, gram, sq, app, rows_nt, cols_t, rows_t, cols_nt, out;
  int64_t tot_ew = 0, tot_sym = 0, tot_app = 0, tot_out = 0;
  for (int k = 0; k < nm; ++k) {
    const MatPlan& mp = P.mats[k];
    const int nt = (mp.rp + T - 1) / T, ntc = (mp.cp + T - 1) / T;
    ew.push_back({k, mp.ntile_ew, 0});
    fin.push_back({k, 1, 0});
    gram.push_back({k, nt * (nt + 1) / 2, mp.cp});  // per-tile work ~ contraction length
    sq.push_back({k, nt * (nt + 1) / 2, mp.rp});
    app.push_back({k, nt * ntc, mp.rp});
    const int rows_blocks = (mp.r + 3) / 4, col_blocks = (mp.c + 63) / 64;
    if (mp.tall) { cols_t.push_back({k, col_blocks, 0}); rows_t.push_back({k, rows_blocks, 0}); }
    else { rows_nt.push_back({k, rows_blocks, 0}); cols_nt.push_back({k, col_blocks, 0}); }
    out.push_back({k, ((mp.m + kEw - 1) / kEw) * ((mp.n + kEw - 1) / kEw), 0});
    tot_ew += mp.ntile_ew;
    tot_sym += nt * (nt + 1) / 2;
    tot_app += static_cast<int64_t>(nt) * ntc;
    tot_out += static_cast<int64_t>((mp.m + kEw - 1) / kEw) * ((mp.n + kEw - 1) / kEw);
  }
  const int64_t kMaxGrid = (int64_t(1) << 31) - 1;
  if (tot_ew > kMaxGrid || tot_sym > kMaxGrid || tot_app > kMaxGrid || tot_out > kMaxGrid)
    return fail(MA_E_UNSUPPORTED, "step too large for one launch");
  P.ew = add_map(P, ew);
  P.fin_all = add_map(P, fin);
  if (hp->ns_dtype == MA_BF16) {
    // One XCD per matrix for all three GEMMs: longest total work first onto
    // the least-loaded XCD.
    std::vector<int64_t> work(nm);
    for (int k = 0; k < nm; ++k)
      work[k] = gram[k].key * gram[k].tiles + sq[k].key * sq[k].tiles + app[k].key * app[k].tiles;
    std::vector<int> order(nm), xcd_of(nm, 0);
    for (int k = 0; k < nm; ++k) order[k] = k;
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return work[a] > work[b]; });
    int64_t load[kXcds] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int k : order) {
      int b = 0;
      for (int x = 1; x < kXcds; ++x)
        if (load[x] < load[b]) b = x;
      xcd_of[k] = b;
      load[b] += work[k];
    }
    P.gram = add_map(P, gram, &xcd_of);
    P.sq = add_map(P, sq, &xcd_of);
    P.app = add_map(P, app, &xcd_of);
    // Queues of the persistent launch: per XCD, segments in (iteration,
    // product, matrix) order, matrices longest first; a segment needs every
    // earlier product of its matrix complete. They are built whenever the
    // launch could be used, so the workspace size does not depend on the
    // device or on the schedule a call takes.
    if (nm <= kMaxPersistMats) {
      P.persist = true;
      while (P.ints.size() % 4) P.ints.push_back(0);
      P.segs_off = P.ints.size() * sizeof(int32_t);
      int32_t nrec = 0;
      for (int x = 0; x < kXcds; ++x) {
        std::vector<int> ms;
        for (int k : order)
          if (xcd_of[k] == x) ms.push_back(k);
        P.seg_off[x] = nrec;
        int32_t start = 0;
        for (int it = 0; it < hp->ns_steps; ++it)
          for (int op = 0; op < 3; ++op)
            for (int k : ms) {
              const int g = gram[k].tiles, q2 = sq[k].tiles, a = app[k].tiles;
              const int tiles = op == 0 ? g : (op == 1 ? q2 : a);
              const int64_t need = static_cast<int64_t>(it) * (g + q2 + a) + (op >= 1 ? g : 0) + (op >= 2 ? q2 : 0);
              if (need > INT32_MAX || static_cast<int64_t>(start) + tiles > INT32_MAX)
                return fail(MA_E_UNSUPPORTED, "Newton-Schulz task queue too long");
              P.ints.insert(P.ints.end(), {k, it * 4 + op, start, static_cast<int32_t>(need)});
              start += tiles;
              ++nrec;
            }
        P.ints.insert(P.ints.end(), {0, 0, start, 0});   // sentinel: queue length
        P.nseg[x] = nrec - P.seg_off[x];
        ++nrec;
      }
      P.counter_ints = 8 * 32 + 32 + nm * 32;
    }
  } else {
    P.gram = add_map(P, gram);
    P.sq = add_map(P, sq);
    P.app = add_map(P, app);
  }
  P.rows_nt = add_map(P, rows_nt);
  P.cols_t = add_map(P, cols_t);
  P.rows_t = add_map(P, rows_t);
  P.cols_nt = add_map(P, cols_nt);
  P.out = add_map(P, out);
  // the (a, b, c) of every iteration, as float bits
  P.coefs_off = P.ints.size() * sizeof(int32_t);
  for (int it = 0; it < hp->ns_steps; ++it)
    for (int k = 0; k < 3; ++k) {
      const float f = ns_coef(hp, it, k);
      int32_t bits;
      std::memcpy(&bits, &f, 4);
      P.ints.push_back(bits);
    }

  // Workspace layout: [status header][MatDesc x nm][int tables] then
  // per-matrix buffers. The header and the tables are uploaded together at
  // the start of every call, which also clears the status word.
  P.desc_bytes = align_up(sizeof(MatDesc) * std::max(nm, 1));
  P.table_bytes = kHeaderBytes + P.desc_bytes + align_up(P.ints.size() * sizeof(int32_t));
  size_t off = P.table_bytes;
  const size_t es = dtype_size(hp->ns_dtype);
  for (MatPlan& mp : P.mats) {
    const size_t xb = align_up(static_cast<size_t>(mp.rp) * mp.cp * es);
    const size_t ab = align_up(static_cast<size_t>(mp.rp) * mp.rp * es);
    mp.off_x0 = off; off += xb;
    mp.off_x1 = off; off += xb;
    mp.off_a = off; off += ab;
    mp.off_b = off; off += ab;
    mp.off_part = off; off += align_up(static_cast<size_t>(mp.ntile_ew) * sizeof(double));
    mp.off_stat = off; off += kAlign;
    mp.off_csr = off; off += align_up(static_cast<size_t>(mp.rp) * 4);
    mp.off_csc = off; off += align_up(static_cast<size_t>(mp.cp) * 4);
    mp.off_rf = off; off += align_up(static_cast<size_t>(mp.m) * 4);
    mp.off_cf = off; off += align_up(static_cast<size_t>(mp.n) * 4);
  }
  if (P.persist) {
    P.off_counters = off;
    off += align_up(static_cast<size_t>(P.counter_ints) * sizeof(int32_t));
  }
  P.ws_bytes = off;
  return MA_OK;
}

// Plan cache. A training loop calls muon_step with the same tensor list every
// step; its plan (expansion, buckets, tile maps, queues, layout) is built once
// and kept, keyed by what structure_plan() reads. Validation still runs on
// every call, and the descriptors (pointers, lr, wd) are filled per call.
std::vector<int64_t> plan_key(const ma_muon_tensor* t, int32_t n, const ma_muon_hparams* hp) {
  std::vector<int64_t> k;
  k.reserve(4 + 4 * static_cast<size_t>(n) + 3 * static_cast<size_t>(hp->ns_steps));
  k.push_back(n);
  k.push_back(hp->ns_dtype);
  k.push_back(hp->ns_steps);
  for (int i = 0; i < n; ++i) {
    if (!t[i].grad) {   // contributes no matrix
      k.push_back(-1);
      continue;
    }
    k.push_back(t[i].batch);
    k.push_back(t[i].rows);
    k.push_back(t[i].cols);
    k.push_back(t[i].views);
  }
  for (int it = 0; it < hp->ns_steps; ++it)
    for (int c = 0; c < 3; ++c) {
      const float f = ns_coef(hp, it, c);
      int32_t bits;
      std::memcpy(&bits, &f, 4);
      k.push_back(bits);
    }
  return k;
}

constexpr size_t kMaxCachedPlans = 64;
std::mutex g_plan_mu;
std::map<std::vector<int64_t>, std::shared_ptr<const Plan>> g_plans;

// Validates the call and returns its plan, from the cache when the structure
// has been seen before.
ma_status get_plan(const ma_muon_tensor* t, int32_t n, const ma_muon_hparams* hp, bool ns_only,
                   std::shared_ptr<const Plan>& out) {
  ma_status st = validate_tensors(t, n, hp, ns_only);
  if (st != MA_OK) return st;
  std::vector<int64_t> key = plan_key(t, n, hp);
  {
    std::lock_guard<std::mutex> lk(g_plan_mu);
    auto it = g_plans.find(key);
    if (it != g_plans.end()) {
      out = it->second;
      return MA_OK;
    }
  }
  auto P = std::make_shared<Plan>();
  st = structure_plan(t, n, hp, *P);
  if (st != MA_OK) return st;
  std::lock_guard<std::mutex> lk(g_plan_mu);
  if (g_plans.size() >= kMaxCachedPlans) g_plans.clear();
  g_plans.emplace(std::move(key), P);
  out = P;
  return MA_OK;
}

// The persistent Newton-Schulz launch deals one task queue to each of 8 XCDs
// and a block serves the queue of the XCD it runs on (XCC_ID), 32 blocks of
// one CU each per XCD. It runs only on a device that reports 8 XCDs and at
// least 256 CUs (an MI355X as one device); elsewhere, say on a partition of
// the chip, the per-launch schedule runs instead. Cached per device.
std::mutex g_topo_mu;
std::map<int, bool> g_topo;

bool device_runs_persistent() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  std::lock_guard<std::mutex> lk(g_topo_mu);
  auto it = g_topo.find(dev);
  if (it != g_topo.end()) return it->second;
  int cus = 0, xccs = 0;
  bool ok = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
            cus >= kXcds * kPersistBlocksPerXcd;
  if (ok && hipDeviceGetAttribute(&xccs, hipDeviceAttributeNumberOfXccs, dev) == hipSuccess) ok = xccs == kXcds;
  (void)hipGetLastError();   // a runtime without the XCC attribute leaves no error behind
  g_topo[dev] = ok;
  return ok;
}

bool env_is(const char* name, const char* value) {
  const char* v = std::getenv(name);
  return v && std::string(v) == value;
}

TileMap device_map(const MapRef& r, char* tables, size_t desc_bytes) {
  TileMap tm;
  tm.start = reinterpret_cast<const int32_t*>(tables + desc_bytes + r.start_off);
  tm.perm = reinterpret_cast<const int32_t*>(tables + desc_bytes + r.perm_off);
  tm.nmat = r.nmat;
  tm.total = r.total;
  tm.grid = r.grid;
  tm.xcd = r.xcd;
  for (int x = 0; x < 8; ++x) {
    tm.xbase[x] = r.xbase[x];
    tm.xcnt[x] = r.xcnt[x];
  }
  return tm;
}

// Pinned staging buffers for the launch tables. A buffer is reused once the
// copy it last fed has completed (its event has fired); while none has, a new
// one joins the pool, up to kMaxStaging per device, so the host waits for the
// device only when it runs that many calls ahead of it.
struct Staging {
  void* host = nullptr;
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  bool used = false;
};
struct DevState {
  std::vector<Staging> pool;
  size_t next = 0;
};
constexpr size_t kMaxStaging = 64;
std::mutex g_mu;
std::map<int, DevState> g_dev;

ma_status upload(const std::vector<char>& host, void* dst, hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(MA_E_HIP, "hipGetDevice failed");
  std::lock_guard<std::mutex> lk(g_mu);
  DevState& ds = g_dev[dev];
  size_t pick = ds.pool.size();
  for (size_t k = 0; k < ds.pool.size() && pick == ds.pool.size(); ++k) {
    const size_t i = (ds.next + k) % ds.pool.size();
    Staging& c = ds.pool[i];
    if (!c.used) {
      pick = i;
      break;
    }
    const hipError_t q = hipEventQuery(c.ev);
    if (q == hipSuccess) pick = i;
    else if (q != hipErrorNotReady) return fail(MA_E_HIP, "staging event query failed");
  }
  if (pick == ds.pool.size()) {
    if (ds.pool.size() < kMaxStaging) {
      ds.pool.emplace_back();
    } else {   // every buffer still in flight: wait for the oldest
      pick = ds.next % ds.pool.size();
      if (hipEventSynchronize(ds.pool[pick].ev) != hipSuccess) return fail(MA_E_HIP, "staging event wait failed");
    }
  }
  ds.next = pick + 1;
  Staging& st = ds.pool[pick];
  if (st.cap < host.size()) {
    if (st.host) (void)hipHostFree(st.host);
    st.host = nullptr;
    st.cap = 0;
    if (hipHostMalloc(&st.host, host.size(), hipHostMallocDefault) != hipSuccess)
      return fail(MA_E_HIP, "pinned staging allocation failed");
    st.cap = host.size();
  }
  if (!st.ev && hipEventCreateWithFlags(&st.ev, hipEventDisableTiming) != hipSuccess)
    return fail(MA_E_HIP, "event creation failed");
  std::memcpy(st.host, host.data(), host.size());
  if (hipMemcpyAsync(dst, st.host, host.size(), hipMemcpyHostToDevice, s) != hipSuccess)
    return fail(MA_E_HIP, "table upload failed");
  if (hipEventRecord(st.ev, s) != hipSuccess) return fail(MA_E_HIP, "event record failed");
  st.used = true;
  return MA_OK;
}

// ---------------------------------------------------------------------------
// Optional per-kernel event timing (ma_profile_begin / ma_profile_end)
// ---------------------------------------------------------------------------
struct ProfRec {
  const char* name;
  hipEvent_t e0, e1;
};
struct ProfState {
  bool on = false;
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> pool;
};
thread_local ProfState g_prof;

hipEvent_t prof_event() {
  if (!g_prof.pool.empty()) {
    hipEvent_t e = g_prof.pool.back();
    g_prof.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs `launch`; when profiling, brackets it with events on `s`.
template <typename F>
void timed(const char* name, hipStream_t s, F&& launch) {
  if (!g_prof.on) {
    launch();
    return;
  }
  ProfRec r{name, prof_event(), prof_event()};
  if (r.e0) (void)hipEventRecord(r.e0, s);
  launch();
  if (r.e1) (void)hipEventRecord(r.e1, s);
  if (r.e0 && r.e1) g_prof.recs.push_back(r);
}

// Fills the descriptors for a workspace at `ws` and enqueues the whole step.
ma_status run_plan(const Plan& P, const ma_muon_tensor* t, const ma_muon_hparams* hp, bool ns_only, void* ws,
                   hipStream_t s) {
  const int nm = static_cast<int>(P.mats.size());
  if (nm == 0) return MA_OK;
  char* base = static_cast<char*>(ws);
  char* tables = base + kHeaderBytes;   // descriptors, then the int tables
  // operand layout of SQUARE and APPLY: by size unless the environment
  // forces one (the results are the same bits either way)
  const int operands = env_is("MA_NS_OPERANDS", "kmajor") ? 1 : (env_is("MA_NS_OPERANDS", "rows") ? 2 : 0);
  std::vector<char> host(P.table_bytes, 0);   // the header (status word 0) and the tables
  MatDesc* D = reinterpret_cast<MatDesc*>(host.data() + kHeaderBytes);
  for (int k = 0; k < nm; ++k) {
    const MatPlan& mp = P.mats[k];
    const ma_muon_tensor& x = t[mp.tensor];
    const size_t pes = dtype_size(x.param_dtype), ges = dtype_size(x.grad_dtype);
    MatDesc& d = D[k];
    d.param = static_cast<char*>(x.param) + mp.elem_off * pes;
    d.grad = static_cast<const char*>(x.grad) + mp.elem_off * ges;
    d.mom = ns_only ? nullptr : x.momentum + mp.elem_off;
    d.row_v = (hp->normuon && x.row_v) ? x.row_v + mp.rowv_off : nullptr;
    d.m = mp.m; d.n = mp.n; d.r = mp.r; d.c = mp.c; d.rp = mp.rp; d.cp = mp.cp;
    d.tall = mp.tall;
    d.pdt = x.param_dtype;
    d.gdt = x.grad_dtype;
    const uintptr_t al = reinterpret_cast<uintptr_t>(d.param) | reinterpret_cast<uintptr_t>(d.grad) |
                         reinterpret_cast<uintptr_t>(d.mom);
    d.vec = (mp.n % 4 == 0) && (al % 16 == 0);
    const double lr = x.lr, wd = x.weight_decay;
    d.decay = static_cast<float>(1.0 - lr * wd);
    d.lrwd = static_cast<float>(lr * wd);
    d.step = static_cast<float>(lr * mp.scale);
    d.scale = mp.scale;
    d.x0 = base + mp.off_x0;
    d.x1 = base + mp.off_x1;
    d.a = base + mp.off_a;
    d.b = base + mp.off_b;
    d.part = reinterpret_cast<double*>(base + mp.off_part);
    d.stat = reinterpret_cast<float*>(base + mp.off_stat);
    d.csum_r = reinterpret_cast<float*>(base + mp.off_csr);
    d.csum_c = reinterpret_cast<float*>(base + mp.off_csc);
    d.rfac = reinterpret_cast<float*>(base + mp.off_rf);
    d.cfac = reinterpret_cast<float*>(base + mp.off_cf);
    d.ntile_ew = mp.ntile_ew;
    d.clip = ns_only ? nullptr : hp->clip;
    d.kmajor = operands == 1 || (operands == 0 && mp.rp <= kKmajorMaxRows);
  }
  std::memcpy(host.data() + kHeaderBytes + P.desc_bytes, P.ints.data(), P.ints.size() * sizeof(int32_t));
  ma_status st = upload(host, ws, s);
  if (st != MA_OK) return st;

  const MatDesc* mats = reinterpret_cast<const MatDesc*>(tables);
  auto TM = [&](const MapRef& r) { return device_map(r, tables, P.desc_bytes); };
  const float beta = static_cast<float>(hp->beta);
  const float omb = static_cast<float>(1.0 - hp->beta);
  (void)hipGetLastError();
  const int ew_dt = P.ns_dt;
  timed("momentum", s, [&] { launch_momentum(mats, TM(P.ew), ew_dt, beta, omb, hp->nesterov, s); });
  timed("norm_finalize", s,
        [&] { launch_norm_finalize(mats, TM(P.fin_all), P.ns_dt, hp->ns_eps, ns_norm_scale(hp), s); });
  static const char* const kNsNames[2][3] = {{"ns_gram_f32", "ns_square_f32", "ns_apply_f32"},
                                             {"ns_gram_bf16", "ns_square_bf16", "ns_apply_bf16"}};
  const int bf = P.ns_dt == MA_BF16;
  // the persistent schedule unless the device cannot run it or the
  // environment asks for one launch per product (MA_NS_SCHEDULE=launches)
  const bool persist = P.persist && !env_is("MA_NS_SCHEDULE", "launches") && device_runs_persistent();
  if (persist) {
    NsQueue q;
    q.segs = reinterpret_cast<const int4*>(tables + P.desc_bytes + P.segs_off);
    q.qhead = reinterpret_cast<int*>(base + P.off_counters);
    q.err = q.qhead + 8 * 32;
    q.count = q.err + 32;
    q.status = reinterpret_cast<int*>(base);
    for (int x = 0; x < 8; ++x) {
      q.seg_off[x] = P.seg_off[x];
      q.nseg[x] = P.nseg[x];
    }
    q.coefs = reinterpret_cast<const float*>(tables + P.desc_bytes + P.coefs_off);
    q.clip = ns_only ? nullptr : hp->clip;
    timed("ns_persistent_bf16", s, [&] { launch_ns_persistent(mats, q, P.counter_ints, s); });
    timed("ns_status", s, [&] { launch_ns_status(q, s); });
  }
  for (int it = 0; it < (persist ? 0 : hp->ns_steps); ++it) {
    for (int op = NS_GRAM; op <= NS_APPLY; ++op) {
      const TileMap tm = TM(op == NS_APPLY ? P.app : (op == NS_GRAM ? P.gram : P.sq));
      timed(kNsNames[bf][op], s, [&] {
        const float a = ns_coef(hp, it, 0), b = ns_coef(hp, it, 1), c = ns_coef(hp, it, 2);
        if (bf)
          launch_ns_bf16(op, mats, tm, it & 1, it == 0, a, b, c, s);
        else
          launch_ns_f32(op, mats, tm, it & 1, it == 0, a, b, c, s);
      });
    }
  }
  const int src = hp->ns_steps & 1;  // buffer holding the final output
  int use_rf = 0, use_cf = 0;
  if (!ns_only && (hp->normuon || hp->muon_plus)) {
    if (P.rows_nt.nmat) timed("rowsum", s, [&] { launch_canon_rowsum(mats, TM(P.rows_nt), P.ns_dt, src, 0, s); });
    if (P.cols_t.nmat) timed("colsum", s, [&] { launch_canon_colsum(mats, TM(P.cols_t), P.ns_dt, src, 0, s); });
  }
  if (!ns_only && hp->normuon) {
    timed("finalize_normuon", s, [&] { launch_finalize_normuon(mats, TM(P.fin_all), static_cast<float>(1.0 - hp->normuon_beta2), s); });
    use_rf = 1;
  }
  if (!ns_only && hp->muon_plus) {
    timed("finalize_muon_plus", s,
          [&] { launch_finalize_muon_plus(mats, TM(P.fin_all), 1, hp->muon_plus_eps, s); });
    if (P.cols_nt.nmat) timed("colsum", s, [&] { launch_canon_colsum(mats, TM(P.cols_nt), P.ns_dt, src, 1, s); });
    if (P.rows_t.nmat) timed("rowsum", s, [&] { launch_canon_rowsum(mats, TM(P.rows_t), P.ns_dt, src, 1, s); });
    timed("finalize_muon_plus", s,
          [&] { launch_finalize_muon_plus(mats, TM(P.fin_all), 2, hp->muon_plus_eps, s); });
    use_rf = use_cf = 1;
  }
  timed(ns_only ? "copy_out" : "apply_update", s, [&] {
    launch_apply(mats, TM(P.out), P.ns_dt, src, ns_only ? APPLY_COPY : APPLY_UPDATE, ns_only ? 0 : hp->cautious,
                 use_rf, use_cf, s);
  });
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MA_E_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return MA_OK;
}

ma_status check_workspace(const Plan& P, void* ws, size_t bytes) {
  if (P.mats.empty()) return MA_OK;
  if (!ws) return fail(MA_E_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return fail(MA_E_WORKSPACE, "workspace must be 256-byte aligned");
  if (bytes < P.ws_bytes)
    return fail(MA_E_WORKSPACE, "workspace too small: " + std::to_string(bytes) + " < " + std::to_string(P.ws_bytes));
  return MA_OK;
}

ma_muon_tensor ns_tensor(const void* in, void* out, int64_t batch, int64_t rows, int64_t cols, int32_t dtype) {
  ma_muon_tensor x{};
  x.param = out;
  x.grad = in;
  x.batch = batch;
  x.rows = rows;
  x.cols = cols;
  x.views = 1;
  x.param_dtype = dtype;
  x.grad_dtype = dtype;
  return x;
}

ma_muon_hparams ns_hparams(const ma_muon_hparams* hp) {
  ma_muon_hparams h = *hp;
  h.normuon = 0;
  h.muon_plus = 0;
  h.cautious = 0;
  h.clip = nullptr;
  return h;
}

}  // namespace

extern "C" {

const char* ma_last_error(void) { return g_err.c_str(); }

size_t ma_muon_workspace_bytes(const ma_muon_tensor* tensors, int32_t n, const ma_muon_hparams* hp) {
  std::shared_ptr<const Plan> P;
  if (get_plan(tensors, n, hp, false, P) != MA_OK) return 0;
  return P->mats.empty() ? 0 : P->ws_bytes;
}

ma_status muon_step(const ma_muon_tensor* tensors, int32_t n, const ma_muon_hparams* hp, void* workspace,
                    size_t workspace_bytes, void* stream) {
  std::shared_ptr<const Plan> P;
  ma_status st = get_plan(tensors, n, hp, false, P);
  if (st != MA_OK) return st;
  st = check_workspace(*P, workspace, workspace_bytes);
  if (st != MA_OK) return st;
  return run_plan(*P, tensors, hp, false, workspace, static_cast<hipStream_t>(stream));
}

size_t ma_newton_schulz_workspace_bytes(int64_t batch, int64_t rows, int64_t cols, int32_t dtype,
                                        const ma_muon_hparams* hp) {
  if (!hp) {
    g_err = "hparams is NULL";
    return 0;
  }
  alignas(16) static const char dummy[16] = {0};
  ma_muon_tensor x = ns_tensor(dummy, const_cast<char*>(dummy), batch, rows, cols, dtype);
  ma_muon_hparams h = ns_hparams(hp);
  std::shared_ptr<const Plan> P;
  if (get_plan(&x, 1, &h, true, P) != MA_OK) return 0;
  return P->ws_bytes;
}

ma_status ma_newton_schulz(const void* in, void* out, int64_t batch, int64_t rows, int64_t cols, int32_t dtype,
                           const ma_muon_hparams* hp, void* workspace, size_t workspace_bytes, void* stream) {
  if (!hp) return fail(MA_E_INVALID, "hparams is NULL");
  if (!in || !out) return fail(MA_E_INVALID, "in/out is NULL");
  ma_muon_tensor x = ns_tensor(in, out, batch, rows, cols, dtype);
  ma_muon_hparams h = ns_hparams(hp);
  std::shared_ptr<const Plan> P;
  ma_status st = get_plan(&x, 1, &h, true, P);
  if (st != MA_OK) return st;
  st = check_workspace(*P, workspace, workspace_bytes);
  if (st != MA_OK) return st;
  return run_plan(*P, &x, &h, true, workspace, static_cast<hipStream_t>(stream));
}

ma_status ma_muon_step_status(const void* workspace, int32_t* status, void* stream) {
  if (!workspace || !status) return fail(MA_E_INVALID, "workspace and status must not be NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return fail(MA_E_WORKSPACE, "workspace must be 256-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  int32_t v = 0;
  if (hipMemcpyAsync(&v, workspace, sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess)
    return fail(MA_E_HIP, "status read failed");
  if (hipStreamSynchronize(s) != hipSuccess) return fail(MA_E_HIP, "stream synchronisation failed");
  *status = v;
  return MA_OK;
}

ma_status ma_muon_plan_counts(const ma_muon_tensor* tensors, int32_t n, const ma_muon_hparams* hp,
                              int32_t* n_matrices, int32_t* n_buckets) {
  std::shared_ptr<const Plan> P;
  ma_status st = get_plan(tensors, n, hp, false, P);
  if (st != MA_OK) return st;
  if (n_matrices) *n_matrices = static_cast<int32_t>(P->mats.size());
  if (n_buckets) *n_buckets = P->nbuckets;
  return MA_OK;
}

ma_status ma_muon_matrix_info(const ma_muon_tensor* tensors, int32_t n, const ma_muon_hparams* hp, int32_t k,
                              ma_matrix_info* info) {
  if (!info) return fail(MA_E_INVALID, "info is NULL");
  std::shared_ptr<const Plan> P;
  ma_status st = get_plan(tensors, n, hp, false, P);
  if (st != MA_OK) return st;
  if (k < 0 || k >= static_cast<int32_t>(P->mats.size())) return fail(MA_E_INVALID, "matrix index out of range");
  const MatPlan& mp = P->mats[k];
  std::memset(info, 0, sizeof(*info));
  info->tensor = mp.tensor;
  info->batch_index = mp.bidx;
  info->view = mp.view;
  info->m = mp.m;
  info->n = mp.n;
  info->r = mp.r;
  info->c = mp.c;
  info->rp = mp.rp;
  info->cp = mp.cp;
  info->transposed = mp.tall;
  info->bucket = mp.bucket;
  info->scale = mp.scale;
  info->u_offset = (hp->ns_steps & 1) ? mp.off_x1 : mp.off_x0;
  info->a_offset = mp.off_a;
  info->b_offset = mp.off_b;
  return MA_OK;
}

ma_status ma_muon_queue_info(const ma_muon_tensor* tensors, int32_t n, const ma_muon_hparams* hp,
                             int32_t* nseg, int32_t* segs, int32_t max_segs) {
  if (!nseg) return fail(MA_E_INVALID, "nseg is NULL");
  if (max_segs < 0 || (max_segs > 0 && !segs)) return fail(MA_E_INVALID, "segs is NULL or max_segs is negative");
  std::shared_ptr<const Plan> P;
  ma_status st = get_plan(tensors, n, hp, false, P);
  if (st != MA_OK) return st;
  int32_t w = 0;
  for (int x = 0; x < kXcds; ++x) {
    nseg[x] = P->persist ? P->nseg[x] : 0;
    if (!nseg[x]) continue;
    const int32_t* rec = P->ints.data() + P->segs_off / sizeof(int32_t) + 4 * static_cast<size_t>(P->seg_off[x]);
    for (int i = 0; i < nseg[x]; ++i, ++w)
      if (w < max_segs) std::memcpy(segs + 4 * static_cast<size_t>(w), rec + 4 * i, 4 * sizeof(int32_t));
  }
  return MA_OK;
}

ma_status ma_mfma_bf16_ceiling(float* sink, int32_t blocks, int32_t iters, void* stream) {
  if (!sink || reinterpret_cast<uintptr_t>(sink) % alignof(float))
    return fail(MA_E_INVALID, "sink must be a 4-byte aligned device pointer");
  if (blocks < 1 || blocks > (1 << 20)) return fail(MA_E_INVALID, "blocks must be in [1, 2^20]");
  if (iters < 1 || iters > (1 << 24)) return fail(MA_E_INVALID, "iters must be in [1, 2^24]");
  (void)hipGetLastError();
  launch_mfma_ceiling(sink, blocks, iters, static_cast<hipStream_t>(stream));
  if (hipGetLastError() != hipSuccess) return fail(MA_E_HIP, "ceiling kernel launch failed");
  return MA_OK;
}

ma_status ma_profile_begin(void) {
  for (ProfRec& r : g_prof.recs) {
    g_prof.pool.push_back(r.e0);
    g_prof.pool.push_back(r.e1);
  }
  g_prof.recs.clear();
  g_prof.on = true;
  return MA_OK;
}

int32_t ma_profile_end(ma_kernel_time* out, int32_t max) {
  g_prof.on = false;
  std::vector<std::string> names;
  std::vector<int64_t> counts;
  std::vector<double> totals;
  int32_t rc = 0;
  for (ProfRec& r : g_prof.recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.e1) != hipSuccess || hipEventElapsedTime(&ms, r.e0, r.e1) != hipSuccess) {
      g_err = "profiling event query failed";
      rc = -1;
      break;
    }
    size_t k = 0;
    while (k < names.size() && names[k] != r.name) ++k;
    if (k == names.size()) {
      names.push_back(r.name);
      counts.push_back(0);
      totals.push_back(0.0);
    }
    counts[k] += 1;
    totals[k] += ms;
  }
  for (ProfRec& r : g_prof.recs) {
    g_prof.pool.push_back(r.e0);
    g_prof.pool.push_back(r.e1);
  }
  g_prof.recs.clear();
  if (rc < 0) return rc;
  int32_t w = 0;
  for (size_t k = 0; k < names.size() && w < max && out; ++k, ++w) {
    std::memset(&out[w], 0, sizeof(out[w]));
    std::strncpy(out[w].name, names[k].c_str(), sizeof(out[w].name) - 1);
    out[w].launches = counts[k];
    out[w].total_ms = totals[k];
  }
  return w;
}

namespace {
// Blocks of the grad-norm pass for one gradient reference.
int64_t grad_norm_blocks(const ma_grad_ref& g) {
  if (!g.grad || g.numel <= 0) return 0;
  return (g.numel + kGradNormChunk - 1) / kGradNormChunk;
}
ma_status validate_grads(const ma_grad_ref* grads, int32_t n, int64_t& blocks) {
  blocks = 0;
  if (n < 0) return fail(MA_E_INVALID, "gradient count is negative");
  if (n > 0 && !grads) return fail(MA_E_INVALID, "gradient array is NULL");
  for (int i = 0; i < n; ++i) {
    const ma_grad_ref& g = grads[i];
    const std::string who = "gradient " + std::to_string(i) + ": ";
    if (!dtype_ok(g.dtype)) return fail(MA_E_DTYPE, who + "dtype must be MA_F32 or MA_BF16");
    if (g.numel < 0) return fail(MA_E_INVALID, who + "numel is negative");
    if (g.grad && reinterpret_cast<uintptr_t>(g.grad) % dtype_size(g.dtype))
      return fail(MA_E_INVALID, who + "not aligned to its element size");
    blocks += grad_norm_blocks(g);
  }
  if (blocks > (int64_t(1) << 30)) return fail(MA_E_UNSUPPORTED, "too many gradient elements");
  return MA_OK;
}
}  // namespace

size_t ma_grad_norm_workspace_bytes(const ma_grad_ref* grads, int32_t n) {
  int64_t blocks = 0;
  if (validate_grads(grads, n, blocks) != MA_OK) return 0;
  return align_up(static_cast<size_t>(std::max<int64_t>(blocks, 1)) * sizeof(double));
}

ma_status ma_global_grad_norm(const ma_grad_ref* grads, int32_t n, float max_norm, float* state, void* workspace,
                              size_t workspace_bytes, void* stream) {
  int64_t blocks = 0;
  ma_status st = validate_grads(grads, n, blocks);
  if (st != MA_OK) return st;
  if (!std::isfinite(max_norm)) return fail(MA_E_INVALID, "max_norm must be finite");
  if (!state || reinterpret_cast<uintptr_t>(state) % 16) return fail(MA_E_INVALID, "state must be a 16-byte aligned device pointer");
  const size_t need = align_up(static_cast<size_t>(std::max<int64_t>(blocks, 1)) * sizeof(double));
  if (!workspace) return fail(MA_E_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign) return fail(MA_E_WORKSPACE, "workspace must be 256-byte aligned");
  if (workspace_bytes < need)
    return fail(MA_E_WORKSPACE, "workspace too small: " + std::to_string(workspace_bytes) + " < " + std::to_string(need));
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  double* partial = static_cast<double*>(workspace);
  GradNormLaunch L{};
  L.partial = partial;
  int64_t done_blocks = 0, blocks_here = 0;
  auto flush = [&]() {
    if (L.nt == 0) return;
    L.block_start[L.nt] = static_cast<int32_t>(blocks_here);
    L.partial_off = static_cast<int32_t>(done_blocks);
    timed("grad_sumsq", s, [&] { launch_grad_sumsq(L, static_cast<int>(blocks_here), s); });
    done_blocks += blocks_here;
    blocks_here = 0;
    L.nt = 0;
  };
  for (int i = 0; i < n; ++i) {
    const int64_t nb = grad_norm_blocks(grads[i]);
    if (nb == 0) continue;
    GradNormArg& a = L.t[L.nt];
    a.g = grads[i].grad;
    a.numel = grads[i].numel;
    a.dt = grads[i].dtype;
    L.block_start[L.nt] = static_cast<int32_t>(blocks_here);
    blocks_here += nb;
    ++L.nt;
    if (L.nt == kMaxGradNormTensors) flush();
  }
  flush();
  timed("grad_norm_finalize", s,
        [&] { launch_grad_norm_finalize(partial, static_cast<int>(done_blocks), max_norm, state, s); });
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MA_E_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return MA_OK;
}

ma_status adamw_step(const ma_adamw_tensor* tensors, int32_t n, const ma_adamw_hparams* hp, void* stream) {
  if (!hp) return fail(MA_E_INVALID, "hparams is NULL");
  if (n < 0) return fail(MA_E_INVALID, "tensor count is negative");
  if (n > 0 && !tensors) return fail(MA_E_INVALID, "tensor array is NULL");
  if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0) || !(hp->beta2 >= 0.0 && hp->beta2 < 1.0))
    return fail(MA_E_INVALID, "betas must be in [0, 1)");
  if (!(hp->eps >= 0.0) || !std::isfinite(hp->eps)) return fail(MA_E_INVALID, "eps must be finite and >= 0");
  if (hp->step < 1) return fail(MA_E_INVALID, "step must be >= 1");
  if (hp->cautious == MA_CAUTIOUS_WD_MASK)
    return fail(MA_E_UNSUPPORTED, "the weight-decay mask is Muon's rule; AdamW takes none or the wrapper");
  if (hp->cautious != MA_CAUTIOUS_NONE && hp->cautious != MA_CAUTIOUS_WRAPPER)
    return fail(MA_E_INVALID, "cautious must be 0 (none) or 2 (wrapper)");
  if (reinterpret_cast<uintptr_t>(hp->clip) % 16) return fail(MA_E_INVALID, "clip state must be 16-byte aligned");
  std::vector<Range> ranges;
  for (int i = 0; i < n; ++i) {
    const ma_adamw_tensor& x = tensors[i];
    const std::string who = "tensor " + std::to_string(i) + ": ";
    if (!dtype_ok(x.param_dtype) || !dtype_ok(x.grad_dtype) || !dtype_ok(x.moment_dtype))
      return fail(MA_E_DTYPE, who + "param/grad/moment dtype must be MA_F32 or MA_BF16 (complex is not supported)");
    if (x.numel < 0) return fail(MA_E_INVALID, who + "numel is negative");
    if (!std::isfinite(x.lr) || !std::isfinite(x.weight_decay))
      return fail(MA_E_INVALID, who + "lr and weight_decay must be finite");
    if (!x.grad || x.numel == 0) continue;
    if (!x.param || !x.m || !x.v) return fail(MA_E_INVALID, who + "param, m and v must not be NULL");
    if (x.numel > (int64_t(1) << 40)) return fail(MA_E_UNSUPPORTED, who + "tensor too large");
    const uintptr_t pb = reinterpret_cast<uintptr_t>(x.param), mb = reinterpret_cast<uintptr_t>(x.m),
                    vb = reinterpret_cast<uintptr_t>(x.v);
    const size_t mes = dtype_size(x.moment_dtype);
    if (pb % dtype_size(x.param_dtype) || mb % mes || vb % mes ||
        reinterpret_cast<uintptr_t>(x.grad) % dtype_size(x.grad_dtype))
      return fail(MA_E_INVALID, who + "buffers not aligned to their element size");
    const uintptr_t ne = static_cast<uintptr_t>(x.numel);
    ranges.push_back({pb, pb + ne * dtype_size(x.param_dtype), i, "param"});
    ranges.push_back({mb, mb + ne * mes, i, "m"});
    ranges.push_back({vb, vb + ne * mes, i, "v"});
  }
  ma_status st = check_overlaps(ranges);
  if (st != MA_OK) return st;
  if (ranges.empty()) return MA_OK;  // nothing to step: no HIP call at all

  AdamLaunch L{};
  const double b1 = hp->beta1, b2 = hp->beta2;
  L.b1 = static_cast<float>(b1);
  L.omb1 = static_cast<float>(1.0 - b1);
  L.b2 = static_cast<float>(b2);
  L.omb2 = static_cast<float>(1.0 - b2);
  L.eps = static_cast<float>(hp->eps);
  L.inv_bc1 = static_cast<float>(1.0 / (1.0 - std::pow(b1, static_cast<double>(hp->step))));
  L.inv_sqrt_bc2 = static_cast<float>(1.0 / std::sqrt(1.0 - std::pow(b2, static_cast<double>(hp->step))));
  L.cautious = hp->cautious == MA_CAUTIOUS_WRAPPER;
  L.clip = hp->clip;
  // stochastic-rounding key of (tensor, moment): SplitMix64's output of the
  // seed mixed with (step, tensor, moment)
  auto sr_key = [&](int leaf, int moment) {
    const uint64_t c = (static_cast<uint64_t>(hp->step) << 32) + (static_cast<uint64_t>(leaf) << 1) +
                       static_cast<uint64_t>(moment);
    return splitmix64_mix(hp->seed ^ splitmix64_mix(c));
  };
  hipStream_t s = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  int64_t blocks = 0;
  auto flush = [&]() {
    if (L.nt == 0) return;
    L.block_start[L.nt] = static_cast<int32_t>(blocks);
    timed("adamw", s, [&] { launch_adamw(L, static_cast<int>(blocks), s); });
    L.nt = 0;
    blocks = 0;
  };
  for (int i = 0; i < n; ++i) {
    const ma_adamw_tensor& x = tensors[i];
    if (!x.grad || x.numel == 0) continue;
    int64_t nb = (x.numel + kAdamChunk - 1) / kAdamChunk;
    int64_t done = 0;
    while (nb > 0) {
      // split very large tensors so block indices stay in int32
      const int64_t room = (int64_t(1) << 30) - blocks;
      const int64_t take = std::min(nb, room);
      AdamTensorArg& a = L.t[L.nt];
      const size_t mes = dtype_size(x.moment_dtype);
      a.p = static_cast<char*>(x.param) + done * kAdamChunk * dtype_size(x.param_dtype);
      a.g = static_cast<const char*>(x.grad) + done * kAdamChunk * dtype_size(x.grad_dtype);
      a.m = static_cast<char*>(x.m) + done * kAdamChunk * mes;
      a.v = static_cast<char*>(x.v) + done * kAdamChunk * mes;
      a.numel = std::min(x.numel - done * kAdamChunk, take * kAdamChunk);
      a.index0 = done * kAdamChunk;
      a.key_m = sr_key(i, 0);
      a.key_v = sr_key(i, 1);
      a.pdt = x.param_dtype;
      a.gdt = x.grad_dtype;
      a.mdt = x.moment_dtype;
      a.lr = x.lr;
      a.wd = x.weight_decay;
      L.block_start[L.nt] = static_cast<int32_t>(blocks);
      blocks += take;
      ++L.nt;
      done += take;
      nb -= take;
      if (L.nt == kMaxAdamTensors || blocks >= (int64_t(1) << 30)) flush();
    }
  }
  flush();
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(MA_E_HIP, std::string("kernel launch failed: ") + hipGetErrorString(e));
  return MA_OK;
}

}  // extern "C"
