// C ABI of the fused linear cross-entropy library: argument checks, the
// execution plan, the stream-ordered workspace, the per-chunk kernel sequence
// and the timing instrumentation.
#include <hip/hip_runtime.h>

#include <climits>
#include <mutex>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <vector>

#include "flce.h"
#include "flce_internal.h"

namespace flce {

namespace {

constexpr size_t kAlign = 256;
constexpr size_t kDefaultProbBudget = size_t(1) << 30;  // bytes for the chunk's [C, vp] buffer
constexpr size_t kLowmemBudget = size_t(256) << 20;     // bytes for a vocabulary slice's [C, vb] buffer
constexpr int64_t kVocabPad = 256;
constexpr int64_t kMaxDim = int64_t(1) << 24;  // d <= 2^24, v <= 2^24 - 256
constexpr int64_t kMaxRows = INT32_MAX;         // n_valid is counted in 32 bits
constexpr int64_t kCus = 256;                   // compute units of an MI355X

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int64_t env_i64(const char* name, int64_t fallback) {
  const char* s = getenv(name);
  if (s == nullptr || *s == '\0') return fallback;
  char* end = nullptr;
  long long v = strtoll(s, &end, 10);
  if (end == s || v <= 0) return fallback;
  return static_cast<int64_t>(v);
}

bool mul_ok(int64_t a, int64_t b) { return a > 0 && b > 0 && a <= (int64_t(1) << 62) / b; }

}  // namespace

// The split count s in [1, smax] of a reduction over `tiles` output tiles that
// minimises ceil(tiles * s / slots) / s, the waves of `slots` concurrent
// workgroups per unit of reduction length; the smallest such s.
static int64_t best_splits(int64_t tiles, int64_t slots, int64_t smax) {
  int64_t best = 1;
  int64_t best_waves = (tiles + slots - 1) / slots;  // compare waves_s / s as waves_s * best <  best_waves * s
  for (int64_t s = 2; s <= smax; ++s) {
    const int64_t waves = (tiles * s + slots - 1) / slots;
    if (waves * best < best_waves * s) {
      best = s;
      best_waves = waves;
    }
  }
  return best;
}

// Chunk rows C: as many rows as the probability-buffer budget allows (a
// multiple of 256 rows once that many fit), never more than half of the rows
// (rounded up to 16) so that the buffer stays well below the [n, v] logits it
// replaces, and at least 16.
int make_plan(int64_t n, int64_t d, int64_t v, int32_t dtype, int32_t with_bwd, Plan* p, int allow_pair,
              int64_t budget_req, int whole_rows) {
  if (p == nullptr || n <= 0 || d <= 0 || v <= 0) return FLCE_ERR_INVALID_ARG;
  if (dtype != FLCE_BF16 && dtype != FLCE_F32) return FLCE_ERR_INVALID_ARG;
  if (!mul_ok(n, d) || !mul_ok(v, d) || v > (int64_t(1) << 40) || n > kMaxRows) return FLCE_ERR_INVALID_ARG;
  // Row strides (d, and v rounded up to 256) stay below 2^24 elements, so the
  // 32-bit offsets of the matrix engine's buffer loads cannot overflow.
  if (d > kMaxDim || v > kMaxDim - 256) return FLCE_ERR_INVALID_ARG;
  Plan q;
  memset(&q, 0, sizeof(q));
  q.n = n;
  q.d = d;
  q.v = v;
  q.dtype = dtype;
  q.with_bwd = with_bwd ? 1 : 0;
  q.engine = dtype == FLCE_BF16 ? ENGINE_MFMA : ENGINE_FMA;
  q.group = q.engine == ENGINE_MFMA ? 128 : 32;  // each engine's logits tile width along the vocabulary
  const int64_t prob_elem = q.engine == ENGINE_MFMA ? 2 : 4;
  q.vp = (v + kVocabPad - 1) / kVocabPad * kVocabPad;
  q.ngroups = (v + q.group - 1) / q.group;

  const int64_t budget =
      budget_req > 0 ? budget_req : env_i64("FLCE_WORKSPACE_CAP_BYTES", static_cast<int64_t>(kDefaultProbBudget));
  int64_t c_budget = budget / (q.vp * prob_elem);
  c_budget = c_budget >= 256 ? c_budget / 256 * 256 : (c_budget / 16) * 16;
  if (c_budget < 16) c_budget = 16;
  const int64_t half = ((n + 1) / 2 + 15) / 16 * 16;
  const int64_t c_cap = whole_rows ? n : half;
  int64_t c = c_budget < c_cap ? c_budget : c_cap;
  if (!with_bwd) {
    // No probability buffer: a forward-only chunk holds just its rows' group
    // partials (8 bytes per row and group), so it spans every row that fits
    // the same budget, and one launch covers the tokens of several chunks.
    int64_t c_fwd = budget / (q.ngroups * 8);
    c_fwd = c_fwd >= 256 ? c_fwd / 256 * 256 : (c_fwd / 16) * 16;
    if (c_fwd < 16) c_fwd = 16;
    c = c_fwd < n ? c_fwd : n;
  }
  c = env_i64("FLCE_CHUNK_ROWS", c);
  if (c > n) c = n;
  q.chunk = c;
  q.nchunks = (n + c - 1) / c;
  // dH = G.W has few output tiles (ceil(C/256) x ceil(d/256) on the matrix
  // engine, 64 x 32 tiles on the FMA engine); its vocabulary reduction is split
  // in s parts, s chosen by best_splits: the fewest waves of one workgroup per
  // CU (256 on MI355X) per unit of work.  Each split keeps at least 4096
  // (matrix engine) or 256 (FMA engine) vocabulary columns; splits cost fp32
  // partials and a reduction pass, so unsplit wins once the tiles fill the chip.
  q.dh_splits = 1;
  if (with_bwd) {
    const bool mfma = q.engine == ENGINE_MFMA;
    const int64_t tm = mfma ? 256 : 64, tn = mfma ? 256 : kFmaDhTileCols;
    const int64_t tiles = ((q.chunk + tm - 1) / tm) * ((d + tn - 1) / tn);
    int64_t smax = q.vp / (mfma ? 4096 : 256);
    if (smax > (mfma ? 8 : 16)) smax = mfma ? 8 : 16;
    // the fp32 partials ([S][C][d]) stay within the chunk buffer's bytes, and the
    // whole workspace below the fp32 [n, v] logits the method avoids (the chunk
    // buffer, the group partials and the per-row arrays taken into account)
    const int64_t part_bytes = q.chunk * d * 4;
    int64_t s_bytes = (q.chunk * q.vp * prob_elem) / part_bytes;
    const int64_t others = q.chunk * q.vp * prob_elem + 8 * q.ngroups * q.chunk + 16 * n + 16 * q.chunk + 4096;
    if (mul_ok(n, v) && n * v * 4 > others) {
      const int64_t s_fit = (n * v * 4 - others) / part_bytes;
      if (s_fit < s_bytes) s_bytes = s_fit;
    }
    if (smax > s_bytes) smax = s_bytes < 1 ? 1 : s_bytes;
    if (whole_rows) smax = 1;  // a vocabulary slice of the low-memory path: no partials
    int64_t s = best_splits(tiles, kCus, smax);
    s = env_i64("FLCE_DH_SPLITS", s);
    if (s > q.vp / 64) s = q.vp / 64;  // every split keeps at least one 64-column stage
    q.dh_splits = s < 1 ? 1 : s;
  }
  q.dw_acc = (with_bwd && dtype == FLCE_BF16 && q.nchunks > 1) ? 1 : 0;
  // Runs of four or more chunks keep two chunk buffers side by side, so that
  // one dW launch reduces over 2 C tokens: half the launches and half the
  // passes over the running sum, for one more chunk buffer.
  q.dw_pair = (allow_pair && q.dw_acc && q.nchunks >= env_i64("FLCE_DW_PAIR_CHUNKS", 4)) ? 1 : 0;
  // The one-pass backward of the matrix engine folds the softmax factor into a
  // per-row factor applied to dH's rows and to dW's token operand (a bf16 copy
  // of the chunk's H), where the vocabulary is wide enough for that copy to be
  // small next to the chunk buffer.
  const bool one_pass = with_bwd != 0 && with_bwd != 2;
  q.fold = (one_pass && q.engine == ENGINE_MFMA && q.vp >= 2 * d && env_i64("FLCE_INPLACE_GRAD", 0) == 0) ? 1 : 0;
  // Tile orders (see tile_coords): consecutive tiles share operand tiles in L2.
  q.group_m[0] = env_i64("FLCE_GROUP_LOGITS", 8);
  q.group_m[1] = env_i64("FLCE_GROUP_DH", 8);
  q.group_m[2] = env_i64("FLCE_GROUP_DW", 4);
  if (!mul_ok(q.chunk, q.vp) || !mul_ok(q.ngroups, q.chunk)) return FLCE_ERR_INVALID_ARG;

  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  q.off_nvalid = take(sizeof(int32_t));
  q.off_zy = take(sizeof(float) * q.chunk);
  q.off_gy = take(sizeof(float) * q.chunk);
  q.off_lse = take(sizeof(float) * n);
  q.off_loss = take(sizeof(float) * n);
  q.off_pm = take(sizeof(float) * q.ngroups * q.chunk);
  q.off_ps = take(sizeof(float) * q.ngroups * q.chunk);
  q.prob_bytes = with_bwd ? static_cast<size_t>(q.chunk * q.vp * prob_elem) * (q.dw_pair ? 2 : 1) : 0;
  q.off_prob = take(q.prob_bytes);
  q.off_dwacc = take(q.dw_acc ? sizeof(uint16_t) * static_cast<size_t>(v * d) : 0);
  q.off_dhpart = take(with_bwd && q.dh_splits > 1 ? sizeof(float) * q.dh_splits * q.chunk * d : 0);
  q.off_uref = take(q.fold ? sizeof(float) * q.chunk : 0);
  q.off_flag = take(q.fold ? sizeof(int32_t) * q.chunk : 0);
  q.off_rowf = take(q.fold ? sizeof(float) * static_cast<size_t>((q.chunk + 255) / 256 * 256) : 0);
  q.off_hs = take(q.fold ? sizeof(uint16_t) * static_cast<size_t>(q.chunk * d) * (q.dw_pair ? 2 : 1) : 0);
  q.total = off;
  *p = q;
  return FLCE_OK;
}

namespace {

// ---- library-owned stream-ordered memory pool, one per device --------------------

std::mutex g_pool_mu;
hipMemPool_t g_pools[64];
bool g_pool_init[64];

hipError_t device_pool(int dev, hipMemPool_t* out) {
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_pool_mu);
  if (!g_pool_init[dev]) {
    hipMemPoolProps props;
    memset(&props, 0, sizeof(props));
    props.allocType = hipMemAllocationTypePinned;
    props.handleTypes = hipMemHandleTypeNone;
    props.location.type = hipMemLocationTypeDevice;
    props.location.id = dev;
    hipMemPool_t pool;
    hipError_t e = hipMemPoolCreate(&pool, &props);
    if (e != hipSuccess) return e;
    uint64_t keep = UINT64_MAX;  // keep freed blocks cached for the next call
    e = hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep);
    if (e != hipSuccess) {
      (void)hipMemPoolDestroy(pool);
      return e;
    }
    g_pools[dev] = pool;
    g_pool_init[dev] = true;
  }
  *out = g_pools[dev];
  return hipSuccess;
}

// A stream-ordered workspace from the device's pool; false when it cannot be had.
// FLCE_TEST_ALLOC_LIMIT_BYTES (a test hook) makes every request above that many
// bytes fail here, before anything is enqueued, as a real allocation failure would.
bool pool_alloc(void** base, size_t bytes, hipMemPool_t pool, hipStream_t stream) {
  *base = nullptr;
  const int64_t limit = env_i64("FLCE_TEST_ALLOC_LIMIT_BYTES", 0);
  if (limit > 0 && bytes > static_cast<size_t>(limit)) return false;
  if (hipMallocFromPoolAsync(base, bytes, pool, stream) != hipSuccess || *base == nullptr) {
    (void)hipGetLastError();
    return false;
  }
  return true;
}

// ---- timing instrumentation -------------------------------------------------------

struct Prof {
  std::mutex mu;
  bool on = false;
  struct Pending {
    int kind;
    hipEvent_t a, b;
  };
  std::vector<Pending> pending;
  int64_t launches[K_NUM_KINDS] = {};
  double ms[K_NUM_KINDS] = {};
};
Prof g_prof;

const char* const kKindNames[K_NUM_KINDS] = {"label_scan", "logits_lse", "lse_merge",   "grad_inplace", "dh_gemm",
                                             "dh_reduce",  "dw_gemm",    "loss_reduce", "ce_rows",      "dequant_e4m3",
                                             "target_ref", "fold_patch"};

template <class F>
hipError_t timed(int kind, hipStream_t s, F&& launch) {
  if (!g_prof.on) return launch();
  hipEvent_t a = nullptr, b = nullptr;
  if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return hipErrorOutOfMemory;
  hipEventRecord(a, s);
  hipError_t e = launch();
  hipEventRecord(b, s);
  std::lock_guard<std::mutex> lk(g_prof.mu);
  g_prof.pending.push_back({kind, a, b});
  return e;
}

int status_of(hipError_t e) { return e == hipSuccess ? FLCE_OK : FLCE_ERR_HIP; }

bool aligned(const void* ptr, size_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

int check_common(const void* h, const void* w, const int64_t* labels, int64_t n, int64_t d, int64_t v,
                 flce_dtype dtype, flce_reduction reduction, const float* loss_out, const float* lse_out) {
  if (h == nullptr || w == nullptr || labels == nullptr || loss_out == nullptr) return FLCE_ERR_INVALID_ARG;
  if (n <= 0 || d <= 0 || v <= 0) return FLCE_ERR_INVALID_ARG;
  if (dtype != FLCE_BF16 && dtype != FLCE_F32) return FLCE_ERR_INVALID_ARG;
  if (reduction != FLCE_MEAN && reduction != FLCE_SUM) return FLCE_ERR_INVALID_ARG;
  const int64_t elem = dtype == FLCE_BF16 ? 2 : 4;
  if ((d * elem) % 16 != 0 || !aligned(h, 16) || !aligned(w, 16)) return FLCE_ERR_ALIGNMENT;
  if (!aligned(labels, 8) || !aligned(loss_out, 4) || (lse_out != nullptr && !aligned(lse_out, 4)))
    return FLCE_ERR_ALIGNMENT;
  return FLCE_OK;
}

Work carve(const Plan& p, char* base) {
  Work w;
  w.base = base;
  w.nvalid = reinterpret_cast<int32_t*>(base + p.off_nvalid);
  w.zy = reinterpret_cast<float*>(base + p.off_zy);
  w.gy = reinterpret_cast<float*>(base + p.off_gy);
  w.lse = reinterpret_cast<float*>(base + p.off_lse);
  w.loss_rows = reinterpret_cast<float*>(base + p.off_loss);
  w.pm = reinterpret_cast<float*>(base + p.off_pm);
  w.ps = reinterpret_cast<float*>(base + p.off_ps);
  w.prob = base + p.off_prob;
  w.dwlo = reinterpret_cast<uint16_t*>(base + p.off_dwacc);
  w.dhpart = reinterpret_cast<float*>(base + p.off_dhpart);
  w.uref = reinterpret_cast<float*>(base + p.off_uref);
  w.flag = reinterpret_cast<int32_t*>(base + p.off_flag);
  w.rowf = reinterpret_cast<float*>(base + p.off_rowf);
  w.hs = base + p.off_hs;
  return w;
}

// The workspace as chunk c sees it: with paired chunk buffers, odd chunks use
// the second buffer, which follows the first, so that a pair's gradient rows
// are one contiguous [2 C, vp] array.
Work chunk_work(const Plan& p, const Work& wk, int64_t c) {
  Work wc = wk;
  if (p.dw_pair && (c & 1)) {
    const size_t elem = p.engine == ENGINE_MFMA ? 2 : 4;
    wc.prob = static_cast<char*>(wk.prob) + static_cast<size_t>(p.chunk * p.vp) * elem;
    wc.hs = static_cast<char*>(wk.hs) + static_cast<size_t>(p.chunk * p.d) * sizeof(uint16_t);
  }
  return wc;
}

// dW after chunk c.  Unpaired: this chunk's contribution, first/middle/last by
// position.  Paired: after each odd chunk (and after an even last chunk), one
// launch over the group's rows, which start at the first buffer; the groups
// take the first/middle/last roles, and a plan pairs only from four chunks on,
// so there are always at least two groups.
hipError_t run_dw(const Plan& p, const Work& wk, const ChunkArgs& a, int64_t c, const char* h, int64_t elem,
                  hipStream_t s) {
  if (!p.dw_pair)
    return timed(K_DW, s, [&] { return p.engine == ENGINE_MFMA ? mfma_dw(p, wk, a, s) : fma_dw(p, wk, a, s); });
  if (!(c & 1) && c != p.nchunks - 1) return hipSuccess;  // the pair's first chunk: wait for its partner
  const int64_t first = c & ~int64_t(1);
  const int64_t group = first / 2, groups = (p.nchunks + 1) / 2;
  ChunkArgs ad = a;
  ad.row0 = first * p.chunk;
  ad.rows = a.row0 + a.rows - ad.row0;
  ad.h = h + ad.row0 * p.d * elem;
  ad.dw_mode = group == 0 ? DW_FIRST : (group == groups - 1 ? DW_LAST : DW_MID);
  return timed(K_DW, s, [&] { return mfma_dw(p, wk, ad, s); });
}

// The kernel sequence of one call; workspace already allocated.
// zy_out (optional): the per-row target logit (0 for ignored rows and for
// labels outside [0, v)); loss_out may be null when zy_out is given.
// h_scale / w_scale (optional, forward only): h and w hold e4m3 bytes, the
// plan's d counting byte pairs, and each row carries its own scale.
hipError_t run(const Plan& p, const Work& wk, const void* h, const void* w, const int64_t* labels,
               int64_t ignore_index, int32_t reduction, float* loss_out, float* lse_out, void* dh_out, void* dw_out,
               hipStream_t s, float* zy_out = nullptr, const float* h_scale = nullptr,
               const float* w_scale = nullptr) {
  const int64_t elem = p.dtype == FLCE_BF16 ? 2 : 4;
  hipError_t e = timed(K_LABEL_SCAN, s, [&] { return launch_label_scan(p, wk, labels, ignore_index, s); });
  if (e != hipSuccess) return e;
  float* lse_base = lse_out != nullptr ? lse_out : wk.lse;
  for (int64_t c = 0; c < p.nchunks; ++c) {
    const Work wc = chunk_work(p, wk, c);
    ChunkArgs a;
    a.row0 = c * p.chunk;
    a.rows = p.n - a.row0 < p.chunk ? p.n - a.row0 : p.chunk;
    a.h = static_cast<const char*>(h) + a.row0 * p.d * elem;
    a.w = w;
    a.labels = labels + a.row0;
    a.ignore_index = ignore_index;
    a.reduction = reduction;
    a.lse_rows = lse_base + a.row0;
    a.dh = dh_out != nullptr ? static_cast<char*>(dh_out) + a.row0 * p.d * elem : nullptr;
    a.dw = dw_out;
    a.dw_mode = p.nchunks == 1 ? DW_SINGLE : (c == 0 ? DW_FIRST : (c == p.nchunks - 1 ? DW_LAST : DW_MID));
    a.lse_in = nullptr;
    a.grad_out = nullptr;
    a.zy_rows = zy_out != nullptr ? zy_out + a.row0 : nullptr;
    a.dh_f32 = 0;
    a.dh_accumulate = 0;
    a.fp8 = h_scale != nullptr ? 1 : 0;
    a.h_scale = h_scale != nullptr ? h_scale + a.row0 : nullptr;
    a.w_scale = w_scale;
    a.fold = p.fold;

    if (a.fold) {
      e = timed(K_TARGET_REF, s, [&] { return launch_target_ref(p, wc, a, s); });
      if (e != hipSuccess) return e;
    }
    const int mode = p.with_bwd ? LOGITS_PROB : LOGITS_STATS;
    e = timed(K_LOGITS, s, [&] {
      return p.engine == ENGINE_MFMA ? mfma_logits(p, wc, a, mode, s) : fma_logits(p, wc, a, mode, s);
    });
    if (e != hipSuccess) return e;
    e = timed(K_LSE_MERGE, s, [&] { return launch_lse_merge(p, wc, a, p.with_bwd ? (a.fold ? 2 : 1) : 0, s); });
    if (e != hipSuccess) return e;
    if (!p.with_bwd) continue;
    if (a.fold)
      e = timed(K_FOLD_PATCH, s, [&] { return launch_fold_patch(p, wc, a, s); });
    else
      e = timed(K_GRAD, s, [&] { return launch_grad(p, wc, a, s); });
    if (e != hipSuccess) return e;
    e = timed(K_DH, s, [&] { return p.engine == ENGINE_MFMA ? mfma_dh(p, wc, a, s) : fma_dh(p, wc, a, s); });
    if (e != hipSuccess) return e;
    if (p.dh_splits > 1) {
      e = timed(K_DH_REDUCE, s, [&] { return launch_dh_reduce(p, wc, a, s); });
      if (e != hipSuccess) return e;
    }
    e = run_dw(p, wk, a, c, static_cast<const char*>(h), elem, s);
    if (e != hipSuccess) return e;
  }
  if (loss_out == nullptr) return hipSuccess;
  return timed(K_LOSS, s, [&] { return launch_loss_reduce(p, wk, reduction, loss_out, s); });
}

// The backward from the saved LSE (recompute): per chunk the logits are
// recomputed and their epilogue writes G directly; then dH and dW as above.
// dh_f32: dh_out is an fp32 array whatever the dtype (a vocabulary shard's dH partial);
// dh_accumulate: dh_out (fp32) already holds a partial sum, to which this call's dH is added.
hipError_t run_bwd(const Plan& p, const Work& wk, const void* h, const void* w, const int64_t* labels,
                   const float* lse, const float* grad_out, int64_t ignore_index, int32_t reduction, void* dh_out,
                   void* dw_out, hipStream_t s, int dh_f32 = 0, int dh_accumulate = 0) {
  const int64_t elem = p.dtype == FLCE_BF16 ? 2 : 4;
  const int64_t dh_elem = dh_f32 ? 4 : elem;
  hipError_t e = timed(K_LABEL_SCAN, s, [&] { return launch_label_scan(p, wk, labels, ignore_index, s); });
  if (e != hipSuccess) return e;
  for (int64_t c = 0; c < p.nchunks; ++c) {
    const Work wc = chunk_work(p, wk, c);
    ChunkArgs a;
    a.row0 = c * p.chunk;
    a.rows = p.n - a.row0 < p.chunk ? p.n - a.row0 : p.chunk;
    a.h = static_cast<const char*>(h) + a.row0 * p.d * elem;
    a.w = w;
    a.labels = labels + a.row0;
    a.ignore_index = ignore_index;
    a.reduction = reduction;
    a.lse_rows = nullptr;
    a.dh = static_cast<char*>(dh_out) + a.row0 * p.d * dh_elem;
    a.dw = dw_out;
    a.dw_mode = p.nchunks == 1 ? DW_SINGLE : (c == 0 ? DW_FIRST : (c == p.nchunks - 1 ? DW_LAST : DW_MID));
    a.lse_in = lse + a.row0;
    a.grad_out = grad_out;
    a.zy_rows = nullptr;
    a.dh_f32 = dh_f32;
    a.dh_accumulate = dh_accumulate;
    a.fp8 = 0;
    a.fold = 0;
    a.h_scale = nullptr;
    a.w_scale = nullptr;
    e = timed(K_LOGITS, s, [&] {
      return p.engine == ENGINE_MFMA ? mfma_logits(p, wc, a, LOGITS_GRAD_FROM_LSE, s)
                                     : fma_logits(p, wc, a, LOGITS_GRAD_FROM_LSE, s);
    });
    if (e != hipSuccess) return e;
    e = timed(K_DH, s, [&] { return p.engine == ENGINE_MFMA ? mfma_dh(p, wc, a, s) : fma_dh(p, wc, a, s); });
    if (e != hipSuccess) return e;
    if (p.dh_splits > 1) {
      e = timed(K_DH_REDUCE, s, [&] { return launch_dh_reduce(p, wc, a, s); });
      if (e != hipSuccess) return e;
    }
    e = run_dw(p, wk, a, c, static_cast<const char*>(h), elem, s);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Allocate the call's workspace from the device's pool, run `body`, free it.
template <class Body>
int with_workspace(const Plan& p, hipStream_t stream, Body&& body) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FLCE_ERR_HIP;
  hipMemPool_t pool;
  if (device_pool(dev, &pool) != hipSuccess) return FLCE_ERR_HIP;
  void* base = nullptr;
  if (!pool_alloc(&base, p.total, pool, stream)) return FLCE_ERR_OOM;
  const Work wk = carve(p, static_cast<char*>(base));
  hipError_t e = body(wk);
  hipError_t f = hipFreeAsync(base, stream);
  if (e != hipSuccess) return FLCE_ERR_HIP;
  return status_of(f);
}

int call(const void* h, const void* w, const int64_t* labels, int64_t n, int64_t d, int64_t v, flce_dtype dtype,
         int64_t ignore_index, flce_reduction reduction, float* loss_out, float* lse_out, void* dh_out,
         void* dw_out, hipStream_t stream, int with_bwd) {
  int st = check_common(h, w, labels, n, d, v, dtype, reduction, loss_out, lse_out);
  if (st != FLCE_OK) return st;
  if (with_bwd) {
    if (dh_out == nullptr || dw_out == nullptr) return FLCE_ERR_INVALID_ARG;
    if (!aligned(dh_out, 16) || !aligned(dw_out, 16)) return FLCE_ERR_ALIGNMENT;
  }
  Plan p;
  st = make_plan(n, d, v, dtype, with_bwd, &p);
  if (st != FLCE_OK) return st;
  return with_workspace(p, stream, [&](const Work& wk) {
    return run(p, wk, h, w, labels, ignore_index, reduction, loss_out, lse_out, dh_out, dw_out, stream);
  });
}

int call_bwd(const void* h, const void* w, const int64_t* labels, const float* lse, const float* grad_out, int64_t n,
             int64_t d, int64_t v, flce_dtype dtype, int64_t ignore_index, flce_reduction reduction, void* dh_out,
             void* dw_out, hipStream_t stream) {
  if (lse == nullptr || dh_out == nullptr || dw_out == nullptr) return FLCE_ERR_INVALID_ARG;
  // check_common wants a loss pointer; the saved LSE stands in (same alignment rule)
  int st = check_common(h, w, labels, n, d, v, dtype, reduction, lse, nullptr);
  if (st != FLCE_OK) return st;
  if (!aligned(dh_out, 16) || !aligned(dw_out, 16) || (grad_out != nullptr && !aligned(grad_out, 4)))
    return FLCE_ERR_ALIGNMENT;
  Plan p;
  st = make_plan(n, d, v, dtype, 2, &p);
  if (st != FLCE_OK) return st;
  return with_workspace(p, stream, [&](const Work& wk) {
    return run_bwd(p, wk, h, w, labels, lse, grad_out, ignore_index, reduction, dh_out, dw_out, stream);
  });
}

// ---- low-memory fused call: the forward statistics over the whole vocabulary,
// then the backward over vocabulary slices with the logits recomputed ----------

}  // namespace

// Plan of flce_fwd_bwd_lowmem: a forward-only plan, then slices of `vb`
// vocabulary rows (the last one narrower), each run as a backward from the
// saved LSE whose chunks span as many token rows as the buffer budget allows
// (all n at the sizes measured here, so a slice's dW is one reduction over all
// tokens with no running sum).  The slices' dH terms add up in an fp32 [n, d]
// array (bf16) or in dh_out itself (fp32).  Layout of the one workspace:
// [lse n fp32][dH sum n x d fp32, bf16 only][shifted labels n int64][union of
// the forward plan's and the slice plans' workspaces, used one after another].
int make_lowmem_plan(int64_t n, int64_t d, int64_t v, int32_t dtype, LowmemPlan* lp) {
  if (lp == nullptr || n <= 0 || d <= 0 || v <= 0) return FLCE_ERR_INVALID_ARG;
  if (dtype != FLCE_BF16 && dtype != FLCE_F32) return FLCE_ERR_INVALID_ARG;
  if (!mul_ok(n, d) || !mul_ok(v, d) || v > (int64_t(1) << 40) || n > kMaxRows) return FLCE_ERR_INVALID_ARG;
  LowmemPlan q;
  memset(&q, 0, sizeof(q));
  q.budget = env_i64("FLCE_LOWMEM_BUFFER_BYTES", static_cast<int64_t>(kLowmemBudget));
  const int64_t prob_elem = dtype == FLCE_BF16 ? 2 : 4;
  // slice width: whole 256-row blocks, as many as one all-token buffer fits, and at
  // most half of the vocabulary, so that no buffer spans [n, v]; a vocabulary of
  // 256 rows or fewer is one slice whose chunks keep below half of the rows
  int64_t vb = q.budget / (n * prob_elem) / 256 * 256;
  if (vb < 256) vb = 256;
  const int64_t half_v = ((v + 1) / 2 + 255) / 256 * 256;
  if (vb > half_v) vb = half_v;
  const int whole_rows = vb < v ? 1 : 0;
  if (vb > v) vb = v;
  q.vb = vb;
  q.nslices = (v + vb - 1) / vb;
  int st = make_plan(n, d, v, dtype, 0, &q.fwd, 1, q.budget);
  if (st != FLCE_OK) return st;
  st = make_plan(n, d, vb, dtype, 2, &q.slice, 0, q.budget, whole_rows);
  if (st != FLCE_OK) return st;
  const int64_t v_last = v - (q.nslices - 1) * vb;
  st = make_plan(n, d, v_last, dtype, 2, &q.last, 0, q.budget, whole_rows);
  if (st != FLCE_OK) return st;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  q.off_lse = take(sizeof(float) * static_cast<size_t>(n));
  q.off_dhsum = take(dtype == FLCE_BF16 ? sizeof(float) * static_cast<size_t>(n) * static_cast<size_t>(d) : 0);
  q.off_labels = take(sizeof(int64_t) * static_cast<size_t>(n));
  q.off_union = off;
  size_t u = q.fwd.total;
  if (q.slice.total > u) u = q.slice.total;
  if (q.last.total > u) u = q.last.total;
  q.total = off + u;
  *lp = q;
  return FLCE_OK;
}

namespace {

int call_lowmem(const void* h, const void* w, const int64_t* labels, int64_t n, int64_t d, int64_t v,
                flce_dtype dtype, int64_t ignore_index, flce_reduction reduction, float* loss_out, float* lse_out,
                void* dh_out, void* dw_out, hipStream_t stream) {
  int st = check_common(h, w, labels, n, d, v, dtype, reduction, loss_out, lse_out);
  if (st != FLCE_OK) return st;
  if (dh_out == nullptr || dw_out == nullptr) return FLCE_ERR_INVALID_ARG;
  if (!aligned(dh_out, 16) || !aligned(dw_out, 16)) return FLCE_ERR_ALIGNMENT;
  LowmemPlan lp;
  st = make_lowmem_plan(n, d, v, dtype, &lp);
  if (st != FLCE_OK) return st;
  // every slice's first id, shifted off the labels and the ignore value, must not wrap
  if (ignore_index < INT64_MIN + v) return FLCE_ERR_INVALID_ARG;
  Plan whole = lp.fwd;
  whole.total = lp.total;
  const int64_t elem = dtype == FLCE_BF16 ? 2 : 4;
  return with_workspace(whole, stream, [&](const Work& all) {
    char* base = all.base;
    float* lse = lse_out != nullptr ? lse_out : reinterpret_cast<float*>(base + lp.off_lse);
    float* dh_sum = dtype == FLCE_BF16 ? reinterpret_cast<float*>(base + lp.off_dhsum) : static_cast<float*>(dh_out);
    int64_t* shifted = reinterpret_cast<int64_t*>(base + lp.off_labels);
    const Work wf = carve(lp.fwd, base + lp.off_union);
    hipError_t e = run(lp.fwd, wf, h, w, labels, ignore_index, reduction, loss_out, lse, nullptr, nullptr, stream);
    for (int64_t q = 0; e == hipSuccess && q < lp.nslices; ++q) {
      const int64_t v0 = q * lp.vb;
      const Plan& ps = q + 1 < lp.nslices ? lp.slice : lp.last;
      const Work ws = carve(ps, base + lp.off_union);
      e = launch_shift_labels(labels, n, v0, shifted, stream);
      if (e != hipSuccess) break;
      e = run_bwd(ps, ws, h, static_cast<const char*>(w) + v0 * d * elem, shifted, lse, nullptr, ignore_index - v0,
                  reduction, dh_sum, static_cast<char*>(dw_out) + v0 * d * elem, stream, 1, q > 0 ? 1 : 0);
    }
    if (e == hipSuccess && dtype == FLCE_BF16)
      e = timed(K_DH_REDUCE, stream, [&] { return launch_sum_parts(dh_sum, 1, n * d, FLCE_BF16, dh_out, stream); });
    return e;
  });
}

// Forward-only call in a workspace the caller provides (no allocation): the
// forward plan's chunk shrinks until its workspace fits `ws_bytes`;
// FLCE_ERR_SCRATCH when even the smallest chunk does not.
int call_fwd_in(const void* h, const void* w, const int64_t* labels, int64_t n, int64_t d, int64_t v,
                flce_dtype dtype, int64_t ignore_index, flce_reduction reduction, float* loss_out, float* lse_out,
                void* ws, size_t ws_bytes, hipStream_t stream) {
  int st = check_common(h, w, labels, n, d, v, dtype, reduction, loss_out, lse_out);
  if (st != FLCE_OK) return st;
  if (ws == nullptr) return FLCE_ERR_INVALID_ARG;
  Plan p;
  int64_t budget = static_cast<int64_t>(ws_bytes);
  for (;;) {
    st = make_plan(n, d, v, dtype, 0, &p, 1, budget);
    if (st != FLCE_OK) return st;
    if (p.total <= ws_bytes) break;
    // shrink the partials' budget by the excess plus one 16-row step of partials
    const int64_t step = static_cast<int64_t>(p.total - ws_bytes) + p.ngroups * 8 * 16;
    if (p.chunk <= 16 || budget <= step) return FLCE_ERR_SCRATCH;
    budget -= step;
  }
  const Work wk = carve(p, static_cast<char*>(ws));
  hipError_t e = run(p, wk, h, w, labels, ignore_index, reduction, loss_out, lse_out, nullptr, nullptr, stream);
  return e == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

int call_ce_logits(const void* logits, const int64_t* labels, int64_t n, int64_t v, flce_dtype dtype,
                   int64_t ignore_index, flce_reduction reduction, const float* lse_in, const float* grad_scale,
                   float* loss_out, float* lse_out, void* grad_out, hipStream_t stream) {
  if (logits == nullptr || labels == nullptr) return FLCE_ERR_INVALID_ARG;
  if (n <= 0 || v <= 0 || n > kMaxRows || v > (int64_t(1) << 40) || !mul_ok(n, v))
    return FLCE_ERR_INVALID_ARG;
  if (dtype != FLCE_BF16 && dtype != FLCE_F32) return FLCE_ERR_INVALID_ARG;
  if (reduction != FLCE_MEAN && reduction != FLCE_SUM) return FLCE_ERR_INVALID_ARG;
  if (lse_in == nullptr && loss_out == nullptr) return FLCE_ERR_INVALID_ARG;   // statistics need a loss output
  if (lse_in != nullptr && grad_out == nullptr) return FLCE_ERR_INVALID_ARG;   // a backward needs a gradient output
  const size_t elem = dtype == FLCE_BF16 ? 2 : 4;
  if (!aligned(logits, elem) || (grad_out != nullptr && !aligned(grad_out, elem)) || !aligned(labels, 8))
    return FLCE_ERR_ALIGNMENT;
  for (const void* q : {static_cast<const void*>(lse_in), static_cast<const void*>(grad_scale),
                        static_cast<const void*>(loss_out), static_cast<const void*>(lse_out)})
    if (q != nullptr && !aligned(q, 4)) return FLCE_ERR_ALIGNMENT;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FLCE_ERR_HIP;
  hipMemPool_t pool;
  if (device_pool(dev, &pool) != hipSuccess) return FLCE_ERR_HIP;
  // workspace: n_valid, per-row loss, and the LSE when the caller wants none back
  const size_t off_loss = kAlign;
  const size_t off_lse = off_loss + ((sizeof(float) * static_cast<size_t>(n) + kAlign - 1) / kAlign) * kAlign;
  const size_t total = off_lse + sizeof(float) * static_cast<size_t>(n);
  void* base = nullptr;
  if (!pool_alloc(&base, total, pool, stream)) return FLCE_ERR_OOM;
  char* b = static_cast<char*>(base);
  CeArgs a;
  a.logits = logits;
  a.n = n;
  a.v = v;
  a.dtype = dtype;
  a.labels = labels;
  a.ignore_index = ignore_index;
  a.reduction = reduction;
  a.nvalid = reinterpret_cast<int32_t*>(b);
  a.lse_in = lse_in;
  a.grad_scale = grad_scale;
  a.loss_rows = reinterpret_cast<float*>(b + off_loss);
  a.lse_out = lse_out != nullptr ? lse_out : reinterpret_cast<float*>(b + off_lse);
  a.grad = grad_out;
  hipError_t e = timed(K_LABEL_SCAN, stream, [&] {
    return launch_label_count(labels, n, ignore_index, reinterpret_cast<int32_t*>(b), stream);
  });
  if (e == hipSuccess) e = timed(K_CE_ROWS, stream, [&] { return launch_ce_rows(a, stream); });
  if (e == hipSuccess && lse_in == nullptr)
    e = timed(K_LOSS, stream, [&] { return launch_loss_sum(a.loss_rows, n, a.nvalid, reduction, loss_out, stream); });
  hipError_t f = hipFreeAsync(base, stream);
  if (e != hipSuccess) return FLCE_ERR_HIP;
  return status_of(f);
}

// ---- fp8 forward -------------------------------------------------------------------

int call_fwd_fp8(const void* h_q, const float* h_scale, const void* w_q, const float* w_scale, const int64_t* labels,
                 int64_t n, int64_t d, int64_t v, int64_t ignore_index, flce_reduction reduction, float* loss_out,
                 float* lse_out, hipStream_t stream) {
  if (h_q == nullptr || w_q == nullptr || h_scale == nullptr || w_scale == nullptr || labels == nullptr ||
      loss_out == nullptr)
    return FLCE_ERR_INVALID_ARG;
  if (n <= 0 || d <= 0 || v <= 0) return FLCE_ERR_INVALID_ARG;
  if (reduction != FLCE_MEAN && reduction != FLCE_SUM) return FLCE_ERR_INVALID_ARG;
  if (d % 16 != 0 || !aligned(h_q, 16) || !aligned(w_q, 16) || !aligned(w_scale, 16) || !aligned(h_scale, 4) ||
      !aligned(labels, 8) || !aligned(loss_out, 4) || (lse_out != nullptr && !aligned(lse_out, 4)))
    return FLCE_ERR_ALIGNMENT;
  Plan p;
  // the matrix engine sees each row of e4m3 bytes as d / 2 sixteen-bit units
  int st = make_plan(n, d / 2, v, FLCE_BF16, 0, &p);
  if (st != FLCE_OK) return st;
  return with_workspace(p, stream, [&](const Work& wk) {
    return run(p, wk, h_q, w_q, labels, ignore_index, reduction, loss_out, lse_out, nullptr, nullptr, stream, nullptr,
               h_scale, w_scale);
  });
}

// The backward from the saved LSE for e4m3 inputs: H and W are dequantised to
// bf16 in the workspace; per chunk the fp8 logits are recomputed (the forward's
// exact logits) and their epilogue writes G, then dH and dW run on the bf16
// copies.  `p` is the bf16 plan over d; `p8` the fp8 plan over d / 2 units,
// whose chunk rows and vocabulary pitch are the same.
int call_bwd_fp8(const void* h_q, const float* h_scale, const void* w_q, const float* w_scale, const int64_t* labels,
                 const float* lse, const float* grad_out, int64_t n, int64_t d, int64_t v, int64_t ignore_index,
                 flce_reduction reduction, void* dh_out, void* dw_out, hipStream_t stream) {
  if (h_q == nullptr || w_q == nullptr || h_scale == nullptr || w_scale == nullptr || labels == nullptr ||
      lse == nullptr || dh_out == nullptr || dw_out == nullptr)
    return FLCE_ERR_INVALID_ARG;
  if (n <= 0 || d <= 0 || v <= 0) return FLCE_ERR_INVALID_ARG;
  if (reduction != FLCE_MEAN && reduction != FLCE_SUM) return FLCE_ERR_INVALID_ARG;
  if (d % 16 != 0 || !aligned(h_q, 16) || !aligned(w_q, 16) || !aligned(w_scale, 16) || !aligned(h_scale, 4) ||
      !aligned(labels, 8) || !aligned(lse, 4) || !aligned(dh_out, 16) || !aligned(dw_out, 16) ||
      (grad_out != nullptr && !aligned(grad_out, 4)))
    return FLCE_ERR_ALIGNMENT;
  Plan p, p8;
  // both plans as for a backward (chunked, unpaired), so that their chunks match
  int st = make_plan(n, d, v, FLCE_BF16, 2, &p, /*allow_pair=*/0);
  if (st != FLCE_OK) return st;
  st = make_plan(n, d / 2, v, FLCE_BF16, 2, &p8, /*allow_pair=*/0);
  if (st != FLCE_OK) return st;
  if (p8.chunk != p.chunk || p8.vp != p.vp || !mul_ok(v, d)) return FLCE_ERR_INVALID_ARG;
  const size_t off_w16 = p.total;
  const size_t off_h16 = off_w16 + align_up(sizeof(uint16_t) * static_cast<size_t>(v) * static_cast<size_t>(d));
  p.total = off_h16 + align_up(sizeof(uint16_t) * static_cast<size_t>(n) * static_cast<size_t>(d));
  return with_workspace(p, stream, [&](const Work& wk) {
    uint16_t* w16 = reinterpret_cast<uint16_t*>(wk.base + off_w16);
    uint16_t* h16 = reinterpret_cast<uint16_t*>(wk.base + off_h16);
    hipError_t e = timed(K_DEQUANT, stream, [&] { return launch_dequant_e4m3(w_q, w_scale, v, d, w16, stream); });
    if (e == hipSuccess)
      e = timed(K_DEQUANT, stream, [&] { return launch_dequant_e4m3(h_q, h_scale, n, d, h16, stream); });
    if (e == hipSuccess) e = timed(K_LABEL_SCAN, stream, [&] { return launch_label_scan(p, wk, labels, ignore_index, stream); });
    if (e != hipSuccess) return e;
    for (int64_t c = 0; c < p.nchunks; ++c) {
      ChunkArgs a;
      a.row0 = c * p.chunk;
      a.rows = p.n - a.row0 < p.chunk ? p.n - a.row0 : p.chunk;
      a.labels = labels + a.row0;
      a.ignore_index = ignore_index;
      a.reduction = reduction;
      a.lse_rows = nullptr;
      a.lse_in = lse + a.row0;
      a.grad_out = grad_out;
      a.zy_rows = nullptr;
      a.dh_f32 = 0;
      a.dh_accumulate = 0;
      a.dw_mode = p.nchunks == 1 ? DW_SINGLE : (c == 0 ? DW_FIRST : (c == p.nchunks - 1 ? DW_LAST : DW_MID));
      a.fold = 0;
      // recompute: fp8 operands, G into the chunk buffer
      a.fp8 = 1;
      a.h = static_cast<const char*>(h_q) + a.row0 * d;
      a.w = w_q;
      a.h_scale = h_scale + a.row0;
      a.w_scale = w_scale;
      a.dh = nullptr;
      a.dw = nullptr;
      e = timed(K_LOGITS, stream, [&] { return mfma_logits(p8, wk, a, LOGITS_GRAD_FROM_LSE, stream); });
      if (e != hipSuccess) return e;
      // the contractions: bf16 copies
      a.fp8 = 0;
      a.h_scale = nullptr;
      a.w_scale = nullptr;
      a.h = h16 + a.row0 * d;
      a.w = w16;
      a.dh = static_cast<char*>(dh_out) + a.row0 * d * 2;
      a.dw = dw_out;
      e = timed(K_DH, stream, [&] { return mfma_dh(p, wk, a, stream); });
      if (e != hipSuccess) return e;
      if (p.dh_splits > 1) {
        e = timed(K_DH_REDUCE, stream, [&] { return launch_dh_reduce(p, wk, a, stream); });
        if (e != hipSuccess) return e;
      }
      e = timed(K_DW, stream, [&] { return mfma_dw(p, wk, a, stream); });
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  });
}

// ---- vocabulary shards ---------------------------------------------------------

// A shard's plan plus room for its shifted labels (int64 [n]) after the plan's workspace.
int shard_plan(int64_t n, int64_t d, int64_t v_shard, int64_t v_first, flce_dtype dtype, int64_t ignore_index,
               int with_bwd, Plan* p, size_t* off_labels) {
  if (v_first < 0 || v_first > (int64_t(1) << 40)) return FLCE_ERR_INVALID_ARG;
  // the shifted ignore value must not wrap
  if (ignore_index < INT64_MIN + v_first) return FLCE_ERR_INVALID_ARG;
  const int st = make_plan(n, d, v_shard, dtype, with_bwd, p);
  if (st != FLCE_OK) return st;
  *off_labels = p->total;
  p->total += align_up(sizeof(int64_t) * static_cast<size_t>(n));
  return FLCE_OK;
}

int call_fwd_shard(const void* h, const void* w_shard, const int64_t* labels, int64_t n, int64_t d, int64_t v_shard,
                   int64_t v_first, flce_dtype dtype, int64_t ignore_index, float* lse_part_out, float* zy_part_out,
                   hipStream_t stream) {
  if (lse_part_out == nullptr || zy_part_out == nullptr) return FLCE_ERR_INVALID_ARG;
  int st = check_common(h, w_shard, labels, n, d, v_shard, dtype, FLCE_SUM, lse_part_out, zy_part_out);
  if (st != FLCE_OK) return st;
  Plan p;
  size_t off_labels = 0;
  st = shard_plan(n, d, v_shard, v_first, dtype, ignore_index, 0, &p, &off_labels);
  if (st != FLCE_OK) return st;
  const int64_t* base_labels = labels;
  return with_workspace(p, stream, [&](const Work& wk) {
    int64_t* shifted = reinterpret_cast<int64_t*>(wk.base + off_labels);
    hipError_t e = launch_shift_labels(base_labels, n, v_first, shifted, stream);
    if (e != hipSuccess) return e;
    return run(p, wk, h, w_shard, shifted, ignore_index - v_first, FLCE_SUM, nullptr, lse_part_out, nullptr,
               nullptr, stream, zy_part_out);
  });
}

int call_merge_shards(const float* lse_parts, const float* zy_parts, int64_t num_shards, const int64_t* labels,
                      int64_t n, int64_t ignore_index, flce_reduction reduction, float* loss_out, float* lse_out,
                      hipStream_t stream) {
  if (lse_parts == nullptr || zy_parts == nullptr || labels == nullptr || loss_out == nullptr)
    return FLCE_ERR_INVALID_ARG;
  if (n <= 0 || num_shards <= 0 || num_shards > (int64_t(1) << 20) || !mul_ok(n, num_shards))
    return FLCE_ERR_INVALID_ARG;
  if (reduction != FLCE_MEAN && reduction != FLCE_SUM) return FLCE_ERR_INVALID_ARG;
  if (!aligned(lse_parts, 4) || !aligned(zy_parts, 4) || !aligned(labels, 8) || !aligned(loss_out, 4) ||
      (lse_out != nullptr && !aligned(lse_out, 4)))
    return FLCE_ERR_ALIGNMENT;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FLCE_ERR_HIP;
  hipMemPool_t pool;
  if (device_pool(dev, &pool) != hipSuccess) return FLCE_ERR_HIP;
  // workspace: n_valid, per-row loss, and the LSE when the caller wants none back
  const size_t off_loss = kAlign;
  const size_t off_lse = off_loss + align_up(sizeof(float) * static_cast<size_t>(n));
  const size_t total = off_lse + sizeof(float) * static_cast<size_t>(n);
  void* base = nullptr;
  if (!pool_alloc(&base, total, pool, stream)) return FLCE_ERR_OOM;
  char* b = static_cast<char*>(base);
  int32_t* nvalid = reinterpret_cast<int32_t*>(b);
  float* loss_rows = reinterpret_cast<float*>(b + off_loss);
  float* lse = lse_out != nullptr ? lse_out : reinterpret_cast<float*>(b + off_lse);
  hipError_t e = timed(K_LABEL_SCAN, stream, [&] { return launch_label_count(labels, n, ignore_index, nvalid, stream); });
  if (e == hipSuccess)
    e = timed(K_LSE_MERGE, stream, [&] {
      return launch_shard_merge(lse_parts, zy_parts, num_shards, n, labels, ignore_index, lse, loss_rows, stream);
    });
  if (e == hipSuccess)
    e = timed(K_LOSS, stream, [&] { return launch_loss_sum(loss_rows, n, nvalid, reduction, loss_out, stream); });
  hipError_t f = hipFreeAsync(base, stream);
  if (e != hipSuccess) return FLCE_ERR_HIP;
  return status_of(f);
}

// accumulate: dh_part_out += the shard's dH term instead of = (one fp32 sum for every shard).
int call_bwd_shard(const void* h, const void* w_shard, const int64_t* labels, const float* lse, const float* grad_out,
                   int64_t n, int64_t d, int64_t v_shard, int64_t v_first, flce_dtype dtype, int64_t ignore_index,
                   flce_reduction reduction, float* dh_part_out, void* dw_shard_out, hipStream_t stream,
                   int accumulate) {
  if (lse == nullptr || dh_part_out == nullptr || dw_shard_out == nullptr) return FLCE_ERR_INVALID_ARG;
  int st = check_common(h, w_shard, labels, n, d, v_shard, dtype, reduction, lse, nullptr);
  if (st != FLCE_OK) return st;
  if (!aligned(dh_part_out, 16) || !aligned(dw_shard_out, 16) || (grad_out != nullptr && !aligned(grad_out, 4)))
    return FLCE_ERR_ALIGNMENT;
  Plan p;
  size_t off_labels = 0;
  st = shard_plan(n, d, v_shard, v_first, dtype, ignore_index, 2, &p, &off_labels);
  if (st != FLCE_OK) return st;
  return with_workspace(p, stream, [&](const Work& wk) {
    int64_t* shifted = reinterpret_cast<int64_t*>(wk.base + off_labels);
    hipError_t e = launch_shift_labels(labels, n, v_first, shifted, stream);
    if (e != hipSuccess) return e;
    return run_bwd(p, wk, h, w_shard, shifted, lse, grad_out, ignore_index - v_first, reduction, dh_part_out,
                   dw_shard_out, stream, 1, accumulate);
  });
}

int call_sum_parts(const float* parts, int64_t num_parts, int64_t count, flce_dtype dtype, void* out,
                   hipStream_t stream) {
  if (parts == nullptr || out == nullptr || num_parts <= 0 || count <= 0 || !mul_ok(num_parts, count))
    return FLCE_ERR_INVALID_ARG;
  if (dtype != FLCE_BF16 && dtype != FLCE_F32) return FLCE_ERR_INVALID_ARG;
  if (!aligned(parts, 4) || !aligned(out, dtype == FLCE_BF16 ? 2 : 4)) return FLCE_ERR_ALIGNMENT;
  return status_of(timed(K_DH_REDUCE, stream, [&] { return launch_sum_parts(parts, num_parts, count, dtype, out, stream); }));
}

int call_scale(void* x, int64_t count, flce_dtype dtype, const float* scale, hipStream_t stream) {
  if (x == nullptr || scale == nullptr || count <= 0 || count > (int64_t(1) << 40)) return FLCE_ERR_INVALID_ARG;
  if (dtype != FLCE_BF16 && dtype != FLCE_F32) return FLCE_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(scale, 4)) return FLCE_ERR_ALIGNMENT;
  return status_of(launch_scale(x, count, dtype, scale, stream));
}

}  // namespace

int fwd_in_workspace(const void* h, const void* w, const int64_t* labels, int64_t n, int64_t d, int64_t v,
                     flce_dtype dtype, int64_t ignore_index, flce_reduction reduction, float* loss_out,
                     float* lse_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  return call_fwd_in(h, w, labels, n, d, v, dtype, ignore_index, reduction, loss_out, lse_out, ws, ws_bytes, stream);
}

}  // namespace flce

extern "C" {

int flce_fwd_bwd(const void* h, const void* w, const int64_t* labels, int64_t n, int64_t d, int64_t v,
                 flce_dtype dtype, int64_t ignore_index, flce_reduction reduction, float* loss_out, float* lse_out,
                 void* dh_out, void* dw_out, hipStream_t stream) {
  return flce::call(h, w, labels, n, d, v, dtype, ignore_index, reduction, loss_out, lse_out, dh_out, dw_out, stream,
                    1);
}

int flce_fwd_bwd_lowmem(const void* h, const void* w, const int64_t* labels, int64_t n, int64_t d, int64_t v,
                        flce_dtype dtype, int64_t ignore_index, flce_reduction reduction, float* loss_out,
                        float* lse_out, void* dh_out, void* dw_out, hipStream_t stream) {
  return flce::call_lowmem(h, w, labels, n, d, v, dtype, ignore_index, reduction, loss_out, lse_out, dh_out, dw_out,
                           stream);
}

size_t flce_workspace_bytes_lowmem(int64_t n, int64_t d, int64_t v, flce_dtype dtype) {
  flce::LowmemPlan lp;
  if (flce::make_lowmem_plan(n, d, v, dtype, &lp) != FLCE_OK) return 0;
  return lp.total;
}

int flce_lowmem_plan_info(int64_t n, int64_t d, int64_t v, flce_dtype dtype, flce_lowmem_plan_t* out) {
  if (out == nullptr) return FLCE_ERR_INVALID_ARG;
  flce::LowmemPlan lp;
  const int st = flce::make_lowmem_plan(n, d, v, dtype, &lp);
  if (st != FLCE_OK) return st;
  out->slice_cols = lp.vb;
  out->num_slices = lp.nslices;
  out->slice_chunk_rows = lp.slice.chunk;
  out->slice_chunks = lp.slice.nchunks;
  out->fwd_chunk_rows = lp.fwd.chunk;
  out->buffer_budget_bytes = static_cast<size_t>(lp.budget);
  out->workspace_bytes = lp.total;
  return FLCE_OK;
}

int flce_fwd(const void* h, const void* w, const int64_t* labels, int64_t n, int64_t d, int64_t v, flce_dtype dtype,
             int64_t ignore_index, flce_reduction reduction, float* loss_out, float* lse_out, hipStream_t stream) {
  return flce::call(h, w, labels, n, d, v, dtype, ignore_index, reduction, loss_out, lse_out, nullptr, nullptr,
                    stream, 0);
}

int flce_bwd(const void* h, const void* w, const int64_t* labels, const float* lse, const float* grad_out, int64_t n,
             int64_t d, int64_t v, flce_dtype dtype, int64_t ignore_index, flce_reduction reduction, void* dh_out,
             void* dw_out, hipStream_t stream) {
  return flce::call_bwd(h, w, labels, lse, grad_out, n, d, v, dtype, ignore_index, reduction, dh_out, dw_out, stream);
}

int flce_ce_logits(const void* logits, const int64_t* labels, int64_t n, int64_t v, flce_dtype dtype,
                   int64_t ignore_index, flce_reduction reduction, const float* lse_in, const float* grad_scale,
                   float* loss_out, float* lse_out, void* grad_out, hipStream_t stream) {
  return flce::call_ce_logits(logits, labels, n, v, dtype, ignore_index, reduction, lse_in, grad_scale, loss_out,
                              lse_out, grad_out, stream);
}

int flce_fwd_fp8(const void* h_q, const float* h_scale, const void* w_q, const float* w_scale, const int64_t* labels,
                 int64_t n, int64_t d, int64_t v, int64_t ignore_index, flce_reduction reduction, float* loss_out,
                 float* lse_out, hipStream_t stream) {
  return flce::call_fwd_fp8(h_q, h_scale, w_q, w_scale, labels, n, d, v, ignore_index, reduction, loss_out, lse_out,
                            stream);
}

int flce_bwd_fp8(const void* h_q, const float* h_scale, const void* w_q, const float* w_scale, const int64_t* labels,
                 const float* lse, const float* grad_out, int64_t n, int64_t d, int64_t v, int64_t ignore_index,
                 flce_reduction reduction, void* dh_out, void* dw_out, hipStream_t stream) {
  return flce::call_bwd_fp8(h_q, h_scale, w_q, w_scale, labels, lse, grad_out, n, d, v, ignore_index, reduction,
                            dh_out, dw_out, stream);
}

int flce_fwd_shard(const void* h, const void* w_shard, const int64_t* labels, int64_t n, int64_t d, int64_t v_shard,
                   int64_t v_first, flce_dtype dtype, int64_t ignore_index, float* lse_part_out, float* zy_part_out,
                   hipStream_t stream) {
  return flce::call_fwd_shard(h, w_shard, labels, n, d, v_shard, v_first, dtype, ignore_index, lse_part_out,
                              zy_part_out, stream);
}

int flce_merge_shards(const float* lse_parts, const float* zy_parts, int64_t num_shards, const int64_t* labels,
                      int64_t n, int64_t ignore_index, flce_reduction reduction, float* loss_out, float* lse_out,
                      hipStream_t stream) {
  return flce::call_merge_shards(lse_parts, zy_parts, num_shards, labels, n, ignore_index, reduction, loss_out,
                                 lse_out, stream);
}

int flce_bwd_shard(const void* h, const void* w_shard, const int64_t* labels, const float* lse, const float* grad_out,
                   int64_t n, int64_t d, int64_t v_shard, int64_t v_first, flce_dtype dtype, int64_t ignore_index,
                   flce_reduction reduction, float* dh_part_out, void* dw_shard_out, hipStream_t stream) {
  return flce::call_bwd_shard(h, w_shard, labels, lse, grad_out, n, d, v_shard, v_first, dtype, ignore_index,
                              reduction, dh_part_out, dw_shard_out, stream, 0);
}

int flce_bwd_shard_accumulate(const void* h, const void* w_shard, const int64_t* labels, const float* lse,
                              const float* grad_out, int64_t n, int64_t d, int64_t v_shard, int64_t v_first,
                              flce_dtype dtype, int64_t ignore_index, flce_reduction reduction, float* dh_acc,
                              void* dw_shard_out, hipStream_t stream) {
  return flce::call_bwd_shard(h, w_shard, labels, lse, grad_out, n, d, v_shard, v_first, dtype, ignore_index,
                              reduction, dh_acc, dw_shard_out, stream, 1);
}

int flce_sum_parts(const float* parts, int64_t num_parts, int64_t count, flce_dtype dtype, void* out,
                   hipStream_t stream) {
  return flce::call_sum_parts(parts, num_parts, count, dtype, out, stream);
}

int flce_scale(void* x, int64_t count, flce_dtype dtype, const float* scale, hipStream_t stream) {
  return flce::call_scale(x, count, dtype, scale, stream);
}

size_t flce_workspace_bytes(int64_t n, int64_t d, int64_t v, flce_dtype dtype, int with_bwd) {
  flce::Plan p;
  if (flce::make_plan(n, d, v, dtype, with_bwd, &p) != FLCE_OK) return 0;
  return p.total;
}

int flce_plan_info(int64_t n, int64_t d, int64_t v, flce_dtype dtype, int with_bwd, flce_plan_t* out) {
  if (out == nullptr) return FLCE_ERR_INVALID_ARG;
  flce::Plan p;
  const int st = flce::make_plan(n, d, v, dtype, with_bwd, &p);
  if (st != FLCE_OK) return st;
  out->chunk_rows = p.chunk;
  out->num_chunks = p.nchunks;
  out->vocab_pitch = p.vp;
  out->group_cols = p.group;
  out->dh_splits = p.dh_splits;
  out->engine = p.engine;
  out->dw_accumulator = p.dw_acc;
  out->workspace_bytes = p.total;
  out->prob_buffer_bytes = p.prob_bytes;
  out->dw_pairs = p.dw_pair;
  out->folded_factor = p.fold;
  return FLCE_OK;
}

const char* flce_strerror(int status) {
  switch (status) {
    case FLCE_OK: return "success";
    case FLCE_ERR_INVALID_ARG: return "invalid argument (null pointer, non-positive size, unknown enum or size overflow)";
    case FLCE_ERR_ALIGNMENT: return "misaligned pointer or row pitch (rows must start on 16-byte boundaries)";
    case FLCE_ERR_OOM: return "workspace allocation failed";
    case FLCE_ERR_HIP: return "HIP runtime or kernel launch error";
    case FLCE_ERR_SCRATCH: return "problem too large for the fixed scratch area of flce_fwd_noalloc";
    default: return "unknown status";
  }
}

int flce_profile_enable(int on) {
  std::lock_guard<std::mutex> lk(flce::g_prof.mu);
  flce::g_prof.on = on != 0;
  return FLCE_OK;
}

int flce_profile_read(int max_kinds, int64_t* launches, double* total_ms) {
  using flce::g_prof;
  std::lock_guard<std::mutex> lk(g_prof.mu);
  int status = FLCE_OK;
  for (auto& q : g_prof.pending) {
    float ms = 0.0f;
    if (hipEventSynchronize(q.b) != hipSuccess || hipEventElapsedTime(&ms, q.a, q.b) != hipSuccess)
      status = FLCE_ERR_HIP;
    g_prof.launches[q.kind] += 1;
    g_prof.ms[q.kind] += ms;
    hipEventDestroy(q.a);
    hipEventDestroy(q.b);
  }
  g_prof.pending.clear();
  for (int k = 0; k < flce::K_NUM_KINDS && k < max_kinds; ++k) {
    if (launches) launches[k] = g_prof.launches[k];
    if (total_ms) total_ms[k] = g_prof.ms[k];
    g_prof.launches[k] = 0;
    g_prof.ms[k] = 0.0;
  }
  return status;
}

const char* flce_profile_kind_name(int kind) {
  if (kind < 0 || kind >= flce::K_NUM_KINDS) return nullptr;
  return flce::kKindNames[kind];
}

int flce_memory_reserved(uint64_t* reserved_bytes) {
  if (reserved_bytes == nullptr) return FLCE_ERR_INVALID_ARG;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FLCE_ERR_HIP;
  hipMemPool_t pool;
  if (flce::device_pool(dev, &pool) != hipSuccess) return FLCE_ERR_HIP;
  uint64_t v = 0;
  if (hipMemPoolGetAttribute(pool, hipMemPoolAttrReservedMemCurrent, &v) != hipSuccess) return FLCE_ERR_HIP;
  *reserved_bytes = v;
  return FLCE_OK;
}

int flce_pool_trim(uint64_t keep_bytes) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FLCE_ERR_HIP;
  hipMemPool_t pool;
  if (flce::device_pool(dev, &pool) != hipSuccess) return FLCE_ERR_HIP;
  return hipMemPoolTrimTo(pool, static_cast<size_t>(keep_bytes)) == hipSuccess ? FLCE_OK : FLCE_ERR_HIP;
}

int flce_memory_high_water(int reset, uint64_t* used_high_bytes) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FLCE_ERR_HIP;
  hipMemPool_t pool;
  if (flce::device_pool(dev, &pool) != hipSuccess) return FLCE_ERR_HIP;
  if (used_high_bytes != nullptr) {
    uint64_t v = 0;
    if (hipMemPoolGetAttribute(pool, hipMemPoolAttrUsedMemHigh, &v) != hipSuccess) return FLCE_ERR_HIP;
    *used_high_bytes = v;
  }
  if (reset) {
    uint64_t zero = 0;
    if (hipMemPoolSetAttribute(pool, hipMemPoolAttrUsedMemHigh, &zero) != hipSuccess) return FLCE_ERR_HIP;
  }
  return FLCE_OK;
}

}  // extern "C"
