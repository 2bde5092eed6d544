// Internal declarations shared by the host orchestration and the kernel
// translation units of the fused linear cross-entropy library (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "flce.h"

namespace flce {

enum Engine : int32_t { ENGINE_MFMA = 0, ENGINE_FMA = 1 };

// Output tiles of the dH contraction: 256 x 256 on the matrix engine, 64 rows x
// kFmaDhTileCols columns on the fp32 engine (the plan's split choice counts them).
constexpr int kFmaDhTileCols = 32;

// dW epilogue mode for one chunk of the token reduction.
enum DwMode : int32_t {
  DW_SINGLE = 0,  // only chunk: out = partial
  DW_FIRST = 1,   // acc = partial
  DW_MID = 2,     // acc += partial
  DW_LAST = 3     // out = acc + partial
};

// Execution plan: how a call is cut into chunks and where its workspace lives.
struct Plan {
  int64_t n, d, v;
  int32_t dtype;
  int32_t engine;
  int32_t with_bwd;
  int64_t chunk;       // token rows per chunk (C)
  int64_t nchunks;
  int64_t vp;          // row pitch (elements) of the chunk's probability/gradient buffer
  int64_t group;       // vocabulary columns per partial (max, sum-exp) pair
  int64_t ngroups;
  int64_t dh_splits;   // split of the K = vocabulary reduction of dH
  int32_t dw_acc;      // dW's running sum needs a workspace low half (bf16 path, several chunks)
  int32_t dw_pair;     // two chunk buffers; each dW launch reduces over a pair of consecutive chunks
  int32_t fold;        // one-pass backward with the softmax factor folded into a per-row factor (see run())
  int64_t group_m[3];  // tile-row group of the logits, dH and dW tile orders
  // byte offsets inside the single workspace allocation
  size_t off_nvalid, off_zy, off_gy, off_lse, off_loss, off_pm, off_ps, off_prob, off_dwacc, off_dhpart;
  size_t off_uref, off_flag, off_rowf, off_hs;
  size_t total;
  size_t prob_bytes;
};

// with_bwd: 0 forward only, 2 backward by recomputing the logits from a saved
// LSE (run_bwd), any other value forward and one-pass backward (run).
// allow_pair = 0 keeps one chunk buffer (for loops that run dW chunk by chunk).
// budget > 0 replaces the default byte budget of one chunk's buffer (or, for a
// forward-only plan, of its group partials).  whole_rows = 1 lets a chunk hold
// every row that fits the budget, up to all n (a vocabulary slice's buffer,
// which is narrower than the vocabulary); otherwise a gradient plan keeps its
// chunks below half of the rows.
int make_plan(int64_t n, int64_t d, int64_t v, int32_t dtype, int32_t with_bwd, Plan* p, int allow_pair = 1,
              int64_t budget = 0, int whole_rows = 0);

// Plan of the low-memory fused call (flce_fwd_bwd_lowmem).
struct LowmemPlan {
  Plan fwd;          // forward-only plan over the whole vocabulary
  Plan slice, last;  // backward plans of a full-width and of the last vocabulary slice
  int64_t vb;        // vocabulary rows per slice
  int64_t nslices;
  int64_t budget;    // bytes of one slice's gradient buffer (and of the forward's group partials)
  size_t off_lse, off_dhsum, off_labels, off_union, total;
};
int make_lowmem_plan(int64_t n, int64_t d, int64_t v, int32_t dtype, LowmemPlan* lp);

// Forward only (flce_fwd) inside a workspace of ws_bytes at ws, allocating nothing;
// FLCE_ERR_SCRATCH when the sizes need more.
int fwd_in_workspace(const void* h, const void* w, const int64_t* labels, int64_t n, int64_t d, int64_t v,
                     flce_dtype dtype, int64_t ignore_index, flce_reduction reduction, float* loss_out,
                     float* lse_out, void* ws, size_t ws_bytes, hipStream_t stream);

// Pointers into the workspace for one call.
struct Work {
  char* base;        // the call's whole workspace
  int32_t* nvalid;   // [1]
  float* zy;         // [C]   target logit of each chunk row (0 until found)
  float* gy;         // [C]   gradient value at the target column
  float* lse;        // [n]   used when the caller passes no lse_out
  float* loss_rows;  // [n]   per-row NLL (unscaled; 0 for ignored rows)
  float* pm;         // [G][C] partial row max per vocabulary group; becomes the softmax factor
  float* ps;         // [G][C] partial sum of exp(z - max) per group
  void* prob;        // [C][vp] exp(z - group max), turned into G in place (dtype of the engine);
                     // folded: exp(z - r_g), with the target column patched in place
  uint16_t* dwlo;    // [v][d] lower 16 bits of the fp32 running dW sum; dw_out holds the upper 16
  float* dhpart;     // [S][C][d] fp32 split-vocabulary partials of dH (when dh_splits > 1)
  // folded one-pass backward (plan.fold)
  float* uref;       // [C] u_t, the row's target logit (+-1e30, see target_ref_kernel)
  int32_t* flag;     // [C] 1 where some group max exceeds u_t by more than kFoldMargin
  float* rowf;       // [C rounded up to 256] per-row factor F_t = scale * exp(ref_t - lse_t),
                     // ref_t = u_t, or the row max for a flagged row
  void* hs;          // [C][d] bf16(F * H) (two such with paired buffers): dW's token operand
};

// Folded backward: group g of row t is stored as exp(z - r_g) with
// r_g = max(u_t, group max - kFoldMargin), at most exp(kFoldMargin); for an
// unflagged row u_t >= row max - kFoldMargin, so F_t >= scale * exp(-kFoldMargin - log v)
// stays a normal number.
constexpr float kFoldMargin = 30.0f;

// Kernel kinds for the timing instrumentation.
enum Kind : int {
  K_LABEL_SCAN = 0,
  K_LOGITS = 1,
  K_LSE_MERGE = 2,
  K_GRAD = 3,
  K_DH = 4,
  K_DH_REDUCE = 5,
  K_DW = 6,
  K_LOSS = 7,
  K_CE_ROWS = 8,
  K_DEQUANT = 9,
  K_TARGET_REF = 10,
  K_FOLD_PATCH = 11,
  K_NUM_KINDS = 12
};

// What the logits contraction's epilogue produces.
enum LogitsMode : int32_t {
  LOGITS_STATS = 0,          // per-group (max, sum-exp) partials and the target logit
  LOGITS_PROB = 1,           // ... and exp(z - group max) into the chunk's buffer
  LOGITS_GRAD_FROM_LSE = 2   // the gradient G itself, from the saved per-row LSE (recompute backward)
};

// --- per-chunk launch arguments --------------------------------------------------

struct ChunkArgs {
  const void* h;            // chunk's first row of H
  const void* w;
  const int64_t* labels;    // chunk's first label
  int64_t rows;             // rows in this chunk (<= plan.chunk)
  int64_t row0;             // index of the chunk's first row in the whole call
  int64_t ignore_index;
  int32_t reduction;
  float* lse_rows;          // chunk's slice of the LSE output
  void* dh;                 // chunk's first row of dH output
  void* dw;                 // dW output
  int32_t dw_mode;
  const float* lse_in;      // chunk's slice of the saved LSE (recompute backward), else nullptr
  const float* grad_out;    // upstream gradient of the loss (device scalar) or nullptr for 1
  float* zy_rows;           // chunk's slice of a per-row target-logit output, or nullptr
  int32_t dh_f32;           // 1: dh is an fp32 array whatever the dtype (a shard's dH partial)
  int32_t dh_accumulate;    // 1: dh (fp32) already holds a partial sum; this chunk's term is added to it
  int32_t fp8;              // 1: h and w hold e4m3 bytes (d counts byte pairs), scaled per row
  const float* h_scale;     // fp8: chunk's first token scale
  const float* w_scale;     // fp8: vocabulary row scales
  int32_t fold;             // 1: folded one-pass backward (plan.fold, run() only)
};

// --- launchers (each returns the launch status) ---------------------------------

// Small kernels (kernels_common.hip).
hipError_t launch_label_scan(const Plan& p, const Work& w, const int64_t* labels, int64_t ignore_index,
                             hipStream_t s);
hipError_t launch_lse_merge(const Plan& p, const Work& w, const ChunkArgs& a, int with_grad, hipStream_t s);
hipError_t launch_grad(const Plan& p, const Work& w, const ChunkArgs& a, hipStream_t s);
hipError_t launch_target_ref(const Plan& p, const Work& w, const ChunkArgs& a, hipStream_t s);
hipError_t launch_fold_patch(const Plan& p, const Work& w, const ChunkArgs& a, hipStream_t s);
hipError_t launch_loss_reduce(const Plan& p, const Work& w, int32_t reduction, float* loss_out, hipStream_t s);
hipError_t launch_dh_reduce(const Plan& p, const Work& w, const ChunkArgs& a, hipStream_t s);
hipError_t launch_label_count(const int64_t* labels, int64_t n, int64_t ignore_index, int32_t* nvalid, hipStream_t s);
hipError_t launch_loss_sum(const float* loss_rows, int64_t n, const int32_t* nvalid, int32_t reduction,
                           float* loss_out, hipStream_t s);
// e4m3 rows with one scale per row -> bf16 (d a multiple of 16).
hipError_t launch_dequant_e4m3(const void* q, const float* scale, int64_t rows, int64_t d, void* out, hipStream_t s);
// Vocabulary shards.
hipError_t launch_shift_labels(const int64_t* labels, int64_t n, int64_t first, int64_t* out, hipStream_t s);
hipError_t launch_shard_merge(const float* lse_parts, const float* zy_parts, int64_t shards, int64_t n,
                              const int64_t* labels, int64_t ignore_index, float* lse_out, float* loss_rows,
                              hipStream_t s);
hipError_t launch_scale(void* x, int64_t count, int32_t dtype, const float* scale, hipStream_t s);
hipError_t launch_sum_parts(const float* parts, int64_t num_parts, int64_t count, int32_t dtype, void* out,
                            hipStream_t s);

// Cross-entropy on given logits (ce_logits.hip).
struct CeArgs {
  const void* logits;       // [n, v], dtype
  int64_t n, v;
  int32_t dtype;
  const int64_t* labels;
  int64_t ignore_index;
  int32_t reduction;
  const int32_t* nvalid;
  const float* lse_in;      // saved LSE (skip the statistics pass) or nullptr
  const float* grad_scale;  // device scalar or nullptr for 1
  float* lse_out;           // [n] (statistics pass)
  float* loss_rows;         // [n] (statistics pass)
  void* grad;               // [n, v] dtype, may alias logits, or nullptr
};
hipError_t launch_ce_rows(const CeArgs& a, hipStream_t s);

// fp32 FMA engine (engine_fma.hip): FLCE_F32 (dw_out itself accumulates).
hipError_t fma_logits(const Plan& p, const Work& w, const ChunkArgs& a, int mode, hipStream_t s);
hipError_t fma_dh(const Plan& p, const Work& w, const ChunkArgs& a, hipStream_t s);
hipError_t fma_dw(const Plan& p, const Work& w, const ChunkArgs& a, hipStream_t s);

// bf16 matrix-core engine (engine_mfma.hip): FLCE_BF16.
hipError_t mfma_logits(const Plan& p, const Work& w, const ChunkArgs& a, int mode, hipStream_t s);
hipError_t mfma_dh(const Plan& p, const Work& w, const ChunkArgs& a, hipStream_t s);
hipError_t mfma_dw(const Plan& p, const Work& w, const ChunkArgs& a, hipStream_t s);

}  // namespace flce
