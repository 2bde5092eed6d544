/*
 * flce.h -- fused linear cross-entropy (forward + backward) for AMD Instinct
 * MI355X (gfx950), C ABI.
 *
 * The operation (blog page "Liger Kernel: Fused Triton Kernels for LLM
 * Training"; section "1. Fused Linear Cross-Entropy with Online LogSumExp",
 * steps 1-5, and section "2. In-Kernel Gradient Computation During the
 * Backward Pass"; the call shape is the LigerFusedLinearCrossEntropyLoss
 * example of the lecture page "GPU MODE lecture 028 - Liger Kernel"):
 *
 *   z_i   = W . h_i                      logits of token i, never stored whole
 *   lse_i = m_i + log sum_j exp(z_ij - m_i),   m_i = max_j z_ij
 *   loss  = scale * sum_{i valid} (lse_i - z_{i,y_i})
 *   G_ij  = scale_i * (exp(z_ij - lse_i) - [j == y_i])
 *   dH    = G . W                        [n, d]
 *   dW    = G^T . H                      [v, d]
 *
 * A row is valid when its label differs from ignore_index.  scale = 1/n_valid
 * for FLCE_MEAN (0 when n_valid == 0: loss and gradients are then 0) and 1
 * for FLCE_SUM; scale_i = scale for valid rows and 0 for ignored rows.
 * The gradients are those of the returned loss for an upstream gradient of 1.
 *
 * Layout: every tensor pointer is a DEVICE pointer to a dense row-major array:
 *   h [n, d], w [v, d], dh_out [n, d], dw_out [v, d] in `dtype`;
 *   labels int64 [n]; lse_out fp32 [n]; loss_out fp32 [1].
 * h, w, dh_out and dw_out must be 16-byte aligned and d * sizeof(dtype) must
 * be a multiple of 16 (every row starts on a 16-byte boundary); otherwise
 * FLCE_ERR_ALIGNMENT.  labels must be 8-byte aligned, lse_out and loss_out
 * 4-byte aligned.
 *
 * Arithmetic: products accumulate in fp32 (bf16 inputs feed bf16 matrix
 * instructions with fp32 accumulation); loss and lse are fp32; dh_out and
 * dw_out are rounded to `dtype` with round-to-nearest-even.  The full [n, v]
 * logits tensor is never allocated: calls that compute gradients process
 * token rows in chunks of fewer than n rows (for n >= 32); forward-only calls
 * keep no logits at all, only per-row partials of each vocabulary group, and
 * take as many rows per chunk as those fit the workspace budget.  See
 * flce_plan_info().
 *
 * Ownership: the caller owns every argument buffer; inputs are only read,
 * outputs are overwritten (never accumulated into) and must not alias the
 * inputs or each other.  The library allocates its transient workspace
 * stream-ordered on `stream` from a library-owned memory pool and releases it
 * stream-ordered before returning; its size is flce_workspace_bytes().  The
 * pool keeps released memory cached for reuse by later calls.
 *
 * Synchronisation: calls enqueue kernels on `stream` (0 = the null stream) and
 * return without waiting; results are ready when the stream reaches that
 * point.  Calls on different streams may run concurrently.
 *
 * Errors: 0 on success or a negative FLCE_ERR_* code.  Arguments are checked
 * before anything is enqueued, so a failed call writes nothing.  No exception
 * crosses this interface and nothing aborts.
 *
 * Labels: each label must be ignore_index or lie in [0, v).  Any other value
 * is a caller error that is not diagnosed on the device: the kernels index
 * memory with a label only after checking that it lies in [0, v), and such a
 * row counts as valid with a target logit of 0 and no one-hot term.
 *
 * Environment overrides (read at every call and by flce_plan_info and
 * flce_workspace_bytes; meant for tests and tuning, positive integers only,
 * anything else is ignored): FLCE_CHUNK_ROWS (token rows per chunk, capped at
 * n), FLCE_WORKSPACE_CAP_BYTES (budget for one chunk's probability buffer,
 * default 1 GiB; plans of four or more bf16 chunks with gradients hold two),
 * FLCE_LOWMEM_BUFFER_BYTES (flce_fwd_bwd_lowmem's slice budget, default 256 MiB),
 * FLCE_DW_PAIR_CHUNKS (fewest chunks that pair, default 4), FLCE_DH_SPLITS
 * (split of dH's vocabulary reduction), FLCE_GROUP_LOGITS,
 * FLCE_GROUP_DH, FLCE_GROUP_DW (tile-order group sizes of the three
 * contractions on the bf16 engine), FLCE_INPLACE_GRAD (1: flce_fwd_bwd on the
 * bf16 engine rewrites the stored probabilities into G in place instead of
 * applying the softmax factor per row; see flce_fwd_bwd).  Results stay within the
 * stated tolerances under any of them; bitwise results can change.
 * FLCE_TEST_ALLOC_LIMIT_BYTES is a test hook: a workspace request above that
 * many bytes fails as an allocation failure would (FLCE_ERR_OOM, nothing
 * enqueued, nothing written).
 */
#ifndef FLCE_H_
#define FLCE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of h, w, dh_out and dw_out. */
typedef enum { FLCE_BF16 = 0, FLCE_F32 = 1 } flce_dtype;

/* Loss reduction over the valid rows. */
typedef enum { FLCE_MEAN = 0, FLCE_SUM = 1 } flce_reduction;

enum {
  FLCE_OK = 0,
  FLCE_ERR_INVALID_ARG = -1, /* null required pointer, n/d/v <= 0, n >= 2^31, d > 2^24, v > 2^24 - 256, unknown enum,
                                size overflow */
  FLCE_ERR_ALIGNMENT = -2,   /* pointer or row pitch not aligned as documented above */
  FLCE_ERR_OOM = -3,         /* workspace allocation failed */
  FLCE_ERR_HIP = -4,         /* a HIP runtime call or kernel launch failed */
  FLCE_ERR_SCRATCH = -5      /* flce_fwd_noalloc: the sizes need more than its fixed scratch area */
};

/*
 * Loss, per-row log-sum-exp and both gradients in one call.
 * Forward: section "1. Fused Linear Cross-Entropy with Online LogSumExp"
 * (chunked streaming, online LSE, target extraction); backward: section
 * "2. In-Kernel Gradient Computation During the Backward Pass" (softmax minus
 * one-hot, dH = G.W, dW = G^T.H), computed in the same pass from the chunk's
 * logits rather than by recomputing them.  On the bf16 engine (vocabulary
 * rounded up to 256 at least 2 d) the chunk's probabilities are stored against
 * one reference per row and the row's softmax factor is applied to dH's
 * output rows and to a bf16 copy of the chunk's H that dW reads
 * (G = diag(F) P', so G.W = diag(F) (P'.W) and G^T.H = P'^T (diag(F) H)).
 *
 *   h, w           inputs, see Layout above.
 *   labels         int64 [n]; ignore_index marks rows that do not count.
 *   n, d, v        tokens, hidden size, vocabulary size (all > 0; n < 2^31,
 *                  since the count of valid rows is 32-bit; d <= 2^24 and
 *                  v <= 2^24 - 256).
 *   dtype          element type of h, w, dh_out, dw_out.
 *   reduction      FLCE_MEAN or FLCE_SUM.
 *   loss_out       fp32 [1], required.
 *   lse_out        fp32 [n] or NULL; the LSE of every row, ignored rows included.
 *   dh_out, dw_out required; overwritten.
 *   stream         HIP stream the work is enqueued on.
 */
int flce_fwd_bwd(const void* h, const void* w, const int64_t* labels,
                 int64_t n, int64_t d, int64_t v, flce_dtype dtype,
                 int64_t ignore_index, flce_reduction reduction,
                 float* loss_out, float* lse_out, void* dh_out, void* dw_out,
                 hipStream_t stream);

/*
 * Forward only: loss and (optionally) the per-row LSE, the two quantities the
 * forward keeps: section "1. Fused Linear Cross-Entropy with Online
 * LogSumExp", step 5, retains just the loss and each row's normaliser.
 * Arguments as for flce_fwd_bwd.
 */
int flce_fwd(const void* h, const void* w, const int64_t* labels,
             int64_t n, int64_t d, int64_t v, flce_dtype dtype,
             int64_t ignore_index, flce_reduction reduction,
             float* loss_out, float* lse_out, hipStream_t stream);

/*
 * flce_fwd without any allocation, for callers that cannot allocate device
 * memory during the call: code being captured into a HIP graph, tight serving
 * or scoring loops, harnesses that forbid allocation.  Same arguments, results
 * and errors as flce_fwd (loss and LSE bitwise equal to it), but the workspace
 * is a fixed scratch area of FLCE_NOALLOC_SCRATCH_BYTES (64 MiB) of device
 * memory that the library holds on each device it runs on until the process
 * ends; the chunk of token rows per launch shrinks until the workspace fits.
 * Sizes that need more than the area even at the smallest chunk (about
 * 8 n + 8 ceil(v / 128) * 16 bytes) return FLCE_ERR_SCRATCH before anything
 * is enqueued.  Every call on one device shares that device's area: calls
 * that overlap on one GPU (different streams, or different host threads
 * without ordering) race on it and must be serialised by the caller.
 */
#define FLCE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int flce_fwd_noalloc(const void* h, const void* w, const int64_t* labels,
                     int64_t n, int64_t d, int64_t v, flce_dtype dtype,
                     int64_t ignore_index, flce_reduction reduction,
                     float* loss_out, float* lse_out, hipStream_t stream);

/*
 * Low-memory variant of flce_fwd_bwd: the same loss, LSE and gradients (same
 * arguments, layouts, errors and stream semantics) from a workspace of about
 * 4 n d + 256 MiB bytes instead of one chunk's [C, v] buffer plus a v x d
 * running sum.  The forward statistics run over the whole vocabulary first;
 * the backward then walks the vocabulary in slices of vb rows, recomputing each
 * slice's logits from the saved LSE and turning them into G (blog page,
 * section "2. In-Kernel Gradient Computation During the Backward Pass": the
 * backward recomputes tile logits from the per-token LSE).  Each slice's dW
 * rows are one reduction over every token (fp32 accumulation, rounded once);
 * dH sums the slices' terms in fp32.  Cost: 8 N D V flop instead of 6.
 * The slice buffer holds vb = FLCE_LOWMEM_BUFFER_BYTES / (2 n) vocabulary
 * rows (bf16; 4 n for fp32), rounded down to a multiple of 256, default
 * budget 256 MiB; see flce_lowmem_plan_info().
 */
int flce_fwd_bwd_lowmem(const void* h, const void* w, const int64_t* labels,
                        int64_t n, int64_t d, int64_t v, flce_dtype dtype,
                        int64_t ignore_index, flce_reduction reduction,
                        float* loss_out, float* lse_out, void* dh_out, void* dw_out,
                        hipStream_t stream);

/*
 * Backward pass from the saved per-token LSE, recomputing the logits: the
 * backward of the blog page "Liger Kernel: Fused Triton Kernels for LLM
 * Training", section "2. In-Kernel Gradient Computation During the Backward
 * Pass" (the forward keeps only the LSE; the backward recomputes the tile
 * logits and forms softmax - one-hot from it).  Together with flce_fwd it
 * splits flce_fwd_bwd into the forward and backward halves an autograd
 * function needs, at 8 N D V flop instead of 6.
 *
 *   lse       device, [n] fp32: the LSE flce_fwd (or flce_fwd_bwd) returned
 *             for these h, w; read only.
 *   grad_out  device, one fp32: the upstream gradient of the loss (the
 *             scalar autograd passes to the loss's backward), or NULL for 1.
 *             Read by the kernels, so no host synchronisation is needed.
 *   dh_out    device, [n, d] in dtype: overwritten with grad_out * dloss/dH.
 *   dw_out    device, [v, d] in dtype: overwritten with grad_out * dloss/dW.
 * Other arguments, layouts, ownership, stream semantics and error codes as
 * for flce_fwd_bwd.  h, w, labels and ignore_index/reduction must be those
 * of the forward call; a different lse gives the gradient of a different
 * function, which is not checked.
 */
int flce_bwd(const void* h, const void* w, const int64_t* labels, const float* lse, const float* grad_out,
             int64_t n, int64_t d, int64_t v, flce_dtype dtype, int64_t ignore_index, flce_reduction reduction,
             void* dh_out, void* dw_out, hipStream_t stream);

/*
 * Cross-entropy on logits the caller already holds ([n, v], row-major, dtype
 * bf16 or fp32): the LigerCrossEntropyLoss example of the lecture page "GPU
 * MODE lecture 028 - Liger Kernel" (logits as a [B*S, vocab] view) -- per-row
 * log-sum-exp, target logit and loss as in the blog page's
 * section "1. Fused Linear Cross-Entropy with Online LogSumExp" steps 3-5, and
 * the gradient softmax - one-hot of its section "2. In-Kernel Gradient
 * Computation During the Backward Pass", without the GEMM.
 *
 *   logits     device, [n, v] in dtype; read only unless grad_out == logits.
 *   lse_in     device, [n] fp32 or NULL.  NULL: compute the LSE and the loss.
 *              Non-NULL: the LSE of these logits (a backward from the saved
 *              LSE); loss_out and lse_out are then not written.
 *   grad_scale device, one fp32 multiplying the gradient (the upstream
 *              gradient of the loss), or NULL for 1.
 *   loss_out   device, one fp32; required when lse_in is NULL.
 *   lse_out    device, [n] fp32, or NULL.
 *   grad_out   device, [n, v] in dtype, or NULL for no gradient; may equal
 *              logits (the gradient then overwrites the logits in place);
 *              required when lse_in is given.  Ignored rows get zero rows.
 * Stream-ordered; errors as for flce_fwd_bwd (FLCE_ERR_ALIGNMENT when a
 * pointer is not aligned to its element size).
 */
int flce_ce_logits(const void* logits, const int64_t* labels, int64_t n, int64_t v, flce_dtype dtype,
                   int64_t ignore_index, flce_reduction reduction, const float* lse_in, const float* grad_scale,
                   float* loss_out, float* lse_out, void* grad_out, hipStream_t stream);

/*
 * Forward (loss and per-row LSE) from FP8 inputs: H and W as OCP e4m3 bytes
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; 0x7f/0xff are NaN),
 * each row with an fp32 scale, so that
 *   z_ij = h_scale[i] * w_scale[j] * sum_k e4m3(h_q[i, k]) * e4m3(w_q[j, k]).
 * The pages raise FP8 only as an open question of the lecture page "GPU MODE
 * lecture 028 - Liger Kernel" (FP8 training on newer GPUs) and give no method;
 * this call takes quantised inputs and computes exactly the loss of
 * flce_fwd on the dequantised H and W: the products are exact and accumulate
 * in fp32 on the matrix cores' fp8 instructions; the online LSE, target
 * extraction and loss are those of flce_fwd.
 *
 *   h_q      device, [n, d] e4m3 bytes, 16-byte aligned;  h_scale  device, fp32 [n].
 *   w_q      device, [v, d] e4m3 bytes, 16-byte aligned;  w_scale  device, fp32 [v], 16-byte aligned.
 *   d        a multiple of 16 (FLCE_ERR_ALIGNMENT otherwise).
 * labels, ignore_index, reduction, loss_out, lse_out, stream and errors as for flce_fwd;
 * the workspace is flce_workspace_bytes(n, d / 2, v, FLCE_BF16, 0).
 */
int flce_fwd_fp8(const void* h_q, const float* h_scale, const void* w_q, const float* w_scale, const int64_t* labels,
                 int64_t n, int64_t d, int64_t v, int64_t ignore_index, flce_reduction reduction, float* loss_out,
                 float* lse_out, hipStream_t stream);

/*
 * Backward from the saved LSE for the FP8 inputs of flce_fwd_fp8: dH and dW of
 * grad_out * loss with respect to the dequantised H and W (what a caller that
 * keeps fp8 copies of bf16 weights updates them with).  The logits are
 * recomputed from the e4m3 operands exactly as flce_fwd_fp8 formed them and
 * turned into G = softmax - onehot (scaled) as in flce_bwd; the two
 * contractions run on bf16 copies of the dequantised H and W (rounded to
 * nearest even), which the call keeps in its workspace (2 (n + v) d bytes more
 * than flce_bwd's).
 *   lse, grad_out   as for flce_bwd (lse from flce_fwd_fp8 on the same inputs).
 *   dh_out, dw_out  device, bf16 [n, d] and [v, d], 16-byte aligned; overwritten.
 * Other arguments and errors as for flce_fwd_fp8.
 */
int flce_bwd_fp8(const void* h_q, const float* h_scale, const void* w_q, const float* w_scale, const int64_t* labels,
                 const float* lse, const float* grad_out, int64_t n, int64_t d, int64_t v, int64_t ignore_index,
                 flce_reduction reduction, void* dh_out, void* dw_out, hipStream_t stream);

/*
 * Vocabulary shards.  The vocabulary rows of W are split into contiguous
 * shards [v_first, v_first + v_shard); each shard's partial statistics are
 * computed on its own and merged exactly, because the log-sum-exp of a row is
 * the log-sum-exp of its shards' log-sum-exps.  This is the vocabulary split
 * the lecture page "GPU MODE lecture 028 - Liger Kernel" leaves open for
 * vocabularies of a million ids and more (its open questions), built from the
 * online-LSE merge of the blog page's section "1. Fused Linear Cross-Entropy
 * with Online LogSumExp" (step 3), and the per-GPU half of a vocabulary-
 * parallel loss: one GPU per shard, the partials exchanged in between.
 * On one GPU a caller loops over the shards: flce_fwd_shard for each, then
 * flce_merge_shards, then flce_bwd_shard for the first shard and
 * flce_bwd_shard_accumulate for the others with the merged LSE (one fp32 dH
 * sum), then flce_sum_parts over that one part to round it to dtype.
 *
 * Labels are the full-vocabulary ids (ignore_index or [0, V)); a shard sees
 * the labels outside it as "no target in this shard".  A shard call's
 * workspace is flce_workspace_bytes(n, d, v_shard, dtype, 0) (forward) or
 * flce_workspace_bytes(n, d, v_shard, dtype, 2) (backward) plus 8 n bytes
 * (the shard's shifted labels).
 */

/*
 * Partial forward of one shard.
 *   w_shard       device, [v_shard, d] in dtype: rows v_first .. v_first + v_shard - 1 of W.
 *   v_first       first vocabulary id of the shard (>= 0).
 *   lse_part_out  device, fp32 [n]: log sum over the shard's columns of exp(z_ij), every row.
 *   zy_part_out   device, fp32 [n]: z_{i, y_i} when y_i lies in the shard, else 0 (0 for ignored rows).
 * h, labels, n, d, dtype, ignore_index, layouts and errors as for flce_fwd_bwd.
 */
int flce_fwd_shard(const void* h, const void* w_shard, const int64_t* labels, int64_t n, int64_t d, int64_t v_shard,
                   int64_t v_first, flce_dtype dtype, int64_t ignore_index, float* lse_part_out, float* zy_part_out,
                   hipStream_t stream);

/*
 * Merge num_shards partials into the loss and the per-row LSE.
 *   lse_parts, zy_parts  device, fp32 [num_shards][n] (shard q's flce_fwd_shard outputs at offset q * n).
 *   loss_out             device, one fp32; the loss of flce_fwd_bwd over the whole vocabulary.
 *   lse_out              device, fp32 [n] or NULL; the whole-vocabulary LSE (flce_bwd_shard's lse).
 * Stream-ordered; errors as for flce_fwd_bwd.
 */
int flce_merge_shards(const float* lse_parts, const float* zy_parts, int64_t num_shards, const int64_t* labels,
                      int64_t n, int64_t ignore_index, flce_reduction reduction, float* loss_out, float* lse_out,
                      hipStream_t stream);

/*
 * Backward of one shard from the whole-vocabulary LSE (logits recomputed, as
 * flce_bwd): the shard's columns of G = (softmax - onehot) * scale * grad_out.
 *   lse           device, fp32 [n]: the merged LSE from flce_merge_shards.
 *   grad_out      device, one fp32 upstream gradient, or NULL for 1.
 *   dh_part_out   device, fp32 [n, d] (whatever dtype is): this shard's term G_q . W_q of dH;
 *                 dH is the sum over the shards (flce_sum_parts).  16-byte aligned.
 *   dw_shard_out  device, [v_shard, d] in dtype: rows v_first .. v_first + v_shard - 1 of dW.
 * Other arguments as for flce_fwd_shard and flce_bwd.
 */
int flce_bwd_shard(const void* h, const void* w_shard, const int64_t* labels, const float* lse, const float* grad_out,
                   int64_t n, int64_t d, int64_t v_shard, int64_t v_first, flce_dtype dtype, int64_t ignore_index,
                   flce_reduction reduction, float* dh_part_out, void* dw_shard_out, hipStream_t stream);

/*
 * flce_bwd_shard with the shard's dH term added to dh_acc (fp32 [n, d], 16-byte
 * aligned) instead of written over it, so that the shards of one GPU share one
 * fp32 sum; every other argument and error as for flce_bwd_shard.  Calls that
 * add into the same dh_acc must be ordered (one stream), as the sum is not atomic.
 */
int flce_bwd_shard_accumulate(const void* h, const void* w_shard, const int64_t* labels, const float* lse,
                              const float* grad_out, int64_t n, int64_t d, int64_t v_shard, int64_t v_first,
                              flce_dtype dtype, int64_t ignore_index, flce_reduction reduction, float* dh_acc,
                              void* dw_shard_out, hipStream_t stream);

/*
 * out[i] = sum_q parts[q * count + i] for i < count, accumulated in fp32 in
 * shard order and rounded to dtype (round-to-nearest-even for bf16): the dH
 * of a vocabulary-split backward from its shards' partials.
 *   parts  device, fp32 [num_parts][count];  out  device, [count] in dtype.
 */
int flce_sum_parts(const float* parts, int64_t num_parts, int64_t count, flce_dtype dtype, void* out,
                   hipStream_t stream);

/*
 * x[i] *= *scale for i < count, in place: the fp32 product rounded to dtype
 * (round-to-nearest-even for bf16).  The scale is read on the device, so a
 * caller can hand over an upstream gradient without a host synchronisation;
 * a scale of exactly 1 leaves x untouched.  This applies the upstream
 * gradient of the loss (the gradients are those of upstream * loss) to the
 * dH and dW that flce_fwd_bwd computed in the same pass as the loss, as an
 * autograd function whose forward runs flce_fwd_bwd does in its backward.
 *   x      device, [count] in dtype, 16-byte aligned; count in (0, 2^40].
 *   scale  device, one fp32.
 * FLCE_ERR_INVALID_ARG / FLCE_ERR_ALIGNMENT before anything is enqueued.
 */
int flce_scale(void* x, int64_t count, flce_dtype dtype, const float* scale, hipStream_t stream);

/*
 * Bytes of device workspace one call allocates (with_bwd = 0 for flce_fwd,
 * 2 for flce_bwd, 1 or any other value for flce_fwd_bwd); 0 for invalid sizes.  Honours the
 * FLCE_CHUNK_ROWS and FLCE_WORKSPACE_CAP_BYTES environment overrides exactly
 * as the calls do.
 */
size_t flce_workspace_bytes(int64_t n, int64_t d, int64_t v, flce_dtype dtype, int with_bwd);

/* Execution plan a call with these sizes uses (host-only; no device access). */
typedef struct {
  int64_t chunk_rows;      /* token rows per chunk */
  int64_t num_chunks;
  int64_t vocab_pitch;     /* padded row length of the chunk's probability buffer */
  int64_t group_cols;      /* vocabulary columns per partial (max, sum-exp) pair */
  int64_t dh_splits;       /* split of the vocabulary reduction in dH = G.W */
  int32_t engine;          /* 0: bf16 matrix-core engine, 1: fp32 FMA engine */
  int32_t dw_accumulator;  /* 1 if dW keeps the lower 16 bits of its fp32 running sum in the workspace */
  size_t workspace_bytes;
  size_t prob_buffer_bytes;   /* the chunks' [chunk_rows, vocab_pitch] buffer(s) */
  int32_t dw_pairs;        /* 1 if two chunk buffers sit side by side and each dW launch covers two chunks */
  int32_t folded_factor;   /* 1 if the one-pass backward applies the softmax factor per row, to dH's rows
                              and to a bf16 copy of the chunk's H that dW reads (matrix engine, vocabulary
                              pitch at least 2 d) */
} flce_plan_t;

/* Fill *out with the plan for these sizes; returns 0 or FLCE_ERR_INVALID_ARG. */
int flce_plan_info(int64_t n, int64_t d, int64_t v, flce_dtype dtype, int with_bwd, flce_plan_t* out);

/* Workspace bytes of flce_fwd_bwd_lowmem (0 for invalid sizes); host-only. */
size_t flce_workspace_bytes_lowmem(int64_t n, int64_t d, int64_t v, flce_dtype dtype);

/* Plan of flce_fwd_bwd_lowmem (host-only). */
typedef struct {
  int64_t slice_cols;          /* vocabulary rows per slice (the last slice may be narrower) */
  int64_t num_slices;
  int64_t slice_chunk_rows;    /* token rows per chunk inside a slice (n when one chunk holds them all) */
  int64_t slice_chunks;
  int64_t fwd_chunk_rows;      /* token rows per launch of the forward statistics */
  size_t buffer_budget_bytes;  /* the budget the slice width was chosen for */
  size_t workspace_bytes;
} flce_lowmem_plan_t;
int flce_lowmem_plan_info(int64_t n, int64_t d, int64_t v, flce_dtype dtype, flce_lowmem_plan_t* out);

/* Static text for a status code. */
const char* flce_strerror(int status);

/*
 * Kernel timing instrumentation.  While enabled, every kernel launch of later
 * calls is bracketed by HIP events on the call's stream.  flce_profile_read()
 * waits for those events and reports, per kernel kind, the number of launches
 * and their total duration in milliseconds since the last read, then resets
 * the counters.  Kinds: see flce_profile_kind_name().  Not thread-safe; meant
 * for benchmarks.
 */
int flce_profile_enable(int on);
int flce_profile_read(int max_kinds, int64_t* launches, double* total_ms);
const char* flce_profile_kind_name(int kind);

/*
 * High-water mark, in bytes, of the workspace the library's memory pool on
 * the current device has handed out since the last reset (reset != 0 resets
 * it after reading).  Lets a caller compare the extra device memory of a call
 * with the [n, v] logits it does not allocate.
 */
int flce_memory_high_water(int reset, uint64_t* used_high_bytes);

/*
 * The library's pool on the current device keeps the memory of released
 * workspaces reserved for later calls.  flce_memory_reserved() reports how
 * many bytes it holds now; flce_pool_trim() returns all but keep_bytes of the
 * unused part to the device (call it after a synchronisation point, e.g. at
 * the end of a training step, to give that memory back to other allocators).
 */
int flce_memory_reserved(uint64_t* reserved_bytes);
int flce_pool_trim(uint64_t keep_bytes);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_H_ */
