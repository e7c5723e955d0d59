/*
 * vsce.h -- C ABI of the fused large-vocabulary softmax cross-entropy
 * (libvsce.so, HIP for MI355X / gfx950).
 *
 * For each row n of a [rows, vocab] logits matrix x with target y[n] the
 * library computes, in one pass over the row,
 *   m = max_c x[c], d' = sum_{c != first argmax} exp(x[c] - m), x[y], and
 *   S = sum_c w[c] x[c] (only needed under label smoothing),
 * from them the row loss
 *   l = (1 - eps) w[y] (lse - x[y]) + (eps / V) sum_c w[c] (lse - x[c]),
 *   lse = m + log1p(d'),
 * its none / sum / mean reduction (mean divides by W = sum of w[y] over rows
 * whose target is not ignored), the token accuracy, and the logits gradient
 *   g[c] = sigma (p[c] ((1 - eps) w[y] + (eps / V) sum_k w[k]) - (eps / V) w[c]
 *                 - (1 - eps) w[y] [c == y]),   p = softmax(x),
 * computed in fp32 and rounded once to the buffer type.  The true-class term
 * is evaluated once per row from the live m, d' and x[y] and written with a
 * single store (no per-element compare, no read-modify-write).  Optionally
 * the logits are soft-capped first (x -> s tanh(x / s), gradient times
 * 1 - tanh^2) and a z-loss lambda lse^2 is added per valid row (its gradient
 * 2 lambda lse p[c], scaled by 1 / valid rows under mean): see vsce_problem.
 *
 * Sources (page titles and sections):
 *  - Liger-Kernel PR #1268 "perf(ce): single-shot dx_y gradient correction":
 *    the pass-2 gradient hunks, the O(1) true-class correction, and the
 *    embedded commit message of linkedin#1329 (recompute dx_y in fp32 from
 *    the live target logit, max and sum, one store); the embedded commit
 *    message of linkedin#1290 ("The optimization: CE backward memory parity":
 *    scale the saved gradient in place through a raw element-wise kernel).
 *  - Liger-Kernel PR #1622 "perf(flce): drop host syncs that do not feed the
 *    computation", Summary: count / target-weight sum for mean, class-weight
 *    sum times eps = label_smoothing / V, accuracy divided by the count on the
 *    device, grad_output == 1.0 checked on the device (SKIP_IF_ONE).
 *  - TransformerEngine PR #2325 "change fused cross entropy backward grad to
 *    fp32 and reduce one read/write", Greptile summary and sequence diagram:
 *    the forward saves per-row (max, sum, target logit, scaled_x_sum) and the
 *    backward recomputes the gradient in fp32 from them.
 *
 * Conventions for every entry point:
 *  - Every pointer argument is caller-owned DEVICE memory unless stated
 *    otherwise; the problem and output descriptors themselves are host
 *    structs read during the call only.
 *  - The library allocates no memory, never synchronizes the stream or the
 *    device, and never reads device data on the host: all work is enqueued on
 *    `stream` (NULL = the null stream) and the call returns at once.
 *  - Return codes: VSCE_OK (work enqueued), VSCE_ERR_INVALID (an argument is
 *    out of its documented domain; nothing was enqueued),
 *    VSCE_ERR_UNSUPPORTED (a valid combination the library does not handle;
 *    nothing enqueued), VSCE_ERR_LAUNCH (a kernel launch failed).
 *  - Data-dependent errors (a target neither equal to ignore_index nor in
 *    [0, vocab)) are not return codes: the row gets a NaN loss and a zero
 *    gradient, is left out of W and of the valid count, and bit
 *    VSCE_STATUS_BAD_TARGET is set in the workspace status word, which the
 *    caller may read whenever it chooses.
 *  - Calls are reentrant.  Two calls that share a workspace must be ordered
 *    on one stream.  The library's only mutable state is the static workspace
 *    of ce_forward_fused_inplace_noalloc (one per device) and the launch
 *    shapes of the GEMM, computed once per device and kept.
 */
#ifndef VSCE_H
#define VSCE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of the logits / gradient buffer. */
typedef enum vsce_dtype { VSCE_F32 = 0, VSCE_BF16 = 1, VSCE_F16 = 2 } vsce_dtype;

/* Reduction of the per-row losses (PyTorch's names). */
typedef enum vsce_reduction {
  VSCE_REDUCTION_NONE = 0,
  VSCE_REDUCTION_MEAN = 1,
  VSCE_REDUCTION_SUM = 2
} vsce_reduction;

enum {
  VSCE_OK = 0,
  VSCE_ERR_INVALID = -1,
  VSCE_ERR_UNSUPPORTED = -2,
  VSCE_ERR_LAUNCH = -3,
  VSCE_ERR_TOO_LARGE = -4 /* ce_forward_fused_inplace_noalloc: more rows than
                             its static workspace holds; nothing enqueued */
};

/* Bits of the workspace status word. */
#define VSCE_STATUS_BAD_TARGET 1u

/* Floats per row of the saved statistics: (m, d', x[y], S); S = 0 when
   label_smoothing == 0; d' = d - 1 (the sum with the first maximum left out). */
#define VSCE_STATS_STRIDE 4
/* fp32 per row of a vocab-parallel shard record (ce_forward_stats_partial). */
#define VSCE_PARTIAL_STRIDE 8

/* vsce_problem.flags: in the fused forward, rows too long for the on-chip
   kernel take one launch that streams each row twice through a ring of LDS
   stages (direct-to-LDS loads), instead of the default two launches (the
   statistics kernel, then the gradient kernel in place).  Only rows on
   16-byte vectors without class weights can; the others keep the default. */
#define VSCE_FLAG_LONG_ROWS_RING 1u

/*
 * Workspace: caller-allocated device memory of vsce_workspace_bytes(rows)
 * bytes, 256-byte aligned.  Its first 256 bytes are a header the forward
 * writes and the backward reads (so a forward and its backward must get the
 * same workspace); after it come per-row scratch arrays (row losses,
 * accuracies, z-losses, and the statistics of the fused mode's rows that are
 * too long for the chip).  Its contents need no initialisation.  Header
 * fields, at these byte offsets:
 */
#define VSCE_WS_W 0          /* double: W, target-weight sum over valid rows  */
#define VSCE_WS_SUM_W 8      /* double: class-weight sum (vocab if unweighted) */
#define VSCE_WS_N_VALID 16   /* int64: rows whose target is in [0, vocab)     */
#define VSCE_WS_N_INVALID 24 /* int64: rows with a bad target                 */
#define VSCE_WS_STATUS 32    /* uint32: VSCE_STATUS_* bits of the last forward */
#define VSCE_WS_INV_W 40     /* float: 1 / W, rounded once to fp32             */
#define VSCE_WS_INV_N_VALID 44 /* float: 1 / (rows whose target is in range)   */
#define VSCE_WS_HEADER_BYTES 256

/* Bytes of workspace a problem with `rows` rows needs (0 if rows < 0). */
size_t vsce_workspace_bytes(int64_t rows);

/*
 * The problem: one [rows, vocab] matrix and its targets.
 *  rows            BT >= 0 (0 is allowed: nothing to do but the reduction)
 *  vocab           V >= 1
 *  row_stride      elements between the starts of consecutive rows, >= vocab
 *  dtype           vsce_dtype of the logits / gradient buffer
 *  reduction       vsce_reduction
 *  target          [rows] int64 class ids (device)
 *  class_weight    [vocab] fp32 weights (device) or NULL for all ones
 *  ignore_index    target value of rows to ignore (PyTorch default -100); it
 *                  is tested before the range check, so it may lie in [0, V)
 *  label_smoothing eps in [0, 1]
 *  softcap         s >= 0, finite.  s > 0 replaces every logit x by the
 *                  capped logit s * tanh(x / s) before anything else reads it
 *                  (maximum, softmax, smoothing sum, statistics), and the
 *                  gradient with respect to x takes the factor
 *                  1 - tanh^2(x / s); s = 0 leaves the logits as they are.
 *                  (Liger-Kernel PR #1268 names soft-capping among the CE
 *                  features its target correction keeps, What changed and
 *                  Correctness; this is the plain definition.)  The token
 *                  accuracy compares the target with the maximum of the stored
 *                  logits, which capping does not reorder.  The capped value
 *                  and its slope are within a few units of 2^-24 relative for
 *                  caps up to 1e6; past about 1.3e6 the highest coefficient of
 *                  the polynomial used for |x| <= 0.35 s (kept as P3 / s^6)
 *                  leaves fp32's normal range, which costs accuracy only for
 *                  logits within a factor of about 30 of s.
 *  z_loss          lambda >= 0, finite.  Adds lambda * lse^2 to the loss of
 *                  every valid row, lse being the log-sum-exp of the (capped)
 *                  logits (the z-loss that PR #1268 lists in its Correctness
 *                  section).  It is not multiplied by class weights, and the
 *                  mean reduction divides it by the number of valid rows
 *                  (the cross-entropy part keeps W).  0: off.
 *  flags           0 or VSCE_FLAG_LONG_ROWS_RING (a choice of kernels for the
 *                  fused forward, see ce_forward_fused_inplace); other bits
 *                  are rejected.
 *  vocab_offset    for one shard of a vocab-parallel layout (TransformerEngine
 *                  PR #2325, dist_process_group): the global column of this
 *  vocab_total     buffer's first column, and the full vocabulary size V
 *                  (vocab_total = 0 means vocab, i.e. no sharding).  Targets
 *                  are global class ids in [0, vocab_total); class_weight, if
 *                  given, holds all vocab_total weights (one shard reads its
 *                  slice and w[y]); eps is divided by vocab_total.  Only
 *                  ce_forward_stats_partial and ce_backward_from_stats take a
 *                  sharded problem; the other entry points require
 *                  vocab_offset == 0 and vocab_total in {0, vocab}.
 */
typedef struct vsce_problem {
  int64_t rows;
  int64_t vocab;
  int64_t row_stride;
  int32_t dtype;
  int32_t reduction;
  const int64_t *target;
  const float *class_weight;
  int64_t ignore_index;
  float label_smoothing;
  float softcap;
  float z_loss;
  uint32_t flags;   /* 0, or VSCE_FLAG_LONG_ROWS_RING */
  int64_t vocab_offset;
  int64_t vocab_total;
} vsce_problem;

/*
 * Forward outputs (all device fp32):
 *  loss       required; [1] for mean and sum, [rows] for none.  A mean over
 *             zero valid rows is NaN; a bad target makes the reduced loss NaN.
 *  row_loss   optional [rows]: the unreduced per-row loss (0 for ignored rows).
 *  token_acc  optional [rows]: 1 where the row is valid and the first index of
 *             its maximum equals the target, else 0.
 *  acc_mean   optional [1]: the mean of token_acc over valid rows (NaN if none).
 *  z_loss     optional: the z-loss part of the loss alone, reduced like the
 *             loss ([1] for mean, over valid rows, and sum; [rows] for none).
 *             Zeros when the problem's z_loss is 0.
 */
typedef struct vsce_outputs {
  float *loss;
  float *row_loss;
  float *token_acc;
  float *acc_mean;
  float *z_loss;
} vsce_outputs;

/*
 * Fused forward + gradient, in place (Liger-Kernel PR #1268 pass 1 / pass 2
 * with the linkedin#1329 fp32 true-class fold; PR #1622 device-side
 * normalizers).  Reads every valid row once, writes the loss outputs, and
 * overwrites `logits_inout` (a [rows, row_stride] buffer of `dtype`) with the
 * gradient of the reduced loss for grad_output = 1: sigma = 1/W for mean (and
 * 1/valid rows for the z-loss part), 1
 * for sum and none.  Ignored and bad-target rows are overwritten with zeros.
 * Columns in [vocab, row_stride) are neither read nor written.  Apply a
 * grad_output other than 1 afterwards with ce_scale_grad.
 * Rows of at most 32768 16-byte vectors (bf16 / fp16 vocab <= 262144, fp32
 * vocab <= 131072) are held on chip: one read and one write.  Longer rows,
 * and rows not on 16-byte vectors, are read twice: the statistics kernel
 * saves (m, d', x[y], S) in the workspace and the gradient kernel writes in
 * place (two launches), or, with VSCE_FLAG_LONG_ROWS_RING, one launch streams
 * each row twice through an LDS ring.
 */
int ce_forward_fused_inplace(const vsce_problem *problem, void *logits_inout,
                             const vsce_outputs *out, void *workspace,
                             hipStream_t stream);

/*
 * Measurement variant of ce_forward_fused_inplace: identical work, plus
 * hipEventRecord(begin) and hipEventRecord(end) on `stream` immediately
 * before and after the launch of the row kernel (both launches for rows read
 * twice; not the normalizer and reduction launches around them), so that the
 * caller can time the row work alone with hipEventElapsedTime.  The events are created and owned by the
 * caller; either may be NULL.  Returns VSCE_ERR_LAUNCH if recording fails.
 */
int ce_forward_fused_inplace_timed(const vsce_problem *problem, void *logits_inout,
                                   const vsce_outputs *out, void *workspace,
                                   hipStream_t stream, hipEvent_t begin, hipEvent_t end);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * work as ce_forward_fused_inplace, with the workspace taken from a static
 * array inside the library instead of a caller's buffer.  Nothing is
 * allocated: the array (vsce_workspace_bytes(VSCE_NOALLOC_MAX_ROWS) bytes,
 * about 1.8 MB) is part of the library's device code and each device the
 * library runs on holds its own copy until the process ends.  The first call
 * on a device looks up that device's copy (hipGetSymbolAddress, with the
 * device current) and keeps its address.
 *  - rows > VSCE_NOALLOC_MAX_ROWS: returns VSCE_ERR_TOO_LARGE, nothing
 *    enqueued.  Other arguments as ce_forward_fused_inplace.
 *  - Every call on one device shares that device's array, and each forward
 *    rewrites what it reads (the header and the per-row scratch need no
 *    clearing).  Calls that overlap on one device race: order them on one
 *    stream.
 *  - The header (normalizers, status word) stays inside the library: a bad
 *    target still shows as a NaN row loss and a NaN reduced loss.  The
 *    gradient needs nothing more: apply grad_output with ce_scale_grad.
 */
#define VSCE_NOALLOC_MAX_ROWS 65536
int ce_forward_fused_inplace_noalloc(const vsce_problem *problem, void *logits_inout,
                                     const vsce_outputs *out, hipStream_t stream);

/*
 * Split forward (TransformerEngine PR #2325 online_softmax_kernel +
 * cross_entropy_forward_kernel): reads the logits once and writes the loss
 * outputs and `stats` ([rows][VSCE_STATS_STRIDE] fp32: m, d', x[y], S; rows
 * that are not valid get zeros).  The logits are not modified.
 */
int ce_forward_stats(const vsce_problem *problem, const void *logits,
                     float *stats, const vsce_outputs *out, void *workspace,
                     hipStream_t stream);

/*
 * Vocab-parallel split forward, one shard (TransformerEngine PR #2325: each
 * rank of the process group computes the per-row record of its vocabulary
 * slice, to be gathered; the review asks that the 4th value be gathered and
 * summed too).  `problem` describes the shard (vocab = its width,
 * vocab_offset, vocab_total); `logits` is its [rows, row_stride] slice.
 * Writes `partial`, [rows][VSCE_PARTIAL_STRIDE] fp32 (device), per valid row:
 *   [0] m_s    the shard's maximum of the (capped) logits
 *   [1] d'_s   sum over the shard's other columns of exp(x[c] - m_s)
 *   [2] x[y] (capped) if the shard holds column y, else 0
 *   [3] S_s    sum over the shard of w[c] x[c] (0 without label smoothing)
 *   [4] the shard's maximum of the stored logits (capping does not reorder)
 *   [5] the global column of its first occurrence, as int32 bits
 *   [6], [7] 0
 * Rows that are not valid get zeros.  No loss, no workspace: the records of
 * all shards go to ce_merge_stats (gathered across devices by the caller, or
 * stacked in one buffer on one device).
 */
int ce_forward_stats_partial(const vsce_problem *problem, const void *logits,
                             float *partial, hipStream_t stream);

/*
 * Merge of `shards` partial records into the full rows' statistics:
 * `partials` holds [shards][rows][VSCE_PARTIAL_STRIDE] fp32 (device), shards
 * in increasing column order; `problem` is the full one (vocab = vocab_total,
 * vocab_offset 0; logits unused).  Per valid row:
 *   m = max_s m_s, s* the first shard attaining it,
 *   d' = d'_{s*} + sum over s != s* of (1 + d'_s) exp(m_s - m),
 *   x[y] from its owner, S = sum_s S_s, the argmax from [4] / [5];
 * then writes `stats` ([rows][VSCE_STATS_STRIDE], as ce_forward_stats), the
 * loss outputs and the workspace normalizers, exactly as ce_forward_stats
 * would for the unsharded matrix.  Each shard's gradient then comes from
 * ce_backward_from_stats with its sharded problem, these stats and this
 * workspace.
 */
int ce_merge_stats(const vsce_problem *problem, const float *partials, int32_t shards,
                   float *stats, const vsce_outputs *out, void *workspace,
                   hipStream_t stream);

/*
 * Split backward (TransformerEngine PR #2325 cross_entropy_backward_kernel):
 * from the logits and the saved stats, writes grad = RN(sigma * go[n] *
 * dl_n/dx) in fp32 with one rounding, with the true-class term folded in
 * fp32.  `grad` (a [rows, row_stride] buffer of `dtype`) may equal `logits`
 * (in place) but must not otherwise overlap it.  grad_output is fp32 device
 * memory: one value read at grad_output[0] when grad_output_stride == 0 (mean,
 * sum), or [rows] values at grad_output[n * grad_output_stride] when it is 1
 * (none).  `workspace` must be the one the matching ce_forward_stats (or
 * ce_merge_stats) wrote.  Ignored and bad-target rows get zeros.  With a
 * sharded problem, `logits` and `grad` are the shard's slices and `stats` the
 * merged ones; only the shard that holds column y writes the true-class value.
 */
int ce_backward_from_stats(const vsce_problem *problem, const void *logits,
                           void *grad, const float *stats,
                           const float *grad_output, int64_t grad_output_stride,
                           const void *workspace, hipStream_t stream);

/*
 * Scale a gradient in place by grad_output (linkedin#1290 element-wise
 * in-place scale; PR #1622 SKIP_IF_ONE): g <- RN(g * go[n]), with go read on
 * the device at grad_output[n * grad_output_stride] (stride 0: one scalar,
 * stride 1: per row).  Rows whose go equals 1.0 exactly are left untouched
 * when skip_if_one != 0, so the call costs one launch when go == 1.
 */
int ce_scale_grad(void *grad, int64_t rows, int64_t vocab, int64_t row_stride,
                  int32_t dtype, const float *grad_output,
                  int64_t grad_output_stride, int32_t skip_if_one,
                  hipStream_t stream);

/* ---------------------------------------------------------------- FLCE
 * The linear head fused with the cross-entropy (Liger-Kernel PR #1622
 * "perf(flce): drop host syncs that do not feed the computation": the FLCE
 * forward computes the loss and both gradients, chunk by chunk of rows; the
 * #1554 compaction of ignored rows out of the projection products that its
 * Details discuss is done on the device, with no host read of the count).
 */

/* bf16 GEMM on the matrix cores, used by the FLCE and callable on its own:
 * C[m][n] = sum_k A[m][k] B[n][k] with fp32 accumulation.  A is [M][lda] and B
 * [N][ldb] bf16, both contiguous along k, 16-byte aligned, lda and ldb
 * multiples of 8 with K <= lda, ldb < 2^23; K a multiple of 64.  C is
 * [M][ldc], 16-byte aligned, N and ldc multiples of 4, ldc >= N, a row of C
 * at most 2^23 bytes (ldc <= 2^22 for bf16, 2^21 for fp32).  out_mode:
 * VSCE_GEMM_OUT_BF16 (C bf16, each value rounded once to nearest even),
 * VSCE_GEMM_OUT_F32 (C fp32), VSCE_GEMM_OUT_F32_ADD (C fp32, the product added
 * to it).  Returns VSCE_ERR_INVALID for shapes outside these rules. */
#define VSCE_GEMM_OUT_BF16 0
#define VSCE_GEMM_OUT_F32 1
#define VSCE_GEMM_OUT_F32_ADD 2
int vsce_gemm_bf16_nt(const void *A, int64_t lda, const void *B, int64_t ldb, void *C,
                      int64_t ldc, int64_t M, int64_t N, int64_t K, int32_t out_mode,
                      hipStream_t stream);

/* The same product with either operand stored k-major, as the FLCE's
 * backward products need them (dL/dh = G W reads W [V][H] with k = the
 * vocabulary entry; dL/dW = G^T h reads G and h with k = the row): layout
 * VSCE_GEMM_A_K_MAJOR means A is [K][lda] with lda >= M (element (m, k) at
 * A[k * lda + m]), VSCE_GEMM_B_K_MAJOR that B is [K][ldb] with ldb >= N; an
 * operand without its bit is stored as in vsce_gemm_bf16_nt.  Leading
 * dimensions are multiples of 8 below 2^23.  Every layout gives bit-identical
 * C for the same operand values.  layout 0 is vsce_gemm_bf16_nt. */
#define VSCE_GEMM_A_K_MAJOR 1u
#define VSCE_GEMM_B_K_MAJOR 2u
int vsce_gemm_bf16(const void *A, int64_t lda, const void *B, int64_t ldb, void *C,
                   int64_t ldc, int64_t M, int64_t N, int64_t K, uint32_t layout,
                   int32_t out_mode, hipStream_t stream);

/*
 * An FLCE problem: hidden states h [rows][hidden] and the head's weight W
 * [vocab][hidden], both bf16 row-major (nn.Linear's layout), the logits
 * z = h W^T and the cross-entropy of z with the options of vsce_problem.
 *  rows          BT >= 0
 *  hidden        H: a multiple of 64
 *  vocab         V >= 1
 *  chunk_rows    rows whose logits are held at once (rounded up to a multiple
 *                of 64); 0: all rows in one chunk
 *  target .. z_loss, reduction   as in vsce_problem (no vocab sharding)
 */
typedef struct vsce_flce_problem {
  int64_t rows;
  int64_t hidden;
  int64_t vocab;
  int64_t chunk_rows;
  const int64_t *target;
  const float *class_weight;
  int64_t ignore_index;
  float label_smoothing;
  float softcap;
  float z_loss;
  int32_t reduction;
} vsce_flce_problem;

/* Bytes of workspace flce_forward_backward needs for this problem (256-byte
 * aligned device memory; 0 if the problem is invalid).  It holds the chunk's
 * logits and their transposed gradient (2 C V bytes each, C = chunk rows),
 * W^T (2 H V bytes) and the compacted hidden states and their gradient. */
size_t vsce_flce_workspace_bytes(const vsce_flce_problem *problem);

/*
 * Loss outputs (as ce_forward_fused_inplace: loss, and optionally row_loss,
 * token_acc, acc_mean, z_loss, all in the caller's row order) and both
 * gradients: grad_hidden [rows][hidden] bf16 (dL/dh, zero rows for ignored
 * rows; 16-byte aligned) and grad_weight [vocab][hidden] fp32 (dL/dW,
 * overwritten).  grad_output (device fp32) scales both gradients: one value at
 * grad_output[0] when grad_output_stride == 0, or one per row when it is 1
 * (reduction none); NULL means 1.  The logits are bf16 (each rounded once from
 * the fp32 product) and the cross-entropy's gradient G = dL/dz is bf16 when
 * it enters the two gradient products, as in the FLCE the page describes.
 * hidden and weight are 16-byte aligned; nothing is allocated and nothing
 * synchronizes.
 */
int flce_forward_backward(const vsce_flce_problem *problem, const void *hidden,
                          const void *weight, const vsce_outputs *out, const float *grad_output,
                          int64_t grad_output_stride, void *grad_hidden, float *grad_weight,
                          void *workspace, hipStream_t stream);

/* Human-readable name of a return code (static string). */
const char *vsce_strerror(int code);

/* Library version, as MAJOR * 10000 + MINOR * 100 + PATCH. */
int vsce_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VSCE_H */
