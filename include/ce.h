/*
 * ce.h -- C ABI of the MI355X (gfx950) fused cross-entropy library (libce.so).
 *
 * The library computes, for each row i of language-model logits x[N, V]
 * (FP32 or BF16, accumulated in FP32):
 *
 *   lse_i  = log sum_j exp(x_ij)
 *   loss_i = -sum_j q_ij (x_ij - lse_i)
 *   grad_ij = s_i (exp(x_ij - lse_i) - q_ij)
 *
 * with target t_i (a global vocabulary index), label smoothing a spread by
 * the smoothed target distribution q_i of one of two conventions:
 *   CE_SMOOTH_ALL:    q_ij = a / V + (1 - a) [j == t_i]
 *   CE_SMOOTH_OTHERS: q_ij = 1 - a if j == t_i, a / (V - 1) otherwise
 * rows whose target equals ignore_idx contributing loss 0 and gradient 0, and
 * s_i = g_i (per-row upstream gradient, no reduction), g / n (the mean over
 * the n non-ignored rows) or g (the sum over rows).
 *
 * Sources, by the pages' titles and sections:
 *  - interface and semantics: TransformerEngineNPU issue #29 "Parallel Cross
 *    Entropy (Triton)", section 1 (parallel_cross_entropy(inp, target,
 *    label_smoothing, reduce_loss, dist_process_group, ignore_idx=-100);
 *    (B, SQ, V) or (SQ, B, V) input; FP32 accumulation; FP32 loss; gradient
 *    written back in the input dtype) and section 6 (the gradient is staged
 *    in place in the input; the only extra buffers are loss[N] and, under
 *    vocabulary parallelism, the gathered per-rank (m, d, X_y) statistics);
 *  - the log_softmax + NLL identity and the softmax-minus-onehot gradient:
 *    CANN ops-nn page "cross-entropy fusion: three kernel launches to one",
 *    sections "fusion scheme" and "backward";
 *  - vocabulary shards: hyper-parallel issue #269, section 3.1 (forward is a
 *    MAX all-reduce, a SUM all-reduce and a target-logit gather; backward
 *    needs no collective; shards of ceil(V / tp) columns; ignore_index -100).
 *  Label smoothing: CE_SMOOTH_ALL is the uniform a/V of torch's
 *  F.cross_entropy, the precision baseline named in issue #29 section 4;
 *  CE_SMOOTH_OTHERS is the ops-nn page's kernel (forward step 4: (1 - a) NLL
 *  plus a times the mean over the other classes of -log softmax; backward
 *  "pitfall 3": 1 - a at the target, a / (V - 1) elsewhere).
 *  Reductions: issue #29's reduce_loss (mean over non-ignored rows), and the
 *  sum that the hyper-parallel #269 comparison table (row "reduction
 *  semantics") names as Titan's training default, there divided by the
 *  global count of valid tokens: CE_REDUCE_SUM with grad_out[0] = 1 / count
 *  gives that gradient with a single rounding, and loss[0] / count the loss.
 *
 * Conventions for every call:
 *  - All pointers named "device" are HIP device (or managed) memory owned by
 *    the caller; the library allocates nothing on these calls and keeps no
 *    pointer after it returns.
 *  - Calls are asynchronous on `stream` (NULL = the null stream); results are
 *    valid once the stream has reached the enqueued work.  No call
 *    synchronises the host, so the sequence can be captured in a HIP graph.
 *  - Arguments are checked on the host before any HIP call.  On an argument
 *    error the call returns a non-zero ce_status, enqueues nothing and leaves
 *    every buffer untouched; ce_last_error() then describes the problem.
 *  - A non-ignored target outside [0, vocab_total) violates the calls'
 *    precondition: no kernel reads out of bounds because of it, and that
 *    row's loss, lse and gradient are NaN.
 *  - Logical row r = i0 * d1 + i1 (0 <= i0 < d0, 0 <= i1 < d1) starts at
 *    element offset i0 * s0 + i1 * s1 of `data`; its V columns are
 *    contiguous.  (B, SQ, V) is s0 = SQ * V, s1 = V; the transposed (SQ, B, V)
 *    view of (B, SQ, V) storage is s0 = V, s1 = SQ * V.  Loss and lse are
 *    indexed by logical row.  Rows must not overlap in memory.
 */
#ifndef VCE_CE_H
#define VCE_CE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 3: ce_shards_workspace_bytes and ce_shards_fwd_bwd_fused added
 * 4: the backward hand-off pair lse_aux (ce_forward_ex, ce_shard_combine_ex,
 *    ce_backward_inplace_ex); a shard's statistic d leaves out the target
 * 5: ce_fwd_bwd_fused_noalloc
 * 6: ce_linear.gemm (was reserved): the chunked head's GEMM engine; the head's
 *    logits stride in the workspace rounded up to a multiple of 8
 * 7: ce_stream_reference */
#define CE_ABI_VERSION 7

typedef enum ce_status {
  CE_OK = 0,
  CE_EINVAL = 1,      /* NULL pointer, negative size, smoothing outside [0, 1], ... */
  CE_EDTYPE = 2,      /* logits dtype is not CE_F32 or CE_BF16 */
  CE_ELAYOUT = 3,     /* strides, alignment or shard bounds not supported */
  CE_EWORKSPACE = 4,  /* workspace NULL or smaller than required */
  CE_EHIP = 5,        /* a HIP runtime call or kernel launch failed */
  CE_EDEADLOCK = 6    /* a split row's statistics exchange exceeded its wait bound */
} ce_status;

enum { CE_F32 = 0, CE_BF16 = 1 };

/* ce_params.reduce_loss */
enum { CE_REDUCE_NONE = 0, CE_REDUCE_MEAN = 1, CE_REDUCE_SUM = 2 };
/* ce_params.smoothing */
enum { CE_SMOOTH_ALL = 0, CE_SMOOTH_OTHERS = 1 };

/* Logits (or one vocabulary shard of them). */
typedef struct ce_logits {
  void* data;          /* device pointer to logical element (0, 0, 0); aligned to its dtype */
  int32_t dtype;       /* CE_F32 or CE_BF16 */
  int32_t reserved;    /* must be 0 */
  int64_t d0, d1;      /* logical leading dims, d0 >= 0, d1 >= 1; N = d0 * d1 rows */
  int64_t s0, s1;      /* element strides of d0 and d1 (>= 0); the column stride is 1 */
  int64_t v_local;     /* columns present in `data` (>= 1; a row below 4 GiB, else CE_ELAYOUT) */
  int64_t vocab_start; /* global index of local column 0 (0 when unsharded) */
  int64_t vocab_total; /* global vocabulary size V; vocab_start + v_local <= V */
} ce_logits;

/* Targets: int64 global vocabulary indices over the same logical (d0, d1). */
typedef struct ce_targets {
  const int64_t* data; /* device pointer to target (0, 0) */
  int64_t s0, s1;      /* element strides (>= 0) */
} ce_targets;

typedef struct ce_params {
  float label_smoothing; /* a in [0, 1] */
  int32_t reduce_loss;   /* CE_REDUCE_NONE: per-row loss[N], s_i = g_i;
                            CE_REDUCE_MEAN: mean over non-ignored rows, loss[1], s = g / n;
                            CE_REDUCE_SUM:  sum over rows, loss[1], s = g */
  int64_t ignore_idx;    /* rows whose target equals this are skipped (conventionally -100) */
  int32_t split_chunks;  /* 0: automatic.  > 0: ce_fwd_bwd_fused splits each row over this many
                            cooperating workgroups (tuning and testing; at most 64) */
  int32_t smoothing;     /* CE_SMOOTH_ALL or CE_SMOOTH_OTHERS; with CE_SMOOTH_OTHERS and a > 0 the
                            calls that use the smoothing need vocab_total >= 2 (CE_EINVAL otherwise) */
} ce_params;

/*
 * Workspace bytes that ce_forward and ce_fwd_bwd_fused need for logits
 * described by `x` and parameters `p` (a multiple of 256).  Returns 0 (and
 * sets ce_last_error) if the arguments are invalid.  Two calls must not use
 * one workspace concurrently.  ce_fwd_bwd_fused needs the workspace prepared
 * once by ce_workspace_init; ce_forward and ce_shard_combine need no
 * preparation and leave a prepared workspace prepared.
 */
size_t ce_workspace_bytes(const ce_logits* x, const ce_params* p);

/*
 * Prepares a workspace of `ws_bytes` bytes (256-byte aligned, a multiple of
 * 8) for ce_fwd_bwd_fused: enqueues one fill kernel on `stream` that zeroes it
 * and records the size in its header.  Once is enough for any number of
 * later calls whose workspace need is at most `ws_bytes`: each fused call tags
 * the words it exchanges with a fresh value, so words left by earlier calls
 * never need clearing.  Graph-capturable (no memset node).
 */
ce_status ce_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream);

/* Workspace bytes that ce_shard_combine needs for `rows` rows. */
size_t ce_combine_workspace_bytes(int64_t rows, const ce_params* p);

/*
 * Forward only (issue #29 section 1 forward; ops-nn "fusion scheme").
 * Unsharded logits (vocab_start == 0, v_local == vocab_total); read once.
 *   loss    [N] (CE_REDUCE_NONE) or [1] (mean, sum), device FP32, written
 *   lse     [N] device FP32 or NULL; ignored rows get 0
 *   n_valid [1] device int32 or NULL: number of non-ignored rows
 *   ws      device workspace of at least ce_workspace_bytes(x, p) bytes
 * The same as ce_forward_ex with lse_aux NULL.
 */
ce_status ce_forward(const ce_logits* x, const ce_targets* t, const ce_params* p, float* loss, float* lse,
                     int32_t* n_valid, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * The backward hand-off.  Issue #29 section 6 hands the backward the gathered
 * per-rank statistics (m, d, X_y), not a rounded lse; an FP32 lse alone
 * resolves p_t - 1 only to about ulp(lse) where the target holds nearly all
 * the probability.  The forward calls can therefore also write, per row,
 *   lse_aux[r][0] = the residual of lse: lse[r] + lse_aux[r][0] is the row's
 *                   log-sum-exp as the forward's FP32 sums give it, without
 *                   the final rounding to FP32;
 *   lse_aux[r][1] = 1 - p_t = sum_{j != t} softmax_j, from a sum that leaves
 *                   the target's own term out, so it keeps its digits as
 *                   p_t approaches 1;
 * device FP32 [N][2], 8-byte aligned; ignored rows get (0, 0), rows with an
 * invalid target NaN.  ce_backward_inplace_ex given the pair forms the fused
 * call's gradient: s ((1 - q_t) - (1 - p_t)) at a target with p_t > 1/2.
 */
ce_status ce_forward_ex(const ce_logits* x, const ce_targets* t, const ce_params* p, float* loss, float* lse,
                        float* lse_aux, int32_t* n_valid, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Backward, gradient written in place over the logits in their own dtype
 * (issue #29 section 6; ops-nn "backward", smoothing per "pitfall 3").  `x`
 * may be a vocabulary shard: column j is global column vocab_start + j and
 * the smoothing's V is vocab_total (hyper-parallel #269 section 3.1: the
 * backward needs no collective).
 *   lse       [N] device FP32 from ce_forward(_ex) or ce_shard_combine(_ex)
 *   lse_aux   [N][2] device FP32 from the same call's lse_aux, or NULL
 *             (ce_backward_inplace): then 1 - p_t comes from expm1(x_t - lse)
 *             and carries the FP32 lse's resolution
 *   grad_out  device FP32: [N] per-row upstream gradient (CE_REDUCE_NONE) or
 *             [1] (mean, sum); NULL means 1
 *   n_valid   [1] device int32, required with CE_REDUCE_MEAN (unused otherwise)
 * Ignored rows are set to +0.0 without being read.  Unsharded rows of at
 * most 128 columns are recomputed whole from the logits in FP64 (one wave per
 * row), as the fused call computes them; lse and lse_aux are not read there.
 */
ce_status ce_backward_inplace(const ce_logits* x, const ce_targets* t, const ce_params* p, const float* lse,
                              const float* grad_out, const int32_t* n_valid, hipStream_t stream);
ce_status ce_backward_inplace_ex(const ce_logits* x, const ce_targets* t, const ce_params* p, const float* lse,
                                 const float* lse_aux, const float* grad_out, const int32_t* n_valid,
                                 hipStream_t stream);

/*
 * Fused forward + backward: one read of the logits, the gradient written
 * over them once (ops-nn page, fused rows of its comparison table; issue #29
 * section 6 in-place staging).  Unsharded logits.  Rows that do not fit one
 * workgroup's registers are split over cooperating workgroups that exchange
 * (max, sum-exp, target logit, row sum) through the workspace.
 *   grad_out  as for ce_backward_inplace (known before the call); NULL = 1
 *   loss      [N] or [1] device FP32, written
 *   n_valid   [1] device int32 or NULL
 *   ws        device workspace of at least ce_workspace_bytes(x, p) bytes,
 *             prepared by ce_workspace_init.  On a workspace that was not
 *             prepared (or prepared smaller) the loss and the gradient come
 *             out NaN, n_valid is -1 and the workspace status records it
 *             (ce_workspace_check).
 * One kernel launch: the first workgroups also count the non-ignored rows,
 * and the workgroup of the last (row, chunk) item writes n_valid and the
 * mean or the sum.
 */
ce_status ce_fwd_bwd_fused(const ce_logits* x, const ce_targets* t, const ce_params* p, const float* grad_out,
                           float* loss, int32_t* n_valid, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * ce_fwd_bwd_fused for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace, which is a static
 * device array of 16 MiB per device inside the library (held until the
 * process ends).  Calls no hipMalloc, hipFree or allocating routine.
 *   - It holds a call that needs at most 16 MiB of workspace: about
 *     256 + 12 N bytes, plus 32 N K when rows are split into K > 1 chunks
 *     (N = 8192 rows of 128000 BF16 columns, K = 8: 2.2 MB; unsplit rows: up
 *     to about 1.39 million rows).  A larger call returns CE_EWORKSPACE
 *     before any HIP call.
 *   - The array used is that of the device `stream` belongs to (NULL: the
 *     current device).  The first call on a device prepares it on `stream`
 *     (one fill kernel) and must not be captured in a graph (CE_EINVAL);
 *     later calls may be.
 *   - Every call on a device shares its array: calls that overlap on one
 *     device (unordered streams) race, as two calls sharing one workspace do.
 *   - Results, errors and ce_workspace_check's record are as for
 *     ce_fwd_bwd_fused; the record is not reachable from the caller here.
 */
ce_status ce_fwd_bwd_fused_noalloc(const ce_logits* x, const ce_targets* t, const ce_params* p,
                                   const float* grad_out, float* loss, int32_t* n_valid, hipStream_t stream);

/*
 * The vocabulary-shard flow in one launch, each shard read once: S shards
 * (1 <= S <= 16) of one row set -- separate buffers, same dtype, rows and
 * vocab_total, tiling [0, vocab_total) in order (shards[s].vocab_start is
 * the sum of the previous shards' v_local; widths may differ, ceil(V / S)
 * with a short last shard as on hyper-parallel #269 section 3.1).  Every
 * shard's piece of a row stays in registers while the shards exchange
 * (max, sum-exp, target logit, row sum) through the workspace, as the chunks
 * of a split row do in ce_fwd_bwd_fused; then each shard's gradient is
 * written over it.  Same loss, gradient, reduction and workspace protocol as
 * ce_fwd_bwd_fused (ws from ce_shards_workspace_bytes, prepared by
 * ce_workspace_init).  The exchange sits where a multi-GPU run would
 * exchange the statistics between devices.  Shard rows of up to 4096 16-byte
 * vectors form one chunk; longer ones are cut, with at most 64 chunks per row.
 * `shards` is a host array of S descriptors (read during the call only); the
 * shards' data, t, grad_out, loss, n_valid and ws are device memory as for
 * ce_fwd_bwd_fused.  Errors, found on the host before anything is enqueued:
 * CE_EINVAL (NULL shards, S outside [1, 16], split_chunks != 0, a bad
 * descriptor field, targets or loss), CE_ELAYOUT (shards that differ in
 * dtype, rows or vocab_total, do not tile the vocabulary in order, or need
 * more than 64 chunks per row), CE_EWORKSPACE.  ce_shards_workspace_bytes
 * returns 0 for a shard set the call would refuse.
 */
size_t ce_shards_workspace_bytes(const ce_logits* shards, int32_t S, const ce_params* p);
ce_status ce_shards_fwd_bwd_fused(const ce_logits* shards, int32_t S, const ce_targets* t, const ce_params* p,
                                  const float* grad_out, float* loss, int32_t* n_valid, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/*
 * Deferred upstream gradient (TENPU #29 section 6 stages the gradient in the
 * input; the autograd backward then applies the upstream gradient).  `x`
 * holds a gradient written by ce_fwd_bwd_fused or ce_backward_inplace for an
 * upstream gradient of 1; this multiplies row r by grad_out[r] (per_row = 1,
 * grad_out device FP32 [N]) or every row by grad_out[0] (per_row = 0, [1]),
 * in place, in x's dtype (FP32 multiply, then RNE to BF16: a second rounding
 * of a BF16 gradient unless the factor is a power of two).  A row whose
 * factor is exactly 1 is neither read nor written, so the common case costs
 * one small launch and no traffic, with no host synchronisation.  Zeros stay
 * +0.0, so ignored rows keep their bit pattern for any factor.
 */
ce_status ce_scale_grad_inplace(const ce_logits* x, const float* grad_out, int32_t per_row, hipStream_t stream);

/*
 * Per-shard partial statistics (issue #29 section 6 gathers (m, d, X_y);
 * hyper-parallel #269 section 3.1 reduces MAX and SUM and gathers the target
 * logit).  For every logical row of the shard:
 *   stats[r*4 + 0] = m = max_j x_rj                      (natural units)
 *   stats[r*4 + 1] = d = sum_{j != t_r} exp(x_rj - m)   (the target's own term
 *                    left out; only the shard that holds t_r has it)
 *   stats[r*4 + 2] = y = x_r,(t_r - vocab_start) if the shard holds t_r, else 0
 *   stats[r*4 + 3] = r = sum_j x_rj
 * The combine restores the target's term from y, and keeping it out of d
 * keeps 1 - p_t = D_excl / D exact to the sum's precision when the target
 * holds nearly all the probability.  Rows of at most 128 columns are summed
 * in FP64 and rounded once.  Ignored rows are not read and get (0, 0, 0, 0).
 * `stats` is device FP32 [N][4].
 */
ce_status ce_shard_partial_stats(const ce_logits* shard, const ce_targets* t, const ce_params* p, float* stats,
                                 hipStream_t stream);

/*
 * Combine S shards' statistics stats[S][N][4] (device FP32, shard-major) into
 * per-row loss and lse over the full vocabulary of vocab_total columns:
 *   M = max_s m_s, D_excl = sum_s d_s exp(m_s - M) (s ascending),
 *   x_t = sum_s y_s, D = D_excl + exp(x_t - M), lse = M + log D,
 *   loss = lse - (q_t - q_o) x_t - q_o sum_s r_s,
 * in FP64, each output rounded once to FP32; q_t and q_o are the smoothed
 * target probability of the target and of any other class (a / V + 1 - a
 * and a / V, or 1 - a and a / (V - 1)).  This is the point where a multi-GPU
 * run would exchange the statistics.
 *   loss [N] or [1], lse [N] (may be NULL), n_valid [1] (may be NULL),
 *   ws of at least ce_combine_workspace_bytes(d0 * d1, p) bytes.
 * ce_shard_combine_ex also writes the backward hand-off pair lse_aux [N][2]
 * (see ce_forward_ex; may be NULL) with 1 - p_t = D_excl / D.
 */
ce_status ce_shard_combine(const float* stats, int32_t S, int64_t d0, int64_t d1, int64_t vocab_total,
                           const ce_targets* t, const ce_params* p, float* loss, float* lse, int32_t* n_valid,
                           void* ws, size_t ws_bytes, hipStream_t stream);
ce_status ce_shard_combine_ex(const float* stats, int32_t S, int64_t d0, int64_t d1, int64_t vocab_total,
                              const ce_targets* t, const ce_params* p, float* loss, float* lse, float* lse_aux,
                              int32_t* n_valid, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Chunked linear + cross-entropy: the language-model head's matrix product
 * and the loss, forward and backward, over row chunks, so that only one
 * chunk of logits exists at a time (hyper-parallel #269: Titan's
 * ChunkedLossWrapper, the sequence-chunked lm_head of its comparison table
 * row 9 and task P2 #9, against the O(B x L x V) peak of whole logits).
 * For each chunk of `chunk_rows` consecutive rows c:
 *   logits_c = h_c W^T                in the input dtype (FP32 accumulation,
 *                                      on the matrix cores: see `gemm`)
 *   loss, G_c in place of logits_c    ce_fwd_bwd_fused (smoothing and ignore
 *                                      rules as above)
 *   dh_c  = G_c W                      in the input dtype (FP32 accumulation)
 *   dW   += G_c^T h_c                  FP32
 * The mean divides by the count over all N rows (counted before the first
 * chunk) and every chunk's gradient uses s = g / n; the sum and the per-row
 * loss need no count.  G_c is rounded to the input dtype before the two
 * backward products, as the fused call writes it.
 */
/* The engine of the three products (ce_linear.gemm):
 *   CE_GEMM_NATIVE   the library's own MFMA kernel (v_mfma_f32_32x32x16_bf16,
 *                    256 x 256 output tiles, operands loaded straight into
 *                    two LDS stages) wherever it applies: BF16, h and w
 *                    16-byte aligned, h_ld, w_ld and D multiples of 8; other
 *                    calls, and FP32 heads, run on the GEMM library
 *   CE_GEMM_LIBRARY  hipBLASLt, ROCm's GEMM library, for every product
 *   CE_GEMM_AUTO     per product, the engine measured faster on gfx950 at the
 *                    head's shapes (currently the native kernel for dh and
 *                    dW, the library for the logits)
 * Both engines accumulate in FP32 and round the output once; their results
 * differ only in the summation order. */
#define CE_GEMM_AUTO 0
#define CE_GEMM_NATIVE 1
#define CE_GEMM_LIBRARY 2

typedef struct ce_linear {
  const void* h;      /* device [N, D] hidden states, row stride h_ld elements, columns contiguous */
  const void* w;      /* device [V, D] head weight (torch Linear layout: logits = h W^T), row stride w_ld */
  int32_t dtype;      /* CE_BF16 or CE_F32, for h, w and dh */
  int32_t gemm;       /* CE_GEMM_AUTO (0), CE_GEMM_NATIVE or CE_GEMM_LIBRARY; else CE_EINVAL */
  int64_t N, D, V;    /* rows, hidden size, vocabulary (N >= 0, D >= 1, V >= 1) */
  int64_t h_ld, w_ld; /* >= D */
} ce_linear;

/* Workspace bytes of ce_linear_cross_entropy for `lin`, `p` and chunk_rows
 * (0: automatic, about 1 GiB of logits per chunk); 0 if the arguments are
 * invalid.  `*chunk_rows_out` (may be NULL) receives the chunk size used. */
size_t ce_linear_workspace_bytes(const ce_linear* lin, const ce_params* p, int64_t chunk_rows,
                                 int64_t* chunk_rows_out);

/*
 *   targets   device int64, row r's target at targets[r * t_stride]
 *   grad_out  as for ce_fwd_bwd_fused over N rows ([N] or [1]; NULL = 1)
 *   loss      [N] or [1] device FP32, written
 *   n_valid   [1] device int32 or NULL: the number of non-ignored rows
 *   dh        device [N, D] in the input dtype (row stride dh_ld), written; NULL: not computed
 *   dw        device FP32 [V, D] (row stride dw_ld); accumulate_dw = 0 overwrites it, 1 adds to it;
 *             NULL: not computed
 *   ws        device workspace of ce_linear_workspace_bytes bytes (256-byte aligned), prepared by
 *             ce_workspace_init; it holds the chunk's logits (row stride V rounded up to a multiple
 *             of 8), the fused call's exchange words and the GEMM library's scratch
 * The first call on a device creates that device's GEMM library handle (host
 * state kept until the process ends) and each new shape that runs on the
 * library queries its heuristics once; after that the call allocates nothing.  The
 * calls are asynchronous on `stream`, with no host synchronisation.
 */
ce_status ce_linear_cross_entropy(const ce_linear* lin, const int64_t* targets, int64_t t_stride,
                                  const ce_params* p, const float* grad_out, float* loss, int32_t* n_valid,
                                  void* dh, int64_t dh_ld, float* dw, int64_t dw_ld, int32_t accumulate_dw,
                                  int64_t chunk_rows, void* ws, size_t ws_bytes, hipStream_t stream);

/* Which of the three products ce_linear_cross_entropy would run on the
 * library's MFMA kernel for `lin` (lin->gemm and the layout checks): bit 0
 * the logits product, bit 1 dh, bit 2 dW; -1 if `lin` is NULL or invalid.
 * Host only, no HIP calls. */
int32_t ce_linear_gemm_plan(const ce_linear* lin);

/*
 * Optional, once per shape before a training loop: for the GEMMs that
 * ce_linear_cross_entropy runs with these arguments (a whole chunk, the last
 * chunk, dh and dW as requested), times the GEMM library's first candidate
 * algorithms on the given buffers and keeps the fastest for this process.
 * Synchronises `stream`; writes scratch values into dh, dw and the
 * workspace's chunk buffer (run the real call afterwards).  Without it the
 * call uses the library heuristic's first choice.
 */
ce_status ce_linear_tune(const ce_linear* lin, const ce_params* p, void* dh, int64_t dh_ld, float* dw,
                         int64_t dw_ld, int64_t chunk_rows, void* ws, size_t ws_bytes, hipStream_t stream);

/* Waits for `stream` and reports whether any call that used `ws` since it was
 * prepared or last checked gave up waiting in a split-row exchange or count
 * (CE_EDEADLOCK; its results were NaN) or found the workspace unprepared
 * (CE_EWORKSPACE), then clears that record.  A diagnostic: synchronises, so
 * not for the hot path. */
ce_status ce_workspace_check(void* ws, hipStream_t stream);

/*
 * Reference streaming pass for benchmarks (not a step of the method): a
 * plain one-pass kernel moving the bytes a fused call moves, whose rate is
 * reported beside that call's.  `bytes` (a multiple of 16; 0 does nothing) of device
 * memory are read once and written once with the same 16-byte non-temporal
 * buffer loads and stores as the fused kernel streams logits with, in
 * 64 KiB workgroup spans.  src == dst: every 32-bit word is XORed with
 * 0x80008000 in place (the sign of each BF16 half flips, so two passes restore
 * the buffer); otherwise src is copied to dst, which must not overlap it.  Both
 * 16-byte aligned.  Asynchronous on `stream`; ce_profile_start times it like
 * the calls listed there.  CE_EINVAL for a bad size, NULL, misaligned or
 * partly overlapping buffers, before any launch.
 */
ce_status ce_stream_reference(const void* src, void* dst, int64_t bytes, hipStream_t stream);

/*
 * Kernel timing for benchmarks.  After ce_profile_start(capacity), each of
 * the next `capacity` calls of ce_forward(_ex), ce_backward_inplace(_ex),
 * ce_fwd_bwd_fused(_noalloc), ce_shards_fwd_bwd_fused, ce_shard_partial_stats,
 * ce_scale_grad_inplace or ce_stream_reference that launch work records a pair
 * of HIP events on its stream around its main (bandwidth-dominant) kernel.
 * ce_profile_stop(ms, cap, count) waits for those events, writes up to `cap`
 * durations in milliseconds to host array `ms`, the number recorded to
 * *count, and releases the events.  Not thread-safe; adds no synchronisation
 * to the timed calls.
 */
ce_status ce_profile_start(int32_t capacity);
ce_status ce_profile_stop(float* ms, int32_t cap, int32_t* count);

const char* ce_status_string(ce_status s);
/* Detail of the last non-OK status returned on the calling thread. */
const char* ce_last_error(void);
int32_t ce_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VCE_CE_H */
