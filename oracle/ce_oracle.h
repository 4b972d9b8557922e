/*
 * ce_oracle.h -- declarations of the FP64 CPU oracle (ce_oracle.c).
 *
 * TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
 * CPU baseline may use it; the library never does.  Definitions, sources and
 * pins are described at the top of ce_oracle.c.
 */
#ifndef CE_ORACLE_H
#define CE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OR_F32 0
#define OR_BF16 1

#define OR_EBADTARGET (-1)
#define OR_EINVAL (-2)

#define OR_SMOOTH_ALL 0    /* a / V on every class (torch's F.cross_entropy) */
#define OR_SMOOTH_OTHERS 1 /* a / (V - 1) on every class but the target (ops-nn kernel) */

#define OR_REDUCE_NONE 0
#define OR_REDUCE_MEAN 1
#define OR_REDUCE_SUM 2

typedef struct or_logits {
  const void* data;
  int32_t dtype;       /* OR_F32 or OR_BF16 */
  int32_t pad_;
  int64_t d0, d1;      /* logical leading dims; rows = d0 * d1 */
  int64_t s0, s1;      /* element strides of the two leading dims */
  int64_t v_local;     /* columns present in this buffer */
  int64_t vocab_start; /* global index of local column 0 */
  int64_t vocab_total; /* global vocabulary size V */
} or_logits;

typedef struct or_targets {
  const int64_t* data;
  int64_t s0, s1;
} or_targets;

int64_t or_count_valid(const or_targets* t, int64_t d0, int64_t d1, int64_t ignore_idx);
int or_loss_rows(const or_logits* x, const or_targets* t, double alpha, int32_t smooth, int64_t ignore_idx,
                 const int64_t* rows, int64_t nrows, double* loss_out, double* lse_out);
int or_grad_rows(const or_logits* x, const or_targets* t, double alpha, int32_t smooth, int64_t ignore_idx,
                 int32_t reduce, const double* g_row, double g_scalar, int64_t n_valid,
                 const int64_t* rows, int64_t nrows, double* grad_out);
double or_mean_loss(const double* loss, int64_t nrows, int64_t n_valid);
double or_sum_loss(const double* loss, int64_t nrows);
int or_shard_stats(const or_logits* x, const or_targets* t, int64_t ignore_idx,
                   const int64_t* rows, int64_t nrows, double* stats_out);
int or_shard_combine(const double* stats, int32_t S, int64_t nrows, int64_t vocab_total,
                     const or_targets* t, int64_t d1, double alpha, int32_t smooth, int64_t ignore_idx,
                     const int64_t* rows, double* loss_out, double* lse_out);
int or_shard_grad(const or_logits* x, const or_targets* t, double alpha, int32_t smooth, int64_t ignore_idx,
                  int32_t reduce, const double* g_row, double g_scalar, int64_t n_valid,
                  const int64_t* rows, int64_t nrows, const double* lse, double* grad_out);
int or_linear_ce(const void* h, const void* w, int32_t dtype, int64_t N, int64_t D, int64_t V, int64_t h_ld,
                 int64_t w_ld, const int64_t* t, int64_t t_stride, double alpha, int32_t smooth, int64_t ignore_idx,
                 int32_t reduce, const double* g_row, double g_scalar, int64_t n_valid, int32_t round_mode,
                 double* loss_out, double* dh_out, double* dw_out, double* g_out);
int or_max_threads(void);

#ifdef __cplusplus
}
#endif

#endif /* CE_ORACLE_H */
