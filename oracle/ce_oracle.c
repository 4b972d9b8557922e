/*
 * ce_oracle.c -- plain, slow, FP64 CPU oracle for fused (vocabulary-parallel)
 * cross-entropy over language-model logits.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the yardstick that the GPU library is
 * measured against.  Only the tests, the smoke check and the CPU-baseline leg
 * of the benchmark may load it; the product path never does.  It shares no
 * code, header, table or helper with the HIP library.
 *
 * What it computes (plain definitions, FP64 accumulation, rows one by one):
 *
 *   Cross-entropy of row i with target t_i over V classes, label smoothing a:
 *     softmax_ij = exp(x_ij) / sum_k exp(x_ik)
 *     q_ij       = a/V + (1 - a) [j == t_i]      (smoothed target distribution)
 *     loss_i     = - sum_j q_ij log softmax_ij
 *   The fused method rests on log softmax_ij = x_ij - lse_i with
 *   lse_i = log sum_k exp(x_ik), so no N x V intermediate is needed
 *   ("CANN ops-nn CE fusion" page, section "fusion scheme: log_softmax + NLL").
 *   lse is evaluated with the row maximum taken out first, the standard guard
 *   against exp overflow (same page, "pitfall 1: exp overflow").
 *   The default smoothing convention (OR_SMOOTH_ALL) is the uniform a/V one
 *   of torch's F.cross_entropy, which the TransformerEngineNPU issue #29 page
 *   names as the precision baseline (section 4).  The ops-nn page's kernel
 *   (step 4 of its forward, and "pitfall 3" for the backward) spreads a over
 *   the V-1 classes other than the target instead (OR_SMOOTH_OTHERS):
 *     q_ij = 1 - a if j == t_i, a / (V - 1) otherwise
 *     loss_i = (1 - a) (lse_i - x_it) + a sum_{j != t} (lse_i - x_ij) / (V - 1)
 *   computed in that form (the NLL term plus the mean of the other classes'
 *   negative log-probabilities).  With V = 1 there is no other class: a > 0
 *   is rejected, a = 0 is plain NLL.
 *
 *   A term whose weight q_ij is 0 contributes nothing to the loss (0 log 0 =
 *   0), so a logit of -inf (a masked class) leaves the loss finite unless the
 *   smoothing gives it weight, as in torch's F.cross_entropy.
 *
 *   Rows whose target equals ignore_idx have loss 0 and gradient 0
 *   (ops-nn page, both kernels; default ignore_idx -100 per issue #29 section 1
 *   and the hyper-parallel issue #269 section 3.1).
 *
 *   Gradient (ops-nn page, section "backward"; smoothing correction from its
 *   "pitfall 3", with q of either convention):
 *     grad_ij = s_i (softmax_ij - q_ij)
 *   with s_i = g_i (per-row upstream gradient) when the loss is not reduced
 *   (OR_REDUCE_NONE), s_i = g / n for the mean over the n rows whose target
 *   is not ignored (OR_REDUCE_MEAN; issue #29 section 1 "reduce_loss",
 *   section 7 counts n_non_ignore), and s_i = g for the sum over rows
 *   (OR_REDUCE_SUM; the hyper-parallel issue #269 comparison table, row
 *   "reduction semantics": Titan trains on the sum divided by the global
 *   count of valid tokens, which here is g = 1 / that count).
 *
 *   Vocabulary shards (hyper-parallel issue #269, section 3.1: forward is a
 *   MAX all-reduce, a SUM all-reduce and a gather of the target logit;
 *   issue #29 section 6 gathers the per-rank (m, d, X_y) triple):
 *     shard k holds global columns [o_k, o_k + V_k)
 *     m_k = max_j x_j,  d_k = sum_{j != t} exp(x_j - m_k),
 *     y_k = x[t - o_k] if o_k <= t < o_k + V_k else 0,  r_k = sum_j x_j
 *     M = max_k m_k,  x_t = sum_k y_k,  R = sum_k r_k,
 *     D = sum_k d_k exp(m_k - M) + exp(x_t - M),  lse = M + log D,
 *   d_k leaves out the target's own term (only the shard holding the target
 *   has one) and the combine restores it from the gathered target logit;
 *   the sum is the same, and 1 - p_t = (D - exp(x_t - M)) / D is then the
 *   combine's first term over D, with no difference of nearly equal numbers.
 *     loss = lse - (1 - a) x_t - (a / V) R                        (OR_SMOOTH_ALL)
 *     loss = (1 - a)(lse - x_t) + a ((V - 1) lse - (R - x_t)) / (V - 1)
 *                                                                 (OR_SMOOTH_OTHERS)
 *   The first line is the expanded form of -sum_j q_j (x_j - lse), the second
 *   the ops-nn form with sum_{j != t} (lse - x_j) written through R; the row
 *   sum r_k is the extra statistic that a > 0 needs.
 *
 * Inputs are read as the exact stored bits: BF16 is widened to FP32 by a
 * 16-bit shift and then to double, FP32 is widened to double.  Logical row
 * r = i0 * d1 + i1 lives at element offset i0 * s0 + i1 * s1; columns are
 * contiguous.  Targets are int64 at i0 * ts0 + i1 * ts1.
 *
 * Every function returns 0 on success and a negative code on bad input:
 *   -1  a non-ignored target outside [0, V)
 *   -2  bad argument (sizes, dtype, NULL)
 *
 * Pins (tests/test_oracle_pins.py): decimal brute force of the unfused
 * softmax -> log -> NLL chain (both smoothing conventions), the closed form
 * loss = ln V for uniform logits and the ops-nn page's worked lse value,
 * torch's float64 F.cross_entropy and its autograd gradient (mean, sum and
 * per-row reductions; the a/(V-1) convention is torch's a/V smoothing with
 * a' = a V / (V - 1), which puts the same mass on every class), central
 * finite differences, shift invariance, gradient rows summing to zero, and
 * sharded == unsharded.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "ce_oracle.h"

/* Exact widening of one stored logit to double. */
static double or_elem(const or_logits* x, int64_t off) {
  if (x->dtype == OR_F32) return (double)((const float*)x->data)[off];
  uint32_t bits = (uint32_t)((const uint16_t*)x->data)[off] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static int64_t or_row_offset(const or_logits* x, int64_t r) {
  int64_t i0 = r / x->d1, i1 = r % x->d1;
  return i0 * x->s0 + i1 * x->s1;
}

static int64_t or_target(const or_targets* t, int64_t d1, int64_t r) {
  int64_t i0 = r / d1, i1 = r % d1;
  return t->data[i0 * t->s0 + i1 * t->s1];
}

static int or_check(const or_logits* x) {
  if (!x || !x->data) return OR_EINVAL;
  if (x->dtype != OR_F32 && x->dtype != OR_BF16) return OR_EINVAL;
  if (x->d0 < 0 || x->d1 <= 0 || x->v_local <= 0) return OR_EINVAL;
  if (x->vocab_start < 0 || x->vocab_start + x->v_local > x->vocab_total) return OR_EINVAL;
  return 0;
}

/* The smoothing convention is known and usable with V classes. */
static int or_smooth_ok(int32_t smooth, double alpha, int64_t V) {
  if (smooth != OR_SMOOTH_ALL && smooth != OR_SMOOTH_OTHERS) return 0;
  return !(smooth == OR_SMOOTH_OTHERS && alpha > 0.0 && V < 2);
}

/* Smoothed target probability q_j of class j of a V-class row with target t. */
static double or_q(int32_t smooth, double alpha, int64_t V, int is_target) {
  if (smooth == OR_SMOOTH_OTHERS) return is_target ? 1.0 - alpha : (alpha > 0.0 ? alpha / (double)(V - 1) : 0.0);
  return alpha / (double)V + (is_target ? 1.0 - alpha : 0.0);
}

/* Upstream scale s of row r (OR_REDUCE_* as in the header comment). */
static double or_scale(int32_t reduce, const double* g_row, double g_scalar, int64_t n_valid, int64_t r) {
  if (reduce == OR_REDUCE_MEAN) return g_scalar / (double)n_valid;
  if (reduce == OR_REDUCE_SUM) return g_scalar;
  return g_row ? g_row[r] : 1.0;
}

/* n = number of rows whose target is not ignore_idx. */
int64_t or_count_valid(const or_targets* t, int64_t d0, int64_t d1, int64_t ignore_idx) {
  int64_t n = 0;
  for (int64_t r = 0; r < d0 * d1; ++r)
    if (or_target(t, d1, r) != ignore_idx) ++n;
  return n;
}

/* lse of one full row: m + log sum_j exp(x_j - m). */
static double or_row_lse(const or_logits* x, int64_t off) {
  int64_t V = x->v_local;
  double m = -INFINITY;
  for (int64_t j = 0; j < V; ++j) {
    double v = or_elem(x, off + j);
    if (v > m) m = v;
  }
  double s = 0.0;
  for (int64_t j = 0; j < V; ++j) s += exp(or_elem(x, off + j) - m);
  return m + log(s);
}

/*
 * Loss (and lse) of the listed logical rows of an unsharded row set
 * (v_local == vocab_total).  loss_i = -sum_j q_ij (x_ij - lse_i).
 * lse_out may be NULL; for ignored rows it receives NAN (not defined).
 */
int or_loss_rows(const or_logits* x, const or_targets* t, double alpha, int32_t smooth, int64_t ignore_idx,
                 const int64_t* rows, int64_t nrows, double* loss_out, double* lse_out) {
  if (or_check(x) || x->v_local != x->vocab_total || !t || !rows || !loss_out) return OR_EINVAL;
  const int64_t V = x->v_local;
  if (!or_smooth_ok(smooth, alpha, V)) return OR_EINVAL;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t k = 0; k < nrows; ++k) {
    int64_t r = rows[k];
    int64_t tgt = or_target(t, x->d1, r);
    if (tgt == ignore_idx) {
      loss_out[k] = 0.0;
      if (lse_out) lse_out[k] = NAN;
      continue;
    }
    if (tgt < 0 || tgt >= V) {
      bad = 1;
      continue;
    }
    int64_t off = or_row_offset(x, r);
    double lse = or_row_lse(x, off);
    double loss = 0.0;
    if (smooth == OR_SMOOTH_OTHERS) {
      /* ops-nn: (1 - a) * NLL + a * (mean over the other classes of -log softmax) */
      if (alpha < 1.0) loss = (1.0 - alpha) * (lse - or_elem(x, off + tgt));
      if (alpha > 0.0) {
        double other = 0.0;
        for (int64_t j = 0; j < V; ++j)
          if (j != tgt) other += lse - or_elem(x, off + j);
        loss += alpha * other / (double)(V - 1);
      }
    } else {
      for (int64_t j = 0; j < V; ++j) {
        double q = or_q(smooth, alpha, V, j == tgt);
        if (q != 0.0) loss -= q * (or_elem(x, off + j) - lse); /* 0 log 0 = 0: a masked (-inf) class with q = 0 adds nothing */
      }
    }
    loss_out[k] = loss;
    if (lse_out) lse_out[k] = lse;
  }
  return bad ? OR_EBADTARGET : 0;
}

/*
 * Gradient of the listed rows, unrounded FP64, written as grad_out[k * V + j].
 * s_i = g_row[r] (or 1 when g_row is NULL) for OR_REDUCE_NONE,
 * g_scalar / n_valid for OR_REDUCE_MEAN, g_scalar for OR_REDUCE_SUM.
 * Ignored rows get 0.
 */
int or_grad_rows(const or_logits* x, const or_targets* t, double alpha, int32_t smooth, int64_t ignore_idx,
                 int32_t reduce, const double* g_row, double g_scalar, int64_t n_valid,
                 const int64_t* rows, int64_t nrows, double* grad_out) {
  if (or_check(x) || x->v_local != x->vocab_total || !t || !rows || !grad_out) return OR_EINVAL;
  const int64_t V = x->v_local;
  if (!or_smooth_ok(smooth, alpha, V) || reduce < OR_REDUCE_NONE || reduce > OR_REDUCE_SUM) return OR_EINVAL;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t k = 0; k < nrows; ++k) {
    int64_t r = rows[k];
    double* gout = grad_out + k * V;
    int64_t tgt = or_target(t, x->d1, r);
    if (tgt == ignore_idx) {
      for (int64_t j = 0; j < V; ++j) gout[j] = 0.0;
      continue;
    }
    if (tgt < 0 || tgt >= V) {
      bad = 1;
      continue;
    }
    double s = or_scale(reduce, g_row, g_scalar, n_valid, r);
    int64_t off = or_row_offset(x, r);
    double lse = or_row_lse(x, off);
    for (int64_t j = 0; j < V; ++j) {
      double p = exp(or_elem(x, off + j) - lse);
      gout[j] = s * (p - or_q(smooth, alpha, V, j == tgt));
    }
  }
  return bad ? OR_EBADTARGET : 0;
}

/* Mean of per-row losses over the n non-ignored rows: sum_i loss_i / n. */
double or_mean_loss(const double* loss, int64_t nrows, int64_t n_valid) {
  double s = 0.0;
  for (int64_t i = 0; i < nrows; ++i) s += loss[i];
  return s / (double)n_valid;
}

/* Sum of per-row losses (ignored rows contribute their loss of 0). */
double or_sum_loss(const double* loss, int64_t nrows) {
  double s = 0.0;
  for (int64_t i = 0; i < nrows; ++i) s += loss[i];
  return s;
}

/*
 * Per-shard statistics of the listed rows: stats_out[k*4 + {0,1,2,3}] =
 * (m, d, y, r) as defined in the header comment (d without the target's
 * term).  Targets are global.  Ignored rows get (0, 0, 0, 0).
 */
int or_shard_stats(const or_logits* x, const or_targets* t, int64_t ignore_idx,
                   const int64_t* rows, int64_t nrows, double* stats_out) {
  if (or_check(x) || !t || !rows || !stats_out) return OR_EINVAL;
  const int64_t V = x->v_local, o = x->vocab_start;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t k = 0; k < nrows; ++k) {
    int64_t r = rows[k];
    double* st = stats_out + 4 * k;
    int64_t tgt = or_target(t, x->d1, r);
    if (tgt == ignore_idx) {
      st[0] = st[1] = st[2] = st[3] = 0.0;
      continue;
    }
    int64_t off = or_row_offset(x, r);
    double m = -INFINITY;
    for (int64_t j = 0; j < V; ++j) {
      double v = or_elem(x, off + j);
      if (v > m) m = v;
    }
    double d = 0.0, rs = 0.0;
    for (int64_t j = 0; j < V; ++j) {
      double v = or_elem(x, off + j);
      if (o + j != tgt) d += exp(v - m);
      rs += v;
    }
    st[0] = m;
    st[1] = d;
    st[2] = (tgt >= o && tgt < o + V) ? or_elem(x, off + (tgt - o)) : 0.0;
    st[3] = rs;
  }
  return 0;
}

/*
 * Combine S shards' statistics (stats[s][k][4], k over the listed rows) into
 * loss and lse for those rows.  V in a/V is vocab_total.
 */
int or_shard_combine(const double* stats, int32_t S, int64_t nrows, int64_t vocab_total,
                     const or_targets* t, int64_t d1, double alpha, int32_t smooth, int64_t ignore_idx,
                     const int64_t* rows, double* loss_out, double* lse_out) {
  if (!stats || S <= 0 || vocab_total <= 0 || !t || !rows || !loss_out) return OR_EINVAL;
  if (!or_smooth_ok(smooth, alpha, vocab_total)) return OR_EINVAL;
  int bad = 0;
  for (int64_t k = 0; k < nrows; ++k) {
    int64_t tgt = or_target(t, d1, rows[k]);
    if (tgt == ignore_idx) {
      loss_out[k] = 0.0;
      if (lse_out) lse_out[k] = NAN;
      continue;
    }
    if (tgt < 0 || tgt >= vocab_total) {
      bad = 1;
      continue;
    }
    double M = -INFINITY;
    for (int32_t s = 0; s < S; ++s) {
      double m = stats[((int64_t)s * nrows + k) * 4 + 0];
      if (m > M) M = m;
    }
    double D = 0.0, xt = 0.0, R = 0.0;
    for (int32_t s = 0; s < S; ++s) {
      const double* st = stats + ((int64_t)s * nrows + k) * 4;
      D += st[1] * exp(st[0] - M);
      xt += st[2];
      R += st[3];
    }
    D += exp(xt - M); /* the target's term, left out of every d_k */
    double lse = M + log(D);
    /* terms with a zero weight are left out (0 log 0 = 0), so masked (-inf) logits only matter where q > 0 */
    if (smooth == OR_SMOOTH_OTHERS) {
      double loss = alpha < 1.0 ? (1.0 - alpha) * (lse - xt) : 0.0;
      /* R - x_t is undefined for a masked (-inf) target; the loss is then +inf through the NLL term (a < 1),
         since the other classes' term is never negative */
      const int masked_target = isinf(xt) && xt < 0.0 && alpha < 1.0;
      if (alpha > 0.0 && !masked_target)
        loss += alpha * ((double)(vocab_total - 1) * lse - (R - xt)) / (double)(vocab_total - 1);
      loss_out[k] = loss;
    } else {
      double loss = lse;
      if (alpha < 1.0) loss -= (1.0 - alpha) * xt;
      if (alpha > 0.0) loss -= (alpha / (double)vocab_total) * R;
      loss_out[k] = loss;
    }
    if (lse_out) lse_out[k] = lse;
  }
  return bad ? OR_EBADTARGET : 0;
}

/*
 * Gradient of the listed rows of one shard, given the combined lse of each
 * listed row (lse[k]).  Column j of the shard is global column o + j.
 * grad_out[k * V_local + j]; scale s_i as in or_grad_rows.
 */
int or_shard_grad(const or_logits* x, const or_targets* t, double alpha, int32_t smooth, int64_t ignore_idx,
                  int32_t reduce, const double* g_row, double g_scalar, int64_t n_valid,
                  const int64_t* rows, int64_t nrows, const double* lse, double* grad_out) {
  if (or_check(x) || !t || !rows || !lse || !grad_out) return OR_EINVAL;
  const int64_t V = x->v_local, o = x->vocab_start, Vt = x->vocab_total;
  if (!or_smooth_ok(smooth, alpha, Vt) || reduce < OR_REDUCE_NONE || reduce > OR_REDUCE_SUM) return OR_EINVAL;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t k = 0; k < nrows; ++k) {
    int64_t r = rows[k];
    double* gout = grad_out + k * V;
    int64_t tgt = or_target(t, x->d1, r);
    if (tgt == ignore_idx) {
      for (int64_t j = 0; j < V; ++j) gout[j] = 0.0;
      continue;
    }
    double s = or_scale(reduce, g_row, g_scalar, n_valid, r);
    int64_t off = or_row_offset(x, r);
    for (int64_t j = 0; j < V; ++j) {
      double p = exp(or_elem(x, off + j) - lse[k]);
      gout[j] = s * (p - or_q(smooth, alpha, Vt, o + j == tgt));
    }
  }
  return 0;
}

/*
 * Linear head + cross-entropy (hyper-parallel #269, Titan's chunked loss:
 * the lm_head product and its loss; chunking changes where the logits live,
 * not what is computed, so the oracle works on all rows at once).
 *   logits_ij = sum_d h_id W_jd, in FP64 from the exact stored values, then
 *               materialised as the library does: rounded to FP32 (the GEMM
 *               accumulator), then for BF16 inputs to BF16, both
 *               round-to-nearest-even (round_mode 1); round_mode 0 keeps the
 *               FP64 value (for finite differences);
 *   loss_i, G_ij = s_i (softmax_ij - q_ij) of those logits, as above;
 *   dh_id = sum_j G_ij W_jd,  dW_jd = sum_i G_ij h_id   (FP64, G unrounded).
 * The gradient treats the rounding of the logits as the identity, as
 * autograd does for a low-precision matmul.  h: [N, D] row stride h_ld;
 * W: [V, D] row stride w_ld; dtype OR_F32 or OR_BF16 for both; targets
 * t[r * t_stride].  Outputs: loss_out[N], dh_out[N * D], dw_out[V * D]
 * (either gradient may be NULL) and, when g_out is not NULL, G itself [N * V].
 */
static double or_load(const void* p, int32_t dtype, int64_t off) {
  if (dtype == OR_F32) return (double)((const float*)p)[off];
  uint32_t bits = (uint32_t)((const uint16_t*)p)[off] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/* FP32 value rounded to BF16, nearest even (finite inputs). */
static float or_round_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  u = (u + 0x7fffu + ((u >> 16) & 1u)) & 0xffff0000u;
  memcpy(&f, &u, sizeof f);
  return f;
}

int or_linear_ce(const void* h, const void* w, int32_t dtype, int64_t N, int64_t D, int64_t V, int64_t h_ld,
                 int64_t w_ld, const int64_t* t, int64_t t_stride, double alpha, int32_t smooth, int64_t ignore_idx,
                 int32_t reduce, const double* g_row, double g_scalar, int64_t n_valid, int32_t round_mode,
                 double* loss_out, double* dh_out, double* dw_out, double* g_out) {
  if ((N > 0 && (!h || !t)) || !w || !loss_out || D < 1 || V < 1 || N < 0 || h_ld < D || w_ld < D) return OR_EINVAL;
  if (dtype != OR_F32 && dtype != OR_BF16) return OR_EINVAL;
  if (!or_smooth_ok(smooth, alpha, V) || reduce < OR_REDUCE_NONE || reduce > OR_REDUCE_SUM) return OR_EINVAL;
  double* G = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1) * (size_t)V);
  if (!G) return OR_EINVAL;
  int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
  for (int64_t r = 0; r < N; ++r) {
    double* x = G + r * V;
    const int64_t tgt = t[r * t_stride];
    if (tgt == ignore_idx) {
      loss_out[r] = 0.0;
      for (int64_t j = 0; j < V; ++j) x[j] = 0.0;
      continue;
    }
    if (tgt < 0 || tgt >= V) {
      bad = 1;
      for (int64_t j = 0; j < V; ++j) x[j] = 0.0;
      continue;
    }
    for (int64_t j = 0; j < V; ++j) {
      double acc = 0.0;
      for (int64_t d = 0; d < D; ++d) acc += or_load(h, dtype, r * h_ld + d) * or_load(w, dtype, j * w_ld + d);
      if (round_mode == 1) {
        float f = (float)acc;
        acc = dtype == OR_BF16 ? (double)or_round_bf16(f) : (double)f;
      }
      x[j] = acc;
    }
    double m = -INFINITY;
    for (int64_t j = 0; j < V; ++j)
      if (x[j] > m) m = x[j];
    double ssum = 0.0;
    for (int64_t j = 0; j < V; ++j) ssum += exp(x[j] - m);
    const double lse = m + log(ssum);
    double loss = 0.0;
    for (int64_t j = 0; j < V; ++j) {
      const double q = or_q(smooth, alpha, V, j == tgt);
      if (q != 0.0) loss -= q * (x[j] - lse);
    }
    loss_out[r] = loss;
    const double s = or_scale(reduce, g_row, g_scalar, n_valid, r);
    for (int64_t j = 0; j < V; ++j) x[j] = s * (exp(x[j] - lse) - or_q(smooth, alpha, V, j == tgt));
  }
  if (dh_out) {
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < N; ++r)
      for (int64_t d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int64_t j = 0; j < V; ++j) acc += G[r * V + j] * or_load(w, dtype, j * w_ld + d);
        dh_out[r * D + d] = acc;
      }
  }
  if (dw_out) {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < V; ++j)
      for (int64_t d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int64_t r = 0; r < N; ++r) acc += G[r * V + j] * or_load(h, dtype, r * h_ld + d);
        dw_out[j * D + d] = acc;
      }
  }
  if (g_out) memcpy(g_out, G, sizeof(double) * (size_t)N * (size_t)V);
  free(G);
  return bad ? OR_EBADTARGET : 0;
}

/* Threads the OpenMP runtime would use for the parallel loops above. */
int or_max_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
