// A consumer of the C ABI with no Python and no torch: HIP device memory from
// hipMalloc, libce.so's ce_workspace_init and ce_fwd_bwd_fused on the null
// stream, then ce_shards_fwd_bwd_fused on the same logits held as three
// separately allocated vocabulary shards, each checked against the FP64
// oracle's C library (test infrastructure, linked only here).  Written in
// plain C style; compiled with hipcc.
//
// Inputs: 2 x 37 rows of 5003 BF16 logits (a misaligned row length), label
// smoothing 0.1, mean over the non-ignored rows, every ninth target ignored;
// values from a fixed linear congruential generator; shards of 1668, 1668
// and 1667 columns.  Bar: n exact, loss within 1e-4 max(1, |ref|), gradient
// within 2^-8 |ref| + 1e-7, ignored rows +0.0.  Prints "c abi ok" and exits
// 0, or prints the first mismatch and exits 1.
//
// Then the chunked head on the library's own MFMA GEMM (gemm = CE_GEMM_NATIVE,
// confirmed by ce_linear_gemm_plan): 300 rows of D = 136 BF16 hidden values
// (a K tail past the 128-deep tiles), V = 3001 head rows (a logits row stride
// padded to 3008), chunks of 128 rows (a ragged last chunk), label smoothing
// 0.1, mean reduction, every seventh target ignored.  Inputs sit on a grid
// (h = k/8, W = m/64) so every partial sum of the logits is exact in FP32 and
// the logits match the oracle's bit for bit in any summation order.  Bars:
// n exact, loss within 1e-4 max(1, |ref|); dh and dW within the bars derived
// from the gradient bar and FP32 accumulation (gamma_K = K 2^-24):
//   dh_id: (2^-8 + gamma_V) sum_j |G_ij| |W_jd| + 1e-7 sum_j |W_jd|, plus
//          2^-8 of the result for its BF16 rounding;
//   dW_jd: (2^-8 + gamma_N) sum_i |G_ij| |h_id| + 1e-7 sum_i |h_id| + 2^-23 |ref|.
// Prints "c abi ok (linear, native)".
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "ce.h"
#include "ce_oracle.h"

#define HIP_OK(x)                                                  \
  do {                                                             \
    hipError_t e_ = (x);                                           \
    if (e_ != hipSuccess) {                                        \
      printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
      return 1;                                                    \
    }                                                              \
  } while (0)

static uint64_t lcg_state = 0x9e3779b97f4a7c15ull;
static double lcg_uniform(void) {  // [0, 1)
  lcg_state = lcg_state * 6364136223846793005ull + 1442695040888963407ull;
  return (double)(lcg_state >> 11) * (1.0 / 9007199254740992.0);
}

static uint16_t bf16_of(float f) {  // nearest even
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  u = u + 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static float float_of_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

// n, the mean loss and every gradient element against the oracle's
static int check(const char* what, int32_t n, float loss, int64_t n_ref, double mean_ref, const uint16_t* grad,
                 const double* ref_grad, const int64_t* t, int64_t N, int64_t V, double* max_err) {
  if ((int64_t)n != n_ref) {
    printf("%s: n %d, oracle %lld\n", what, n, (long long)n_ref);
    return 1;
  }
  if (!(fabs((double)loss - mean_ref) <= 1e-4 * fmax(1.0, fabs(mean_ref)))) {
    printf("%s: mean loss %.9g, oracle %.9g\n", what, (double)loss, mean_ref);
    return 1;
  }
  *max_err = 0.0;
  for (int64_t i = 0; i < N * V; ++i) {
    const int64_t r = i / V;
    if (t[r] == -100 && grad[i] != 0) {
      printf("%s: ignored row %lld element %lld is not +0.0\n", what, (long long)r, (long long)(i % V));
      return 1;
    }
    const double g = (double)float_of_bf16(grad[i]), err = fabs(g - ref_grad[i]);
    if (!(err <= ldexp(1.0, -8) * fabs(ref_grad[i]) + 1e-7)) {
      printf("%s: gradient row %lld column %lld: %.9g, oracle %.9g\n", what, (long long)r, (long long)(i % V), g,
             ref_grad[i]);
      return 1;
    }
    if (err > *max_err) *max_err = err;
  }
  return 0;
}

// The chunked head through the C ABI on the native engine, against or_linear_ce.
static int linear_head(void) {
  const int64_t N = 300, D = 136, V = 3001, chunk = 128;
  const float alpha = 0.1f;
  uint16_t* h = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(N * D));
  uint16_t* w = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(V * D));
  uint16_t* dh = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(N * D));
  float* dw = (float*)malloc(sizeof(float) * (size_t)(V * D));
  int64_t* t = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
  double* ref_loss = (double*)malloc(sizeof(double) * (size_t)N);
  double* ref_dh = (double*)malloc(sizeof(double) * (size_t)(N * D));
  double* ref_dw = (double*)malloc(sizeof(double) * (size_t)(V * D));
  double* G = (double*)malloc(sizeof(double) * (size_t)(N * V));
  double* bar_h = (double*)calloc((size_t)(N * D), sizeof(double));
  double* bar_w = (double*)calloc((size_t)(V * D), sizeof(double));
  double* wabs = (double*)calloc((size_t)D, sizeof(double));
  double* habs = (double*)calloc((size_t)D, sizeof(double));
  if (!h || !w || !dh || !dw || !t || !ref_loss || !ref_dh || !ref_dw || !G || !bar_h || !bar_w || !wabs || !habs) {
    printf("host allocation failed\n");
    return 1;
  }
  for (int64_t i = 0; i < N * D; ++i) h[i] = bf16_of((float)((int)(lcg_uniform() * 9.0) - 4) / 8.0f);
  for (int64_t i = 0; i < V * D; ++i) w[i] = bf16_of((float)((int)(lcg_uniform() * 17.0) - 8) / 64.0f);
  for (int64_t r = 0; r < N; ++r) t[r] = r % 7 == 3 ? -100 : (int64_t)(lcg_uniform() * (double)V);

  ce_linear lin;
  memset(&lin, 0, sizeof lin);
  lin.dtype = CE_BF16;
  lin.gemm = CE_GEMM_NATIVE;
  lin.N = N;
  lin.D = D;
  lin.V = V;
  lin.h_ld = D;
  lin.w_ld = D;
  ce_params p;
  memset(&p, 0, sizeof p);
  p.label_smoothing = alpha;
  p.reduce_loss = CE_REDUCE_MEAN;
  p.ignore_idx = -100;
  p.smoothing = CE_SMOOTH_ALL;
  void *dhd, *dwd, *ddh, *ddw, *dt, *dloss, *dn, *dws;
  HIP_OK(hipMalloc(&dhd, sizeof(uint16_t) * (size_t)(N * D)));
  HIP_OK(hipMalloc(&dwd, sizeof(uint16_t) * (size_t)(V * D)));
  HIP_OK(hipMalloc(&ddh, sizeof(uint16_t) * (size_t)(N * D)));
  HIP_OK(hipMalloc(&ddw, sizeof(float) * (size_t)(V * D)));
  HIP_OK(hipMalloc(&dt, sizeof(int64_t) * (size_t)N));
  HIP_OK(hipMalloc(&dloss, sizeof(float)));
  HIP_OK(hipMalloc(&dn, sizeof(int32_t)));
  HIP_OK(hipMemcpy(dhd, h, sizeof(uint16_t) * (size_t)(N * D), hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dwd, w, sizeof(uint16_t) * (size_t)(V * D), hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dt, t, sizeof(int64_t) * (size_t)N, hipMemcpyHostToDevice));
  lin.h = dhd;
  lin.w = dwd;
  int64_t chunk_used = 0;
  const size_t ws_bytes = ce_linear_workspace_bytes(&lin, &p, chunk, &chunk_used);
  if (ws_bytes == 0 || chunk_used != chunk) {
    printf("ce_linear_workspace_bytes: %s (chunk %lld)\n", ce_last_error(), (long long)chunk_used);
    return 1;
  }
  HIP_OK(hipMalloc(&dws, ws_bytes));
  const int32_t plan = ce_linear_gemm_plan(&lin);
  if (plan != 7) {
    printf("ce_linear_gemm_plan: %d, expected 7 (all three products on the native kernel)\n", plan);
    return 1;
  }
  ce_status st = ce_workspace_init(dws, ws_bytes, NULL);
  if (st == CE_OK)
    st = ce_linear_cross_entropy(&lin, (const int64_t*)dt, 1, &p, NULL, (float*)dloss, (int32_t*)dn, ddh, D,
                                 (float*)ddw, D, 0, chunk, dws, ws_bytes, NULL);
  if (st != CE_OK) {
    printf("%s: %s\n", ce_status_string(st), ce_last_error());
    return 1;
  }
  HIP_OK(hipDeviceSynchronize());
  if ((st = ce_workspace_check(dws, NULL)) != CE_OK) {
    printf("%s: %s\n", ce_status_string(st), ce_last_error());
    return 1;
  }
  float loss;
  int32_t n;
  HIP_OK(hipMemcpy(&loss, dloss, sizeof loss, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&n, dn, sizeof n, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(dh, ddh, sizeof(uint16_t) * (size_t)(N * D), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(dw, ddw, sizeof(float) * (size_t)(V * D), hipMemcpyDeviceToHost));

  or_targets ot = {t, N, 1};
  const int64_t n_ref = or_count_valid(&ot, 1, N, -100);
  if (or_linear_ce(h, w, OR_BF16, N, D, V, D, D, t, 1, alpha, OR_SMOOTH_ALL, -100, OR_REDUCE_MEAN, NULL, 1.0, n_ref,
                   1, ref_loss, ref_dh, ref_dw, G)) {
    printf("oracle rejected the head inputs\n");
    return 1;
  }
  const double mean_ref = or_mean_loss(ref_loss, N, n_ref);
  if ((int64_t)n != n_ref) {
    printf("linear: n %d, oracle %lld\n", n, (long long)n_ref);
    return 1;
  }
  if (!(fabs((double)loss - mean_ref) <= 1e-4 * fmax(1.0, fabs(mean_ref)))) {
    printf("linear: mean loss %.9g, oracle %.9g\n", (double)loss, mean_ref);
    return 1;
  }
  // the bars' sums of magnitudes
  for (int64_t i = 0; i < N; ++i)
    for (int64_t j = 0; j < V; ++j) {
      const double g = fabs(G[i * V + j]);
      if (g == 0.0) continue;
      for (int64_t d = 0; d < D; ++d) {
        bar_h[i * D + d] += g * fabs((double)float_of_bf16(w[j * D + d]));
        bar_w[j * D + d] += g * fabs((double)float_of_bf16(h[i * D + d]));
      }
    }
  for (int64_t d = 0; d < D; ++d) {
    for (int64_t j = 0; j < V; ++j) wabs[d] += fabs((double)float_of_bf16(w[j * D + d]));
    for (int64_t i = 0; i < N; ++i) habs[d] += fabs((double)float_of_bf16(h[i * D + d]));
  }
  const double r_g = ldexp(1.0, -8), a_g = 1e-7, eps32 = ldexp(1.0, -24);
  double max_dh = 0.0, max_dw = 0.0;
  for (int64_t i = 0; i < N; ++i)
    for (int64_t d = 0; d < D; ++d) {
      const double ref = ref_dh[i * D + d], got = (double)float_of_bf16(dh[i * D + d]);
      double tol = (r_g + (double)V * eps32) * bar_h[i * D + d] + a_g * wabs[d];
      tol += ldexp(1.0, -8) * (fabs(ref) + tol);
      const double err = fabs(got - ref);
      if (!(err <= tol)) {
        printf("linear: dh row %lld column %lld: %.9g, oracle %.9g, bar %.3g\n", (long long)i, (long long)d, got, ref,
               tol);
        return 1;
      }
      if (err > max_dh) max_dh = err;
    }
  for (int64_t j = 0; j < V; ++j)
    for (int64_t d = 0; d < D; ++d) {
      const double ref = ref_dw[j * D + d], got = (double)dw[j * D + d];
      double tol = (r_g + (double)N * eps32) * bar_w[j * D + d] + a_g * habs[d];
      tol += ldexp(1.0, -23) * (fabs(ref) + tol);
      const double err = fabs(got - ref);
      if (!(err <= tol)) {
        printf("linear: dW row %lld column %lld: %.9g, oracle %.9g, bar %.3g\n", (long long)j, (long long)d, got, ref,
               tol);
        return 1;
      }
      if (err > max_dw) max_dw = err;
    }
  printf("c abi ok (linear, native): n %d, mean loss %.6f (oracle %.6f), max dh error %.2e, max dW error %.2e\n", n,
         (double)loss, mean_ref, max_dh, max_dw);
  hipFree(dhd);
  hipFree(dwd);
  hipFree(ddh);
  hipFree(ddw);
  hipFree(dt);
  hipFree(dloss);
  hipFree(dn);
  hipFree(dws);
  free(h);
  free(w);
  free(dh);
  free(dw);
  free(t);
  free(ref_loss);
  free(ref_dh);
  free(ref_dw);
  free(G);
  free(bar_h);
  free(bar_w);
  free(wabs);
  free(habs);
  return 0;
}

int main(void) {
  const int64_t d0 = 2, d1 = 37, V = 5003, N = d0 * d1;
  const float alpha = 0.1f;
  uint16_t* x = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(N * V));
  uint16_t* grad = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(N * V));
  int64_t* t = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
  double* ref_loss = (double*)malloc(sizeof(double) * (size_t)N);
  double* ref_grad = (double*)malloc(sizeof(double) * (size_t)(N * V));
  int64_t* rows = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
  for (int64_t i = 0; i < N * V; ++i) {
    // sum of four uniforms: mean 0, standard deviation about 2
    double u = lcg_uniform() + lcg_uniform() + lcg_uniform() + lcg_uniform() - 2.0;
    x[i] = bf16_of((float)(u * 3.46));
  }
  for (int64_t r = 0; r < N; ++r) {
    t[r] = r % 9 == 4 ? -100 : (int64_t)(lcg_uniform() * (double)V);
    rows[r] = r;
  }

  void *dx, *dt, *dloss, *dn, *dws;
  HIP_OK(hipMalloc(&dx, sizeof(uint16_t) * (size_t)(N * V)));
  HIP_OK(hipMalloc(&dt, sizeof(int64_t) * (size_t)N));
  HIP_OK(hipMalloc(&dloss, sizeof(float)));
  HIP_OK(hipMalloc(&dn, sizeof(int32_t)));
  HIP_OK(hipMemcpy(dx, x, sizeof(uint16_t) * (size_t)(N * V), hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(dt, t, sizeof(int64_t) * (size_t)N, hipMemcpyHostToDevice));

  ce_logits xl;
  memset(&xl, 0, sizeof xl);
  xl.data = dx;
  xl.dtype = CE_BF16;
  xl.d0 = d0;
  xl.d1 = d1;
  xl.s0 = d1 * V;
  xl.s1 = V;
  xl.v_local = V;
  xl.vocab_total = V;
  ce_targets tl = {(const int64_t*)dt, d1, 1};
  ce_params p;
  memset(&p, 0, sizeof p);
  p.label_smoothing = alpha;
  p.reduce_loss = CE_REDUCE_MEAN;
  p.ignore_idx = -100;
  p.smoothing = CE_SMOOTH_ALL;
  const size_t ws_bytes = ce_workspace_bytes(&xl, &p);
  if (ws_bytes == 0) {
    printf("ce_workspace_bytes: %s\n", ce_last_error());
    return 1;
  }
  HIP_OK(hipMalloc(&dws, ws_bytes));
  ce_status st = ce_workspace_init(dws, ws_bytes, NULL);
  if (st == CE_OK) st = ce_fwd_bwd_fused(&xl, &tl, &p, NULL, (float*)dloss, (int32_t*)dn, dws, ws_bytes, NULL);
  if (st != CE_OK) {
    printf("%s: %s\n", ce_status_string(st), ce_last_error());
    return 1;
  }
  HIP_OK(hipDeviceSynchronize());
  if ((st = ce_workspace_check(dws, NULL)) != CE_OK) {
    printf("%s: %s\n", ce_status_string(st), ce_last_error());
    return 1;
  }
  float loss;
  int32_t n;
  HIP_OK(hipMemcpy(&loss, dloss, sizeof loss, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&n, dn, sizeof n, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(grad, dx, sizeof(uint16_t) * (size_t)(N * V), hipMemcpyDeviceToHost));

  or_logits ol = {x, OR_BF16, 0, d0, d1, d1 * V, V, V, 0, V};
  or_targets ot = {t, d1, 1};
  const int64_t n_ref = or_count_valid(&ot, d0, d1, -100);
  if (or_loss_rows(&ol, &ot, alpha, OR_SMOOTH_ALL, -100, rows, N, ref_loss, NULL) ||
      or_grad_rows(&ol, &ot, alpha, OR_SMOOTH_ALL, -100, OR_REDUCE_MEAN, NULL, 1.0, n_ref, rows, N, ref_grad)) {
    printf("oracle rejected the inputs\n");
    return 1;
  }
  const double mean_ref = or_mean_loss(ref_loss, N, n_ref);
  double max_err = 0.0;
  if (check("fused", n, loss, n_ref, mean_ref, grad, ref_grad, t, N, V, &max_err)) return 1;
  printf("c abi ok: n %d, mean loss %.6f (oracle %.6f), max gradient error %.2e\n", n, (double)loss, mean_ref,
         max_err);

  // the same logits as three vocabulary shards in their own allocations
  enum { S = 3 };
  const int64_t width = (V + S - 1) / S;
  void* dsh[S];
  ce_logits sl[S];
  for (int s = 0; s < S; ++s) {
    const int64_t a = s * width, w = (a + width <= V ? width : V - a);
    HIP_OK(hipMalloc(&dsh[s], sizeof(uint16_t) * (size_t)(N * w)));
    HIP_OK(hipMemcpy2D(dsh[s], sizeof(uint16_t) * (size_t)w, x + a, sizeof(uint16_t) * (size_t)V,
                       sizeof(uint16_t) * (size_t)w, (size_t)N, hipMemcpyHostToDevice));
    memset(&sl[s], 0, sizeof sl[s]);
    sl[s].data = dsh[s];
    sl[s].dtype = CE_BF16;
    sl[s].d0 = d0;
    sl[s].d1 = d1;
    sl[s].s0 = d1 * w;
    sl[s].s1 = w;
    sl[s].v_local = w;
    sl[s].vocab_start = a;
    sl[s].vocab_total = V;
  }
  const size_t sws_bytes = ce_shards_workspace_bytes(sl, S, &p);
  void* dsws;
  if (sws_bytes == 0) {
    printf("ce_shards_workspace_bytes: %s\n", ce_last_error());
    return 1;
  }
  HIP_OK(hipMalloc(&dsws, sws_bytes));
  st = ce_workspace_init(dsws, sws_bytes, NULL);
  if (st == CE_OK) st = ce_shards_fwd_bwd_fused(sl, S, &tl, &p, NULL, (float*)dloss, (int32_t*)dn, dsws, sws_bytes, NULL);
  if (st != CE_OK) {
    printf("%s: %s\n", ce_status_string(st), ce_last_error());
    return 1;
  }
  HIP_OK(hipDeviceSynchronize());
  if ((st = ce_workspace_check(dsws, NULL)) != CE_OK) {
    printf("%s: %s\n", ce_status_string(st), ce_last_error());
    return 1;
  }
  HIP_OK(hipMemcpy(&loss, dloss, sizeof loss, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&n, dn, sizeof n, hipMemcpyDeviceToHost));
  for (int s = 0; s < S; ++s) {
    const int64_t a = s * width, w = sl[s].v_local;
    HIP_OK(hipMemcpy2D(grad + a, sizeof(uint16_t) * (size_t)V, dsh[s], sizeof(uint16_t) * (size_t)w,
                       sizeof(uint16_t) * (size_t)w, (size_t)N, hipMemcpyDeviceToHost));
  }
  if (check("shards", n, loss, n_ref, mean_ref, grad, ref_grad, t, N, V, &max_err)) return 1;
  printf("c abi ok (3 shards): n %d, mean loss %.6f (oracle %.6f), max gradient error %.2e\n", n, (double)loss,
         mean_ref, max_err);
  for (int s = 0; s < S; ++s) hipFree(dsh[s]);
  hipFree(dsws);
  hipFree(dx);
  hipFree(dt);
  hipFree(dloss);
  hipFree(dn);
  hipFree(dws);
  free(x);
  free(grad);
  free(t);
  free(ref_loss);
  free(ref_grad);
  free(rows);
  return linear_head();
}
