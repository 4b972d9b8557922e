// Chunked linear + cross-entropy (the language-model head and its loss over
// row chunks): argument checks, workspace layout, the GEMM plans, and the
// per-chunk sequence GEMM -> fused cross-entropy -> two backward GEMMs.
//
// Layout in the column-major terms of the GEMM library (row-major [R, C]
// with row stride ld is column-major [C, R] with the same ld):
//   logits_c^T [V, n] = W [V, D] . h_c^T [D, n]   A = W   (col [D, V], op T), B = h_c (col [D, n], op N)
//   dh_c^T     [D, n] = W^T [D, V] . G_c^T [V, n] A = W   (col [D, V], op N), B = G_c (col [V, n], op N)
//   dW^T       [D, V] = h_c^T [D, n] . G_c [n, V] A = h_c (col [D, n], op N), B = G_c (col [V, n], op T)
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <map>
#include <mutex>
#include <tuple>

#include <hip/hip_runtime_api.h>
#include <hipblaslt/hipblaslt.h>

#include "ce.h"
#include "ce_internal.h"

namespace {

ce_status lfail(ce_status s, const char* fmt, ...) {
  char msg[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(msg, sizeof msg, fmt, ap);
  va_end(ap);
  vce::set_last_error(msg);
  return s;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

constexpr size_t kBlasWorkspace = 64ull << 20;   // the GEMM library's scratch, inside the caller's workspace
// automatic chunk: about this many bytes of logits.  On 8192 x 4096 x 128000
// BF16 a step took 32.0 ms in chunks of 1024 rows (256 MiB), 23.2 ms in 2048,
// 21.4 ms in 4096 and 20.8 ms in one chunk: the dh product has few output
// tiles and the dW product re-reads and re-writes its FP32 accumulator
// once per chunk, so small chunks cost GEMM efficiency.  1 GiB is a small
// share of the device's memory and keeps most of the gain.
constexpr size_t kChunkTarget = 1ull << 30;

// ---- GEMM plans: one per (device, types, shape, ops, leading dims, beta != 0),
// built on first use (heuristic query) and kept until the process ends.
struct Plan {
  hipblasLtHandle_t handle = nullptr;
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatrixLayout_t a = nullptr, b = nullptr, c = nullptr;
  hipblasLtMatmulAlgo_t algo;
  bool tuned = false;  // algo chosen by timing the heuristic's candidates (ce_linear_tune)
};
constexpr int kTuneCandidates = 8;
typedef std::tuple<int, int, int, int64_t, int64_t, int64_t, int, int, int64_t, int64_t, int64_t> PlanKey;

std::mutex g_blas_mu;
std::map<int, hipblasLtHandle_t> g_handles;
std::map<PlanKey, Plan> g_plans;

const char* blas_status(hipblasStatus_t s) {
  switch (s) {
    case HIPBLAS_STATUS_SUCCESS: return "success";
    case HIPBLAS_STATUS_NOT_INITIALIZED: return "not initialized";
    case HIPBLAS_STATUS_ALLOC_FAILED: return "allocation failed";
    case HIPBLAS_STATUS_INVALID_VALUE: return "invalid value";
    case HIPBLAS_STATUS_ARCH_MISMATCH: return "architecture mismatch";
    case HIPBLAS_STATUS_EXECUTION_FAILED: return "execution failed";
    case HIPBLAS_STATUS_NOT_SUPPORTED: return "not supported";
    default: return "error";
  }
}

// One GEMM: D = alpha op(A) op(B) + beta D, column-major, m x n x k.
struct Gemm {
  hipDataType ab, cd;
  int64_t m, n, k;
  hipblasOperation_t opa, opb;
  const void* A;
  int64_t lda;
  const void* B;
  int64_t ldb;
  void* D;
  int64_t ldd;
  float beta;
};

ce_status get_plan(int dev, const Gemm& g, Plan** out) {
  std::lock_guard<std::mutex> lk(g_blas_mu);
  hipblasLtHandle_t h;
  auto hi = g_handles.find(dev);
  if (hi == g_handles.end()) {
    hipblasStatus_t s = hipblasLtCreate(&h);
    if (s != HIPBLAS_STATUS_SUCCESS) return lfail(CE_EHIP, "hipblasLtCreate: %s", blas_status(s));
    g_handles[dev] = h;
  } else {
    h = hi->second;
  }
  const PlanKey key{dev, (int)g.ab, (int)g.cd, g.m, g.n, g.k, (int)g.opa, (int)g.opb, g.lda, g.ldb,
                    g.ldd * 2 + (g.beta != 0.f)};
  auto it = g_plans.find(key);
  if (it != g_plans.end()) {
    *out = &it->second;
    return CE_OK;
  }
  Plan p;
  hipblasStatus_t s;
  const int32_t opa = g.opa, opb = g.opb;
  const uint64_t ar = g.opa == HIPBLAS_OP_N ? g.m : g.k, ac = g.opa == HIPBLAS_OP_N ? g.k : g.m;
  const uint64_t br = g.opb == HIPBLAS_OP_N ? g.k : g.n, bc = g.opb == HIPBLAS_OP_N ? g.n : g.k;
  hipblasLtMatmulPreference_t pref = nullptr;
  hipblasLtMatmulHeuristicResult_t res[8];
  int nres = 0;
  const uint64_t wsmax = kBlasWorkspace;
  if ((s = hipblasLtMatmulDescCreate(&p.desc, HIPBLAS_COMPUTE_32F, HIP_R_32F)) ||
      (s = hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opa, sizeof opa)) ||
      (s = hipblasLtMatmulDescSetAttribute(p.desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opb, sizeof opb)) ||
      (s = hipblasLtMatrixLayoutCreate(&p.a, g.ab, ar, ac, g.lda)) ||
      (s = hipblasLtMatrixLayoutCreate(&p.b, g.ab, br, bc, g.ldb)) ||
      (s = hipblasLtMatrixLayoutCreate(&p.c, g.cd, g.m, g.n, g.ldd)) ||
      (s = hipblasLtMatmulPreferenceCreate(&pref)) ||
      (s = hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsmax,
                                                 sizeof wsmax)) ||
      (s = hipblasLtMatmulAlgoGetHeuristic(h, p.desc, p.a, p.b, p.c, p.c, pref, 8, res, &nres))) {
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    return lfail(CE_EHIP, "GEMM plan %lld x %lld x %lld: %s", (long long)g.m, (long long)g.n, (long long)g.k,
                 blas_status(s));
  }
  hipblasLtMatmulPreferenceDestroy(pref);
  int pick = -1;
  for (int i = 0; i < nres && pick < 0; ++i)
    if (res[i].state == HIPBLAS_STATUS_SUCCESS && res[i].workspaceSize <= kBlasWorkspace) pick = i;
  if (pick < 0)
    return lfail(CE_ELAYOUT, "no GEMM algorithm for %lld x %lld x %lld (leading dims %lld, %lld, %lld)",
                 (long long)g.m, (long long)g.n, (long long)g.k, (long long)g.lda, (long long)g.ldb,
                 (long long)g.ldd);
  p.algo = res[pick].algo;
  p.handle = h;
  *out = &g_plans.emplace(key, p).first->second;
  return CE_OK;
}

ce_status run_gemm(int dev, const Gemm& g, void* blas_ws, hipStream_t stream) {
  Plan* p = nullptr;
  ce_status st = get_plan(dev, g, &p);
  if (st) return st;
  const float alpha = 1.f;
  // hipBLASLt states no thread safety for a handle or descriptor shared by host threads, and two threads'
  // calls on one plan at the same time have failed (execution failed), so the enqueue is serialised; the
  // kernels still run concurrently on the callers' streams.  The lock also covers ce_linear_tune replacing
  // the plan's algorithm from another thread.
  hipblasStatus_t s;
  {
    std::lock_guard<std::mutex> lk(g_blas_mu);
    s = hipblasLtMatmul(p->handle, p->desc, &alpha, g.A, p->a, g.B, p->b, &g.beta, g.D, p->c, g.D, p->c, &p->algo,
                        blas_ws, kBlasWorkspace, stream);
  }
  if (s != HIPBLAS_STATUS_SUCCESS)
    return lfail(CE_EHIP, "GEMM %lld x %lld x %lld: %s", (long long)g.m, (long long)g.n, (long long)g.k,
                 blas_status(s));
  return CE_OK;
}

// Times the heuristic's first kTuneCandidates algorithms for g on the given
// buffers (stream synchronised): kTuneRounds interleaved rounds of one
// warm-up and three timed runs each, a candidate's time its best round.  The
// plan switches from the heuristic's first choice only to a candidate at
// least kTuneMargin faster (timings on this chip vary by a few percent with
// power and clocks).
constexpr int kTuneRounds = 3;
constexpr float kTuneMargin = 0.97f;
ce_status tune_gemm(int dev, const Gemm& g, void* blas_ws, hipStream_t stream) {
  Plan* p = nullptr;
  ce_status st = get_plan(dev, g, &p);
  if (st) return st;
  if (p->tuned) return CE_OK;
  hipblasLtMatmulHeuristicResult_t res[kTuneCandidates];
  int nres = 0;
  {
    std::lock_guard<std::mutex> lk(g_blas_mu);  // the plan's descriptors are shared with other threads' calls
    hipblasLtMatmulPreference_t pref = nullptr;
    const uint64_t wsmax = kBlasWorkspace;
    hipblasStatus_t s;
    if ((s = hipblasLtMatmulPreferenceCreate(&pref)) ||
        (s = hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsmax,
                                                   sizeof wsmax)) ||
        (s = hipblasLtMatmulAlgoGetHeuristic(p->handle, p->desc, p->a, p->b, p->c, p->c, pref, kTuneCandidates, res,
                                             &nres))) {
      if (pref) hipblasLtMatmulPreferenceDestroy(pref);
      return lfail(CE_EHIP, "GEMM candidates: %s", blas_status(s));
    }
    hipblasLtMatmulPreferenceDestroy(pref);
  }
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e;
  if ((e = hipEventCreate(&e0)) || (e = hipEventCreate(&e1))) {
    if (e0) (void)hipEventDestroy(e0);
    return lfail(CE_EHIP, "event create: %s", hipGetErrorString(e));
  }
  const float alpha = 1.f;
  float best[kTuneCandidates];
  for (int i = 0; i < kTuneCandidates; ++i) best[i] = 1e30f;
  for (int round = 0; round < kTuneRounds; ++round) {
    for (int i = 0; i < nres; ++i) {
      if (res[i].state != HIPBLAS_STATUS_SUCCESS || res[i].workspaceSize > kBlasWorkspace) continue;
      bool ok = true;
      for (int rep = 0; rep < 4 && ok; ++rep) {
        if (rep == 1 && hipEventRecord(e0, stream)) ok = false;
        std::lock_guard<std::mutex> lk(g_blas_mu);
        ok = ok && hipblasLtMatmul(p->handle, p->desc, &alpha, g.A, p->a, g.B, p->b, &g.beta, g.D, p->c, g.D,
                                   p->c, &res[i].algo, blas_ws, kBlasWorkspace, stream) == HIPBLAS_STATUS_SUCCESS;
      }
      float ms = 0.f;
      if (!ok || hipEventRecord(e1, stream) || hipEventSynchronize(e1) || hipEventElapsedTime(&ms, e0, e1)) continue;
      if (ms < best[i]) best[i] = ms;
    }
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  int pick = 0;
  for (int i = 1; i < nres; ++i)
    if (best[i] < best[pick]) pick = i;
  std::lock_guard<std::mutex> lk(g_blas_mu);
  if (nres > 0 && best[0] < 1e30f && best[pick] < kTuneMargin * best[0]) p->algo = res[pick].algo;
  p->tuned = true;
  return CE_OK;
}

int elem_bytes(int32_t dtype) { return dtype == CE_BF16 ? 2 : 4; }

ce_status check_linear(const ce_linear* lin, const ce_params* p) {
  if (!lin) return lfail(CE_EINVAL, "linear descriptor is NULL");
  if (!p) return lfail(CE_EINVAL, "params is NULL");
  if (lin->dtype != CE_F32 && lin->dtype != CE_BF16) return lfail(CE_EDTYPE, "unsupported dtype %d", lin->dtype);
  if (lin->gemm != CE_GEMM_AUTO && lin->gemm != CE_GEMM_NATIVE && lin->gemm != CE_GEMM_LIBRARY)
    return lfail(CE_EINVAL, "linear.gemm must be CE_GEMM_AUTO, CE_GEMM_NATIVE or CE_GEMM_LIBRARY (got %d)", lin->gemm);
  if (lin->N < 0 || lin->D < 1 || lin->V < 1)
    return lfail(CE_EINVAL, "need N >= 0, D >= 1, V >= 1 (got %lld, %lld, %lld)", (long long)lin->N,
                 (long long)lin->D, (long long)lin->V);
  if (lin->N > 0x7fffffffLL || lin->V > 0x7fffffffLL || lin->D > 0x7fffffffLL)
    return lfail(CE_EINVAL, "sizes above 2^31-1");
  if (lin->h_ld < lin->D || lin->w_ld < lin->D) return lfail(CE_ELAYOUT, "row strides must be >= D");
  const uintptr_t eb = (uintptr_t)elem_bytes(lin->dtype);
  if ((lin->N > 0 && !lin->h) || !lin->w) return lfail(CE_EINVAL, "h or w is NULL");
  if ((uintptr_t)lin->h % eb || (uintptr_t)lin->w % eb) return lfail(CE_ELAYOUT, "h or w not aligned to its dtype");
  if (p->split_chunks != 0) return lfail(CE_EINVAL, "split_chunks must be 0 for the chunked linear call");
  return CE_OK;
}

int64_t auto_chunk(const ce_linear* lin, int64_t chunk_rows) {
  if (lin->N == 0) return 1;
  int64_t c = chunk_rows;
  if (c <= 0) {
    c = (int64_t)(kChunkTarget / ((size_t)lin->V * (size_t)elem_bytes(lin->dtype)));
    if (c >= 256) c -= c % 256;
    if (c < 1) c = 1;
  }
  return c < lin->N ? c : lin->N;
}

// header and fused-call regions | chunk logits | per-chunk loss sums | scale | GEMM scratch
struct LinLayout {
  size_t fused = 0;   // bytes the per-chunk fused call needs (its regions start at 0)
  size_t logits = 0, parts = 0, scale = 0, blas = 0, total = 0;
  int64_t chunk = 0, nchunks = 0;
  int64_t ldl = 0;    // the chunk logits' row stride: V rounded up to a multiple of 8 (16-byte BF16 rows)
};

ce_status lin_layout(const ce_linear* lin, const ce_params* p, int64_t chunk_rows, LinLayout* out) {
  LinLayout w;
  w.chunk = auto_chunk(lin, chunk_rows);
  w.nchunks = lin->N == 0 ? 0 : (lin->N + w.chunk - 1) / w.chunk;
  w.fused = vce::fused_workspace_bytes(w.chunk, lin->dtype, lin->V, p->reduce_loss != CE_REDUCE_NONE);
  w.ldl = (lin->V + 7) & ~(int64_t)7;
  size_t off = align256(w.fused);
  w.logits = off;
  off = align256(off + (size_t)w.chunk * (size_t)w.ldl * (size_t)elem_bytes(lin->dtype));
  w.parts = off;
  off = align256(off + (size_t)(w.nchunks > 0 ? w.nchunks : 1) * 4u);
  w.scale = off;  // float s, int32 n
  off = align256(off + 8u);
  w.blas = off;
  off = align256(off + kBlasWorkspace);
  w.total = off;
  *out = w;
  return CE_OK;
}

// The fused call's checks for a chunk of `rows` rows (shape and parameters
// only: the descriptor's address is a placeholder with the buffer's alignment).
ce_status chunk_plan_ok(const ce_linear* lin, const ce_params* p, int64_t rows) {
  ce_logits x{};
  x.data = reinterpret_cast<void*>((uintptr_t)256);
  x.dtype = lin->dtype;
  x.d0 = 1;
  x.d1 = rows;
  x.s1 = (lin->V + 7) & ~(int64_t)7;
  x.v_local = lin->V;
  x.vocab_total = lin->V;
  return vce::fused_plan(&x, p, nullptr, nullptr, nullptr);
}

// The three products of a chunk.  CE_GEMM_NATIVE runs each on the library's
// MFMA kernel (ce_gemm.hip) where it applies (BF16; h and W 16-byte aligned;
// h_ld, w_ld and D multiples of 8), CE_GEMM_LIBRARY on hipBLASLt; CE_GEMM_AUTO
// takes, per product, the engine measured faster on gfx950 at the head's
// shapes (kAutoNative): at 8192 x 4096 x 128000 in chunks of 4096 rows the
// native products take 3.07 ms for dh and 3.45 / 3.67 ms for dW (written /
// added) against the library's 3.11 and 4.21 / 4.45, and 3.22 ms for the
// logits against the library's 2.87.
enum Product { kLogits = 0, kDh = 1, kDw = 2 };
constexpr bool kAutoNative[3] = {false, true, true};

bool native_layout_ok(const ce_linear* lin) {
  return lin->dtype == CE_BF16 && lin->h_ld % 8 == 0 && lin->w_ld % 8 == 0 && lin->D % 8 == 0 &&
         (uintptr_t)lin->h % 16 == 0 && (uintptr_t)lin->w % 16 == 0;
}

bool use_native(const ce_linear* lin, Product prod) {
  if (!native_layout_ok(lin)) return false;
  return lin->gemm == CE_GEMM_NATIVE || (lin->gemm == CE_GEMM_AUTO && kAutoNative[prod]);
}

// One product on the engine chosen for it: the native kernel when selected and its checks pass, else the
// GEMM library with the column-major form `lib`.
ce_status run_product(int dev, const ce_linear* lin, Product prod, const vce::GemmBf16& nat, const Gemm& lib,
                      void* blas_ws, hipStream_t stream) {
  if (use_native(lin, prod) && vce::gemm_bf16_supported(nat)) {
    hipError_t e = vce::launch_gemm_bf16(nat, stream);
    if (e) return lfail(CE_EHIP, "GEMM %d x %d x %d launch: %s", nat.M, nat.N, nat.K, hipGetErrorString(e));
    return CE_OK;
  }
  return run_gemm(dev, lib, blas_ws, stream);
}

}  // namespace

extern "C" {

size_t ce_linear_workspace_bytes(const ce_linear* lin, const ce_params* p, int64_t chunk_rows,
                                 int64_t* chunk_rows_out) {
  if (check_linear(lin, p)) return 0;
  LinLayout w;
  if (lin_layout(lin, p, chunk_rows, &w) || chunk_plan_ok(lin, p, w.chunk)) return 0;
  if (chunk_rows_out) *chunk_rows_out = w.chunk;
  return w.total;
}

int32_t ce_linear_gemm_plan(const ce_linear* lin) {
  if (!lin || (lin->dtype != CE_F32 && lin->dtype != CE_BF16) || lin->N < 0 || lin->D < 1 || lin->V < 1 ||
      lin->N > 0x7fffffffLL || lin->V > 0x7fffffffLL || lin->D > 0x7fffffffLL || lin->h_ld < lin->D ||
      lin->w_ld < lin->D || (lin->gemm != CE_GEMM_AUTO && lin->gemm != CE_GEMM_NATIVE && lin->gemm != CE_GEMM_LIBRARY))
    return -1;
  // the descriptors a chunk of n rows would use (the checks depend on the layouts, not on n or the buffers)
  const int64_t ldl = (lin->V + 7) & ~(int64_t)7, n = lin->N > 0 ? lin->N : 1;
  void* logits = reinterpret_cast<void*>((uintptr_t)256);
  const int N = (int)n, D = (int)lin->D, V = (int)lin->V;
  const vce::GemmBf16 d[3] = {
      {lin->h, lin->h_ld, true, lin->w, lin->w_ld, true, logits, ldl, 0, N, V, D},
      {logits, ldl, true, lin->w, lin->w_ld, false, logits, lin->D, 0, N, D, V},
      {logits, ldl, false, lin->h, lin->h_ld, false, logits, lin->D, 1, V, D, N}};
  int32_t plan = 0;
  for (int k = 0; k < 3; ++k)
    if (use_native(lin, (Product)k) && vce::gemm_bf16_supported(d[k])) plan |= 1 << k;
  return plan;
}

ce_status ce_linear_tune(const ce_linear* lin, const ce_params* p, void* dh, int64_t dh_ld, float* dw,
                         int64_t dw_ld, int64_t chunk_rows, void* ws, size_t ws_bytes, hipStream_t stream) {
  ce_status st;
  if ((st = check_linear(lin, p))) return st;
  const int64_t N = lin->N, D = lin->D, V = lin->V;
  if (dh && (dh_ld < D || (uintptr_t)dh % (uintptr_t)elem_bytes(lin->dtype)))
    return lfail(CE_ELAYOUT, "dh row stride must be >= D and dh aligned to its dtype");
  if (dw && (dw_ld < D || (uintptr_t)dw % 4u)) return lfail(CE_ELAYOUT, "dw row stride must be >= D, dw 4-byte aligned");
  LinLayout w;
  if ((st = lin_layout(lin, p, chunk_rows, &w)) || (st = chunk_plan_ok(lin, p, w.chunk))) return st;
  if (!ws || ws_bytes < w.total)
    return lfail(CE_EWORKSPACE, "workspace of %zu bytes needed, %zu given", w.total, ws ? ws_bytes : (size_t)0);
  if ((uintptr_t)ws % 256u) return lfail(CE_EWORKSPACE, "workspace must be 256-byte aligned");
  int dev = 0;
  hipError_t e;
  if ((e = hipGetDevice(&dev))) return lfail(CE_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  char* wsb = static_cast<char*>(ws);
  char* logits = wsb + w.logits;
  const hipDataType ab = lin->dtype == CE_BF16 ? HIP_R_16BF : HIP_R_32F;
  // the shapes the call uses: a whole chunk and, when N is not a multiple of it, the last one
  int64_t shapes[2] = {w.chunk, N % w.chunk};
  for (int64_t n : shapes) {
    if (n == 0 || N == 0) continue;
    const int64_t ldl = w.ldl;
    // (products that run on the native kernel have nothing to tune)
    if (!use_native(lin, kLogits)) {
      Gemm g1{ab, ab, V, n, D, HIPBLAS_OP_T, HIPBLAS_OP_N, lin->w, lin->w_ld, lin->h, lin->h_ld, logits, ldl, 0.f};
      if ((st = tune_gemm(dev, g1, wsb + w.blas, stream))) return st;
    }
    if (dh && !use_native(lin, kDh)) {
      Gemm g2{ab, ab, D, n, V, HIPBLAS_OP_N, HIPBLAS_OP_N, lin->w, lin->w_ld, logits, ldl, dh, dh_ld, 0.f};
      if ((st = tune_gemm(dev, g2, wsb + w.blas, stream))) return st;
    }
    if (dw && !use_native(lin, kDw)) {
      for (float beta : {0.f, 1.f}) {
        Gemm g3{ab, HIP_R_32F, D, V, n, HIPBLAS_OP_N, HIPBLAS_OP_T, lin->h, lin->h_ld, logits, ldl, dw, dw_ld,
                beta};
        if ((st = tune_gemm(dev, g3, wsb + w.blas, stream))) return st;
      }
    }
  }
  return CE_OK;
}

ce_status ce_linear_cross_entropy(const ce_linear* lin, const int64_t* targets, int64_t t_stride,
                                  const ce_params* p, const float* grad_out, float* loss, int32_t* n_valid,
                                  void* dh, int64_t dh_ld, float* dw, int64_t dw_ld, int32_t accumulate_dw,
                                  int64_t chunk_rows, void* ws, size_t ws_bytes, hipStream_t stream) {
  ce_status st;
  if ((st = check_linear(lin, p))) return st;
  const int64_t N = lin->N, D = lin->D, V = lin->V;
  if (N > 0 && !targets) return lfail(CE_EINVAL, "targets is NULL");
  if ((uintptr_t)targets % 8u || t_stride < 0) return lfail(CE_ELAYOUT, "targets misaligned or negative stride");
  if (!loss && (N > 0 || p->reduce_loss != CE_REDUCE_NONE)) return lfail(CE_EINVAL, "loss is NULL");
  if (dh && (dh_ld < D || (uintptr_t)dh % (uintptr_t)elem_bytes(lin->dtype)))
    return lfail(CE_ELAYOUT, "dh row stride must be >= D and dh aligned to its dtype");
  if (dw && (dw_ld < D || (uintptr_t)dw % 4u)) return lfail(CE_ELAYOUT, "dw row stride must be >= D, dw 4-byte aligned");
  if (accumulate_dw != 0 && accumulate_dw != 1) return lfail(CE_EINVAL, "accumulate_dw must be 0 or 1");
  if (p->smoothing == CE_SMOOTH_OTHERS && p->label_smoothing > 0.f && V < 2)
    return lfail(CE_EINVAL, "smoothing over the other classes needs V >= 2");
  LinLayout w;
  if ((st = lin_layout(lin, p, chunk_rows, &w))) return st;
  // the per-chunk fused call's own checks (parameters, chunking of V), before anything is enqueued
  if ((st = chunk_plan_ok(lin, p, w.chunk))) return st;
  if (!ws || ws_bytes < w.total)
    return lfail(CE_EWORKSPACE, "workspace of %zu bytes needed, %zu given", w.total, ws ? ws_bytes : (size_t)0);
  if ((uintptr_t)ws % 256u) return lfail(CE_EWORKSPACE, "workspace must be 256-byte aligned");
  ce_params q = *p;
  q.reduce_loss = p->reduce_loss == CE_REDUCE_NONE ? CE_REDUCE_NONE : CE_REDUCE_SUM;
  int dev = 0;
  hipError_t e;
  if ((e = hipGetDevice(&dev))) return lfail(CE_EHIP, "hipGetDevice: %s", hipGetErrorString(e));

  char* wsb = static_cast<char*>(ws);
  char* logits = wsb + w.logits;
  float* parts = reinterpret_cast<float*>(wsb + w.parts);
  float* scale = reinterpret_cast<float*>(wsb + w.scale);
  int32_t* n_out = n_valid ? n_valid : reinterpret_cast<int32_t*>(wsb + w.scale + 4);
  const int red = p->reduce_loss;

  // the count over all rows, and for the mean the scale g / n every chunk uses
  if ((e = vce::launch_linear_prep(targets, t_stride, N, p->ignore_idx, red, grad_out, n_out, scale, stream)))
    return lfail(CE_EHIP, "count launch: %s", hipGetErrorString(e));
  if (dw && !accumulate_dw && N == 0 && (e = vce::launch_fill_f32(dw, V, D, dw_ld, stream)))
    return lfail(CE_EHIP, "fill launch: %s", hipGetErrorString(e));

  const hipDataType ab = lin->dtype == CE_BF16 ? HIP_R_16BF : HIP_R_32F;
  const size_t eb = (size_t)elem_bytes(lin->dtype);
  for (int64_t c = 0; c < w.nchunks; ++c) {
    const int64_t r0 = c * w.chunk;
    const int64_t n = N - r0 < w.chunk ? N - r0 : w.chunk;
    const char* hc = static_cast<const char*>(lin->h) + (size_t)r0 * (size_t)lin->h_ld * eb;
    // logits_c = h_c W^T
    const int64_t ldl = w.ldl;
    Gemm g1{ab, ab, V, n, D, HIPBLAS_OP_T, HIPBLAS_OP_N, lin->w, lin->w_ld, hc, lin->h_ld, logits, ldl, 0.f};
    const vce::GemmBf16 n1{hc, lin->h_ld, true, lin->w, lin->w_ld, true, logits, ldl, 0, (int)n, (int)V, (int)D};
    if ((st = run_product(dev, lin, kLogits, n1, g1, wsb + w.blas, stream))) return st;
    // loss and gradient in place
    ce_logits x{};
    x.data = logits;
    x.dtype = lin->dtype;
    x.d0 = 1;
    x.d1 = n;
    x.s0 = 0;
    x.s1 = ldl;
    x.v_local = V;
    x.vocab_start = 0;
    x.vocab_total = V;
    ce_targets t{targets + r0 * t_stride, 0, t_stride};
    const float* gc = red == CE_REDUCE_NONE ? (grad_out ? grad_out + r0 : nullptr)
                                            : (red == CE_REDUCE_MEAN ? scale : grad_out);
    float* lc = red == CE_REDUCE_NONE ? loss + r0 : parts + c;
    if ((st = ce_fwd_bwd_fused(&x, &t, &q, gc, lc, nullptr, ws, w.fused, stream)))
      return lfail(st, "chunk %lld: %s", (long long)c, ce_last_error());
    // dh_c = G_c W
    if (dh) {
      char* dhc = static_cast<char*>(dh) + (size_t)r0 * (size_t)dh_ld * eb;
      Gemm g2{ab, ab, D, n, V, HIPBLAS_OP_N, HIPBLAS_OP_N, lin->w, lin->w_ld, logits, ldl, dhc, dh_ld, 0.f};
      vce::GemmBf16 n2{logits, ldl, true, lin->w, lin->w_ld, false, dhc, dh_ld, 0, (int)n, (int)D, (int)V};
      n2.scratch = wsb + w.blas;  // for a split K range when the chunk has few output tiles
      n2.scratch_bytes = kBlasWorkspace;
      if ((st = run_product(dev, lin, kDh, n2, g2, wsb + w.blas, stream))) return st;
    }
    // dW (+)= G_c^T h_c
    if (dw) {
      const bool add = c > 0 || accumulate_dw;
      Gemm g3{ab, HIP_R_32F, D, V, n, HIPBLAS_OP_N, HIPBLAS_OP_T, hc, lin->h_ld, logits, ldl, dw, dw_ld,
              add ? 1.f : 0.f};
      const vce::GemmBf16 n3{logits, ldl, false, hc, lin->h_ld, false, dw, dw_ld, add ? 2 : 1, (int)V, (int)D, (int)n};
      if ((st = run_product(dev, lin, kDw, n3, g3, wsb + w.blas, stream))) return st;
    }
  }
  if (red != CE_REDUCE_NONE &&
      (e = vce::launch_linear_finish(parts, w.nchunks, red, n_out, loss, stream)))
    return lfail(CE_EHIP, "finish launch: %s", hipGetErrorString(e));
  return CE_OK;
}

}  // extern "C"
