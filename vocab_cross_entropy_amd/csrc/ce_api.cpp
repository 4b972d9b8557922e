// C ABI of the fused cross-entropy library: argument checks, workspace
// layout, and the sequence of kernel launches for each entry point.
// Every check runs before the first HIP call, so a rejected call enqueues
// nothing and touches no buffer.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "ce.h"
#include "ce_internal.h"

namespace {

thread_local char g_err[512] = "";

ce_status fail(ce_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

ce_status hip_fail(hipError_t e, const char* what) {
  return fail(CE_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int elem_bytes(int32_t dtype) { return dtype == CE_BF16 ? 2 : 4; }

constexpr int64_t kMaxChunks = 64;
constexpr int64_t kMaxGrid = 0x7fffffffLL;

// Rows are addressed at i0*s0 + i1*s1; the gradient is written in place, so
// distinct rows must not overlap: with the non-trivial dims sorted by stride,
// each stride must clear the extent of everything below it.
bool rows_disjoint(int64_t d0, int64_t d1, int64_t s0, int64_t s1, int64_t V) {
  struct Dim {
    int64_t n, s;
  } dims[2];
  int nd = 0;
  if (d0 > 1) dims[nd++] = {d0, s0};
  if (d1 > 1) dims[nd++] = {d1, s1};
  if (nd == 2 && dims[0].s > dims[1].s) {
    Dim tmp = dims[0];
    dims[0] = dims[1];
    dims[1] = tmp;
  }
  int64_t extent = V;  // elements spanned by one row
  for (int i = 0; i < nd; ++i) {
    if (dims[i].s < extent) return false;
    if (dims[i].n - 1 > (INT64_MAX - extent) / dims[i].s) return false;
    extent = dims[i].s * (dims[i].n - 1) + extent;
  }
  return true;
}

// Every row starts on a 16-byte boundary and spans whole 16-byte vectors.
int32_t rows_aligned16(const ce_logits* x) {
  const int64_t b = elem_bytes(x->dtype);
  return ((uintptr_t)x->data % 16u == 0) && (x->d0 <= 1 || (x->s0 * b) % 16 == 0) &&
         ((x->s1 * b) % 16 == 0 || x->d1 == 1) && ((x->v_local * b) % 16 == 0);
}

ce_status check_params(const ce_params* p) {
  if (!p) return fail(CE_EINVAL, "params is NULL");
  const float a = p->label_smoothing;
  if (!(a >= 0.f && a <= 1.f)) return fail(CE_EINVAL, "label_smoothing %g is outside [0, 1]", (double)a);
  if (p->reduce_loss != CE_REDUCE_NONE && p->reduce_loss != CE_REDUCE_MEAN && p->reduce_loss != CE_REDUCE_SUM)
    return fail(CE_EINVAL, "reduce_loss %d is not CE_REDUCE_NONE, CE_REDUCE_MEAN or CE_REDUCE_SUM", p->reduce_loss);
  if (p->split_chunks < 0 || p->split_chunks > kMaxChunks)
    return fail(CE_EINVAL, "split_chunks %d outside [0, %lld]", p->split_chunks, (long long)kMaxChunks);
  if (p->smoothing != CE_SMOOTH_ALL && p->smoothing != CE_SMOOTH_OTHERS)
    return fail(CE_EINVAL, "smoothing %d is not CE_SMOOTH_ALL or CE_SMOOTH_OTHERS", p->smoothing);
  return CE_OK;
}

// Smoothing over the other classes divides a by V - 1: a vocabulary of one
// class has no other class to give it to.
ce_status check_smoothing(const ce_params* p, int64_t vocab_total) {
  if (p->smoothing == CE_SMOOTH_OTHERS && p->label_smoothing > 0.f && vocab_total < 2)
    return fail(CE_EINVAL, "smoothing over the other classes needs vocab_total >= 2 (got %lld)",
                (long long)vocab_total);
  return CE_OK;
}

// The smoothed target distribution: q_t on the target, q_o on every other
// column, in double; the kernels take q_o, q_t - q_o and 1 - q_t rounded once
// to FP32 (and the fused kernel's FP64 path q_o and q_t themselves).
struct Smoothing {
  double q_o, q_t;
  float f_o() const { return (float)q_o; }
  float f_to() const { return (float)(q_t - q_o); }
  float f_rest() const { return (float)(1.0 - q_t); }
};
Smoothing smoothing_of(const ce_params* p, int64_t vocab_total) {
  const double a = p->label_smoothing, V = (double)vocab_total;
  if (p->smoothing == CE_SMOOTH_OTHERS) return Smoothing{a > 0.0 ? a / (V - 1.0) : 0.0, 1.0 - a};
  return Smoothing{a / V, a / V + (1.0 - a)};
}

ce_status check_logits(const ce_logits* x, bool unsharded) {
  if (!x) return fail(CE_EINVAL, "logits descriptor is NULL");
  if (x->dtype != CE_F32 && x->dtype != CE_BF16) return fail(CE_EDTYPE, "unsupported logits dtype %d", x->dtype);
  if (x->reserved != 0) return fail(CE_EINVAL, "logits.reserved must be 0");
  if (x->d0 < 0 || x->d1 < 1) return fail(CE_EINVAL, "need d0 >= 0 and d1 >= 1 (got %lld, %lld)",
                                          (long long)x->d0, (long long)x->d1);
  if (x->v_local < 1) return fail(CE_EINVAL, "v_local must be >= 1");
  // the kernels address a row through 32-bit buffer ranges and byte offsets
  if (x->v_local > (int64_t)(0xffffffffLL / elem_bytes(x->dtype)))
    return fail(CE_ELAYOUT, "rows of %lld columns exceed 4 GiB", (long long)x->v_local);
  if (x->vocab_start < 0 || x->vocab_total < 1 || x->vocab_start > x->vocab_total - x->v_local)
    return fail(CE_ELAYOUT, "shard [%lld, %lld) does not fit a vocabulary of %lld", (long long)x->vocab_start,
                (long long)(x->vocab_start + x->v_local), (long long)x->vocab_total);
  if (unsharded && (x->vocab_start != 0 || x->v_local != x->vocab_total))
    return fail(CE_ELAYOUT, "this call needs unsharded logits (vocab_start 0, v_local == vocab_total)");
  if (x->d0 > 0 && x->d1 > INT64_MAX / x->d0) return fail(CE_EINVAL, "row count overflows");
  const int64_t N = x->d0 * x->d1;
  if (N > 0x7fffffffLL) return fail(CE_EINVAL, "more than 2^31-1 rows");
  if (N > 0 && !x->data) return fail(CE_EINVAL, "logits data is NULL");
  if (((uintptr_t)x->data) % (uintptr_t)elem_bytes(x->dtype) != 0)
    return fail(CE_ELAYOUT, "logits pointer is not aligned to its dtype");
  if (x->s0 < 0 || x->s1 < 0) return fail(CE_ELAYOUT, "negative strides are not supported");
  if (!rows_disjoint(x->d0, x->d1, x->s0, x->s1, x->v_local))
    return fail(CE_ELAYOUT, "rows overlap in memory (strides %lld, %lld with %lld columns)", (long long)x->s0,
                (long long)x->s1, (long long)x->v_local);
  return CE_OK;
}

ce_status check_targets(const ce_targets* t, int64_t N) {
  if (!t) return fail(CE_EINVAL, "targets descriptor is NULL");
  if (N > 0 && !t->data) return fail(CE_EINVAL, "targets data is NULL");
  if (((uintptr_t)t->data) % 8u != 0) return fail(CE_ELAYOUT, "targets pointer is not 8-byte aligned");
  if (t->s0 < 0 || t->s1 < 0) return fail(CE_ELAYOUT, "negative target strides are not supported");
  return CE_OK;
}

struct WsLayout {
  size_t row_loss = 0;         // offset of [N] FP32 per-row losses (ce_forward / ce_shard_combine, reduce only)
  size_t row_loss_tagged = 0;  // offset of [N] tagged per-row losses (ce_fwd_bwd_fused, reduce only)
  size_t slots = 0;            // offset of [N][K][4] tagged exchange words (ce_fwd_bwd_fused, K > 1)
  size_t total = 0;
};

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// header | FP32 per-row losses of the split calls | the fused call's tagged
// per-row losses | its split-row exchange words.  The fused call's regions
// come after everything the other calls write, so a workspace shared by
// several entry points never holds their values where the fused call looks
// for its tags.
WsLayout ws_layout(int64_t N, int32_t K, bool reduce, bool fused) {
  WsLayout w;
  size_t off = vce::kWsHeaderBytes;
  if (reduce) {
    w.row_loss = off;
    off = align256(off + (size_t)N * 4u);
  }
  if (fused) {
    w.row_loss_tagged = off;
    off = align256(off + (size_t)N * 8u);
  }
  if (fused && K > 1) {
    w.slots = off;
    off = align256(off + (size_t)N * (size_t)K * 4u * 8u);
  }
  w.total = off;
  return w;
}


// The divisor of a reduced loss: n for the mean, none (NULL) for the sum.
const int32_t* mean_n(const ce_params* p, const int32_t* n) { return p->reduce_loss == CE_REDUCE_MEAN ? n : nullptr; }

int32_t chunks_for(const ce_logits* x, const ce_params* p) {
  int32_t K = p->split_chunks > 0 ? p->split_chunks : vce::fused_auto_chunks(x->dtype, x->v_local);
  return K < 1 ? 1 : K;
}

vce::RowLayout row_layout(const ce_logits* x, const ce_targets* t, const ce_params* p) {
  vce::RowLayout L;
  L.x = static_cast<char*>(x->data);
  L.dtype = x->dtype;
  L.d1 = x->d1;
  L.s0 = x->s0;
  L.s1 = x->s1;
  L.N = x->d0 * x->d1;
  L.V = x->v_local;
  L.vocab_start = x->vocab_start;
  L.vocab_total = x->vocab_total;
  L.tgt = t->data;
  L.ts0 = t->s0;
  L.ts1 = t->s1;
  L.ignore_idx = p->ignore_idx;
  const Smoothing q = smoothing_of(p, x->vocab_total);
  L.q_o = q.f_o();
  L.q_to = q.f_to();
  L.q_rest = q.f_rest();
  return L;
}

// Whole rows of at most kShortRow columns take the streaming kernels' FP64
// path (one wave per row), with the distribution in double.
void set_short_rows(vce::StatsArgs* a, const ce_logits* x, const ce_params* p) {
  a->short_rows = x->v_local <= vce::kShortRow;
  const Smoothing q = smoothing_of(p, x->vocab_total);
  a->q_o_d = q.q_o;
  a->q_t_d = q.q_t;
  a->phase = vce::phase_buffer((size_t)(x->d0 * x->d1) * 64u);
}

// ---- profiling state (instrumentation only)
std::mutex g_prof_mu;
std::vector<hipEvent_t> g_prof_ev;  // pairs
int32_t g_prof_cap = 0, g_prof_used = 0;

void prof_next(hipEvent_t* e0, hipEvent_t* e1) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  *e0 = *e1 = nullptr;
  if (g_prof_used < g_prof_cap) {
    *e0 = g_prof_ev[2 * g_prof_used];
    *e1 = g_prof_ev[2 * g_prof_used + 1];
    ++g_prof_used;
  }
}

}  // namespace

namespace vce {
#ifdef CE_PHASE_CLOCK
namespace {
unsigned long long* g_phase = nullptr;
size_t g_phase_bytes = 0;
}  // namespace
unsigned long long* phase_buffer(size_t bytes) { return bytes <= g_phase_bytes ? g_phase : nullptr; }
#else
unsigned long long* phase_buffer(size_t) { return nullptr; }
#endif
void set_last_error(const char* msg) { snprintf(g_err, sizeof g_err, "%s", msg); }
size_t fused_workspace_bytes(int64_t N, int32_t dtype, int64_t V, bool reduce) {
  return ws_layout(N, fused_auto_chunks(dtype, V), reduce, true).total;
}
}  // namespace vce

extern "C" {

#ifdef CE_PHASE_CLOCK
// The instrumented build's one extra export (not part of ce.h): the device
// buffer that later fused and statistics calls stamp their phases into, 64
// bytes per workgroup item (fused) or row (statistics); NULL stops it.
ce_status ce_phase_clock(void* buf, size_t bytes) {
  vce::g_phase = static_cast<unsigned long long*>(buf);
  vce::g_phase_bytes = buf ? bytes : 0;
  return CE_OK;
}
#endif

int32_t ce_abi_version(void) { return CE_ABI_VERSION; }

const char* ce_last_error(void) { return g_err; }

const char* ce_status_string(ce_status s) {
  switch (s) {
    case CE_OK: return "CE_OK";
    case CE_EINVAL: return "CE_EINVAL: invalid argument";
    case CE_EDTYPE: return "CE_EDTYPE: unsupported dtype";
    case CE_ELAYOUT: return "CE_ELAYOUT: unsupported layout";
    case CE_EWORKSPACE: return "CE_EWORKSPACE: workspace missing or too small";
    case CE_EHIP: return "CE_EHIP: HIP runtime error";
    case CE_EDEADLOCK: return "CE_EDEADLOCK: split-row exchange gave up waiting";
  }
  return "unknown ce_status";
}

size_t ce_workspace_bytes(const ce_logits* x, const ce_params* p) {
  if (check_params(p) != CE_OK || check_logits(x, false) != CE_OK) return 0;
  return ws_layout(x->d0 * x->d1, chunks_for(x, p), p->reduce_loss != 0, true).total;
}

size_t ce_combine_workspace_bytes(int64_t rows, const ce_params* p) {
  if (check_params(p) != CE_OK) return 0;
  if (rows < 0 || rows > 0x7fffffffLL) {
    fail(CE_EINVAL, "rows %lld out of range", (long long)rows);
    return 0;
  }
  return ws_layout(rows, 1, p->reduce_loss != 0, false).total;
}

ce_status ce_forward_ex(const ce_logits* x, const ce_targets* t, const ce_params* p, float* loss, float* lse,
                        float* lse_aux, int32_t* n_valid, void* ws, size_t ws_bytes, hipStream_t stream) {
  ce_status st;
  if ((st = check_params(p)) || (st = check_logits(x, true)) || (st = check_smoothing(p, x->vocab_total))) return st;
  const int64_t N = x->d0 * x->d1;
  if ((st = check_targets(t, N))) return st;
  if (!loss && (N > 0 || p->reduce_loss)) return fail(CE_EINVAL, "loss is NULL");
  if (((uintptr_t)lse_aux) % 8u) return fail(CE_ELAYOUT, "lse_aux must be 8-byte aligned");
  const WsLayout w = ws_layout(N, 1, p->reduce_loss != 0, false);
  if (!ws || ws_bytes < w.total)
    return fail(CE_EWORKSPACE, "workspace of %zu bytes needed, %zu given", w.total, ws ? ws_bytes : (size_t)0);
  if (((uintptr_t)ws) % 256u) return fail(CE_EWORKSPACE, "workspace must be 256-byte aligned");

  char* wsb = static_cast<char*>(ws);
  auto* hdr = reinterpret_cast<vce::WsHeader*>(wsb);
  int32_t* n_out = n_valid ? n_valid : &hdr->n_valid;
  hipError_t e;
  if (N == 0) {  // nothing to read: n = 0, and the mean of no rows is 0/0
    if ((e = vce::launch_zero_count(n_out, stream))) return hip_fail(e, "count launch");
    if (p->reduce_loss && (e = vce::launch_mean(nullptr, 0, mean_n(p, n_out), loss, stream)))
      return hip_fail(e, "mean launch");
    return CE_OK;
  }
  vce::StatsArgs a;
  a.L = row_layout(x, t, p);
  a.mode = vce::kStatsForward;
  a.row_loss = p->reduce_loss ? reinterpret_cast<float*>(wsb + w.row_loss) : loss;
  a.lse = lse;
  a.lse_aux = lse_aux;
  a.stats = nullptr;
  a.n_out = n_out;  // counted by the stats kernel's workgroup 0
  set_short_rows(&a, x, p);
  hipEvent_t e0, e1;
  prof_next(&e0, &e1);
  if ((e = vce::launch_stats(a, stream, e0, e1))) return hip_fail(e, "forward launch");
  if (p->reduce_loss && (e = vce::launch_mean(a.row_loss, N, mean_n(p, n_out), loss, stream)))
    return hip_fail(e, "mean launch");
  return CE_OK;
}

ce_status ce_forward(const ce_logits* x, const ce_targets* t, const ce_params* p, float* loss, float* lse,
                     int32_t* n_valid, void* ws, size_t ws_bytes, hipStream_t stream) {
  return ce_forward_ex(x, t, p, loss, lse, nullptr, n_valid, ws, ws_bytes, stream);
}

ce_status ce_backward_inplace_ex(const ce_logits* x, const ce_targets* t, const ce_params* p, const float* lse,
                                 const float* lse_aux, const float* grad_out, const int32_t* n_valid,
                                 hipStream_t stream) {
  ce_status st;
  if ((st = check_params(p)) || (st = check_logits(x, false)) || (st = check_smoothing(p, x->vocab_total))) return st;
  const int64_t N = x->d0 * x->d1;
  if ((st = check_targets(t, N))) return st;
  if (N > 0 && !lse) return fail(CE_EINVAL, "lse is NULL");
  if (((uintptr_t)lse_aux) % 8u) return fail(CE_ELAYOUT, "lse_aux must be 8-byte aligned");
  if (p->reduce_loss == CE_REDUCE_MEAN && !n_valid) return fail(CE_EINVAL, "the mean (CE_REDUCE_MEAN) needs n_valid");
  vce::BackwardArgs a;
  a.L = row_layout(x, t, p);
  a.lse = lse;
  a.lse_aux = lse_aux;
  a.reduce = p->reduce_loss;
  a.g = grad_out;
  a.n_valid = n_valid;
  // short rows go to one wave in FP64: whole rows are recomputed from the
  // logits, shard rows of a short vocabulary use the handed-over lse
  a.short_rows = x->vocab_total > vce::kShortRow ? vce::kShortNone
                 : x->v_local == x->vocab_total  ? vce::kShortRecompute
                                                 : vce::kShortFromLse;
  const Smoothing q = smoothing_of(p, x->vocab_total);
  a.q_o_d = q.q_o;
  a.q_t_d = q.q_t;
  hipEvent_t e0, e1;
  prof_next(&e0, &e1);
  hipError_t e;
  if ((e = vce::launch_backward(a, stream, e0, e1))) return hip_fail(e, "backward launch");
  return CE_OK;
}

ce_status ce_backward_inplace(const ce_logits* x, const ce_targets* t, const ce_params* p, const float* lse,
                              const float* grad_out, const int32_t* n_valid, hipStream_t stream) {
  return ce_backward_inplace_ex(x, t, p, lse, nullptr, grad_out, n_valid, stream);
}

}  // extern "C"

namespace vce {
// Every check of ce_fwd_bwd_fused that depends on the logits' shape and the
// parameters (not on the buffers), and the plan it leads to.
ce_status fused_plan(const ce_logits* x, const ce_params* p, int32_t* K_out, int64_t* C_out, FusedShape* shape_out) {
  ce_status st;
  if ((st = check_params(p)) || (st = check_logits(x, true)) || (st = check_smoothing(p, x->vocab_total))) return st;
  const int64_t N = x->d0 * x->d1;
  const int32_t K = chunks_for(x, p);
  if (K > kMaxChunks)
    return fail(CE_ELAYOUT, "rows of %lld columns need %d chunks (at most %lld)", (long long)x->v_local, K,
                (long long)kMaxChunks);
  const int64_t nvmax = vce::max_body_vecs(x->dtype, x->v_local);
  const int64_t C = (nvmax + K - 1) / K;
  const vce::FusedShape shape = vce::fused_shape_for(C);
  if (shape.threads == 0)
    return fail(CE_ELAYOUT, "split_chunks %d leaves %lld vectors per chunk, above one workgroup's %d",
                p->split_chunks, (long long)C, 1024 * 16);
  if (N * K > kMaxGrid) return fail(CE_EINVAL, "rows x chunks exceeds the launch grid");
  if (K_out) *K_out = K;
  if (C_out) *C_out = C;
  if (shape_out) *shape_out = shape;
  return CE_OK;
}
}  // namespace vce

namespace {

// What both fused launches share: the targets, loss and workspace checks,
// the workspace regions, the target slices counted by the first workgroups,
// and the smoothing in double.  With no rows it writes n = 0 (and the mean
// or sum of nothing) itself and sets *launch = false.  L0 is the layout of
// the logits (the first shard for the shard call); K the chunks per row.
ce_status fused_common(const ce_logits* L0, const ce_targets* t, const ce_params* p, int32_t K, int64_t C,
                       const float* grad_out, float* loss, int32_t* n_valid, void* ws, size_t ws_bytes,
                       hipStream_t stream, vce::FusedArgs* a, bool* launch) {
  ce_status st;
  *launch = false;
  const int64_t N = L0->d0 * L0->d1;
  if ((st = check_targets(t, N))) return st;
  if (!loss && (N > 0 || p->reduce_loss)) return fail(CE_EINVAL, "loss is NULL");
  const WsLayout w = ws_layout(N, K, p->reduce_loss != 0, true);
  if (!ws || ws_bytes < w.total)
    return fail(CE_EWORKSPACE, "workspace of %zu bytes needed, %zu given", w.total, ws ? ws_bytes : (size_t)0);
  if (((uintptr_t)ws) % 256u) return fail(CE_EWORKSPACE, "workspace must be 256-byte aligned");

  char* wsb = static_cast<char*>(ws);
  auto* hdr = reinterpret_cast<vce::WsHeader*>(wsb);
  hipError_t e;
  if (N == 0) {  // nothing to read: n = 0, and the mean of no rows is 0/0
    int32_t* n_out = n_valid ? n_valid : &hdr->n_valid;
    if ((e = vce::launch_zero_count(n_out, stream))) return hip_fail(e, "count launch");
    if (p->reduce_loss && (e = vce::launch_mean(nullptr, 0, mean_n(p, n_out), loss, stream)))
      return hip_fail(e, "mean launch");
    return CE_OK;
  }
  a->L = row_layout(L0, t, p);
  a->K = K;
  a->aligned = 0;
  a->C = C;
  a->reduce = p->reduce_loss;
  a->g = grad_out;
  a->n_out = n_valid;
  a->row_loss = p->reduce_loss ? nullptr : loss;
  a->row_loss_tagged = reinterpret_cast<unsigned long long*>(wsb + w.row_loss_tagged);
  a->mean_out = p->reduce_loss ? loss : nullptr;
  a->hdr = hdr;
  a->slots = K > 1 ? reinterpret_cast<unsigned long long*>(wsb + w.slots) : nullptr;
  // at most kMaxSlices target slices of at least 2048 rows, counted by the first workgroups
  a->slice_rows = (N + vce::kMaxSlices - 1) / vce::kMaxSlices;
  if (a->slice_rows < 2048) a->slice_rows = 2048;
  a->nslice = (int32_t)((N + a->slice_rows - 1) / a->slice_rows);
  a->ws_bytes = w.total;
  a->short_rows = 0;
  const Smoothing q = smoothing_of(p, L0->vocab_total);
  a->q_o_d = q.q_o;
  a->q_t_d = q.q_t;
  a->phase = vce::phase_buffer((size_t)N * (size_t)K * 64u);
  *launch = true;
  return CE_OK;
}

ce_status fused_call(const ce_logits* x, const ce_targets* t, const ce_params* p, const float* grad_out,
                     float* loss, int32_t* n_valid, void* ws, size_t ws_bytes, hipStream_t stream) {
  ce_status st;
  int32_t K = 0;
  int64_t C = 0;
  vce::FusedShape shape{0, 0};
  if ((st = vce::fused_plan(x, p, &K, &C, &shape))) return st;
  vce::FusedArgs a;
  bool launch;
  if ((st = fused_common(x, t, p, K, C, grad_out, loss, n_valid, ws, ws_bytes, stream, &a, &launch)) || !launch)
    return st;
  a.aligned = rows_aligned16(x);
  // short whole rows take the FP64 path of the 256 x 1 kernel (its only shape for them)
  a.short_rows = x->v_local <= vce::kShortRow && K == 1;
  if (a.short_rows && (shape.threads != 256 || shape.vecs != 1))
    return fail(CE_ELAYOUT, "internal: rows of %lld columns planned on a %d x %d workgroup", (long long)x->v_local,
                shape.threads, shape.vecs);
  hipEvent_t e0, e1;
  prof_next(&e0, &e1);
  hipError_t e;
  if ((e = vce::launch_fused(a, shape, stream, e0, e1))) return hip_fail(e, "fused launch");
  return CE_OK;
}

}  // namespace

extern "C" {

ce_status ce_fwd_bwd_fused(const ce_logits* x, const ce_targets* t, const ce_params* p, const float* grad_out,
                           float* loss, int32_t* n_valid, void* ws, size_t ws_bytes, hipStream_t stream) {
  return fused_call(x, t, p, grad_out, loss, n_valid, ws, ws_bytes, stream);
}

ce_status ce_fwd_bwd_fused_noalloc(const ce_logits* x, const ce_targets* t, const ce_params* p,
                                   const float* grad_out, float* loss, int32_t* n_valid, hipStream_t stream) {
  ce_status st;
  int32_t K = 0;
  if ((st = vce::fused_plan(x, p, &K, nullptr, nullptr))) return st;
  const size_t need = ws_layout(x->d0 * x->d1, K, p->reduce_loss != 0, true).total;
  if (need > vce::kStaticScratchBytes)
    return fail(CE_EWORKSPACE,
                "this call needs %zu bytes of workspace; the allocation-free call holds %zu (use ce_fwd_bwd_fused "
                "with a workspace of ce_workspace_bytes)",
                need, vce::kStaticScratchBytes);
  void* ws = nullptr;
  hipError_t e;
  if ((e = vce::static_scratch(stream, &ws)))
    return e == hipErrorStreamCaptureUnsupported
               ? fail(CE_EINVAL, "the first ce_fwd_bwd_fused_noalloc call on a device prepares its scratch and "
                                 "must not be captured")
               : hip_fail(e, "static scratch");
  return fused_call(x, t, p, grad_out, loss, n_valid, ws, vce::kStaticScratchBytes, stream);
}

namespace {

// The shard set's checks and plan: S shards of one row set (same dtype,
// rows and vocabulary) that tile [0, vocab_total) in order; each shard row
// is cut into kper chunks of at most 4096 vectors.
struct ShardPlan {
  int32_t kper = 0, K = 0;
  int64_t C = 0;
  vce::FusedShape shape{0, 0};
  bool short_rows = false;  // a vocabulary of at most kShortRow columns: one wave per row, FP64
};

ce_status shard_plan(const ce_logits* shards, int32_t S, const ce_params* p, ShardPlan* out) {
  ce_status st;
  if ((st = check_params(p))) return st;
  if (!shards) return fail(CE_EINVAL, "shards is NULL");
  if (S < 1 || S > vce::kMaxShards) return fail(CE_EINVAL, "S = %d outside [1, %d]", S, vce::kMaxShards);
  if (p->split_chunks != 0) return fail(CE_EINVAL, "split_chunks must be 0 for sharded logits");
  int64_t nv_max = 0, next = 0;
  for (int32_t s = 0; s < S; ++s) {
    const ce_logits* x = &shards[s];
    if ((st = check_logits(x, false))) return fail(st, "shard %d: %s", s, ce_last_error());
    if (x->dtype != shards[0].dtype || x->d0 != shards[0].d0 || x->d1 != shards[0].d1 ||
        x->vocab_total != shards[0].vocab_total)
      return fail(CE_ELAYOUT, "shard %d: dtype, rows and vocab_total must match shard 0", s);
    if (x->vocab_start != next)
      return fail(CE_ELAYOUT, "shard %d starts at column %lld, expected %lld (shards tile the vocabulary in order)",
                  s, (long long)x->vocab_start, (long long)next);
    next += x->v_local;
    const int64_t nv = vce::max_body_vecs(x->dtype, x->v_local);
    if (nv > nv_max) nv_max = nv;
  }
  if (next != shards[0].vocab_total)
    return fail(CE_ELAYOUT, "shards cover %lld of %lld columns", (long long)next, (long long)shards[0].vocab_total);
  if ((st = check_smoothing(p, shards[0].vocab_total))) return st;
  ShardPlan pl;
  pl.kper = (int32_t)((nv_max + 4095) / 4096);
  if (pl.kper < 1) pl.kper = 1;
  pl.K = S * pl.kper;
  if (pl.K > kMaxChunks)
    return fail(CE_ELAYOUT, "%d shards of up to %lld vectors need %d chunks per row (at most %lld)", S,
                (long long)nv_max, pl.K, (long long)kMaxChunks);
  pl.C = (nv_max + pl.kper - 1) / pl.kper;
  if (pl.C < 1) pl.C = 1;
  pl.shape = vce::fused_shape_for(pl.C);
  if (pl.shape.threads == 1024 || pl.shape.vecs == 16) pl.shape = vce::FusedShape{512, 8};  // C <= 4096 here
  if (shards[0].vocab_total <= vce::kShortRow) {
    // FP32 cannot hold s (p - q) where p sits close to a large q (few columns,
    // heavy smoothing): the whole row goes to one wave, which gathers its
    // columns from the shards and works in FP64, as unsharded short rows do
    pl.short_rows = true;
    pl.kper = pl.K = 1;
    pl.C = 1;
    pl.shape = vce::FusedShape{256, 1};
  }
  const int64_t N = shards[0].d0 * shards[0].d1;
  if (N * pl.K > kMaxGrid) return fail(CE_EINVAL, "rows x chunks exceeds the launch grid");
  *out = pl;
  return CE_OK;
}

}  // namespace

size_t ce_shards_workspace_bytes(const ce_logits* shards, int32_t S, const ce_params* p) {
  ShardPlan pl;
  if (shard_plan(shards, S, p, &pl)) return 0;
  return ws_layout(shards[0].d0 * shards[0].d1, pl.K, p->reduce_loss != 0, true).total;
}

ce_status ce_shards_fwd_bwd_fused(const ce_logits* shards, int32_t S, const ce_targets* t, const ce_params* p,
                                  const float* grad_out, float* loss, int32_t* n_valid, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  ce_status st;
  ShardPlan pl;
  if ((st = shard_plan(shards, S, p, &pl))) return st;
  vce::FusedArgs a;
  bool launch;
  if ((st = fused_common(&shards[0], t, p, pl.K, pl.C, grad_out, loss, n_valid, ws, ws_bytes, stream, &a,
                         &launch)) || !launch)
    return st;
  vce::ShardSet ss;
  memset(&ss, 0, sizeof ss);
  ss.S = S;
  ss.kper = pl.kper;
  for (int32_t s = 0; s < S; ++s) ss.L[s] = row_layout(&shards[s], t, p);
  a.short_rows = pl.short_rows ? 1 : 0;
  hipEvent_t e0, e1;
  prof_next(&e0, &e1);
  hipError_t e;
  if ((e = vce::launch_fused_shards(a, ss, pl.shape, stream, e0, e1))) return hip_fail(e, "sharded fused launch");
  return CE_OK;
}

ce_status ce_scale_grad_inplace(const ce_logits* x, const float* grad_out, int32_t per_row, hipStream_t stream) {
  ce_status st;
  if ((st = check_logits(x, false))) return st;
  const int64_t N = x->d0 * x->d1;
  if (N > 0 && !grad_out) return fail(CE_EINVAL, "grad_out is NULL");
  if (per_row != 0 && per_row != 1) return fail(CE_EINVAL, "per_row must be 0 or 1");
  vce::ScaleArgs a;
  a.L.x = static_cast<char*>(x->data);
  a.L.dtype = x->dtype;
  a.L.d1 = x->d1;
  a.L.s0 = x->s0;
  a.L.s1 = x->s1;
  a.L.N = N;
  a.L.V = x->v_local;
  a.L.vocab_start = x->vocab_start;
  a.L.vocab_total = x->vocab_total;
  a.L.tgt = nullptr;
  a.L.ts0 = a.L.ts1 = 0;
  a.L.ignore_idx = 0;
  a.L.q_o = a.L.q_to = a.L.q_rest = 0.f;
  a.g = grad_out;
  a.per_row = per_row;
  hipEvent_t e0, e1;
  prof_next(&e0, &e1);
  hipError_t e;
  if ((e = vce::launch_scale(a, stream, e0, e1))) return hip_fail(e, "scale launch");
  return CE_OK;
}

ce_status ce_stream_reference(const void* src, void* dst, int64_t bytes, hipStream_t stream) {
  if (bytes < 0 || bytes % 16 != 0) return fail(CE_EINVAL, "bytes must be a non-negative multiple of 16");
  if (bytes == 0) return CE_OK;
  if (!src || !dst) return fail(CE_EINVAL, "src or dst is NULL");
  if (((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u)) return fail(CE_EINVAL, "src and dst must be 16-byte aligned");
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
  if (s0 != d0 && s0 < d0 + (uintptr_t)bytes && d0 < s0 + (uintptr_t)bytes)
    return fail(CE_EINVAL, "src and dst overlap without being the same buffer");
  hipEvent_t e0, e1;
  prof_next(&e0, &e1);
  hipError_t e;
  if ((e = vce::launch_stream_ref(src, dst, bytes, s0 == d0 ? 0x80008000u : 0u, stream, e0, e1)))
    return hip_fail(e, "reference stream launch");
  return CE_OK;
}

ce_status ce_shard_partial_stats(const ce_logits* shard, const ce_targets* t, const ce_params* p, float* stats,
                                 hipStream_t stream) {
  ce_status st;
  if ((st = check_params(p)) || (st = check_logits(shard, false))) return st;
  const int64_t N = shard->d0 * shard->d1;
  if ((st = check_targets(t, N))) return st;
  if (N > 0 && !stats) return fail(CE_EINVAL, "stats is NULL");
  if (((uintptr_t)stats) % 16u) return fail(CE_ELAYOUT, "stats must be 16-byte aligned");
  vce::StatsArgs a;
  a.L = row_layout(shard, t, p);
  a.mode = vce::kStatsShard;
  a.row_loss = nullptr;
  a.lse = nullptr;
  a.lse_aux = nullptr;
  a.stats = stats;
  a.n_out = nullptr;
  set_short_rows(&a, shard, p);
  hipEvent_t e0, e1;
  prof_next(&e0, &e1);
  hipError_t e;
  if ((e = vce::launch_stats(a, stream, e0, e1))) return hip_fail(e, "shard stats launch");
  return CE_OK;
}

ce_status ce_shard_combine_ex(const float* stats, int32_t S, int64_t d0, int64_t d1, int64_t vocab_total,
                              const ce_targets* t, const ce_params* p, float* loss, float* lse, float* lse_aux,
                              int32_t* n_valid, void* ws, size_t ws_bytes, hipStream_t stream) {
  ce_status st;
  if (((uintptr_t)lse_aux) % 8u) return fail(CE_ELAYOUT, "lse_aux must be 8-byte aligned");
  if ((st = check_params(p))) return st;
  if (S < 1) return fail(CE_EINVAL, "S must be >= 1");
  if (d0 < 0 || d1 < 1) return fail(CE_EINVAL, "need d0 >= 0 and d1 >= 1");
  if (vocab_total < 1) return fail(CE_EINVAL, "vocab_total must be >= 1");
  if ((st = check_smoothing(p, vocab_total))) return st;
  if (d0 > 0 && d1 > 0x7fffffffLL / d0) return fail(CE_EINVAL, "more than 2^31-1 rows");
  const int64_t N = d0 * d1;
  if ((st = check_targets(t, N))) return st;
  if (N > 0 && !stats) return fail(CE_EINVAL, "stats is NULL");
  if (((uintptr_t)stats) % 16u) return fail(CE_ELAYOUT, "stats must be 16-byte aligned");
  if (!loss && (N > 0 || p->reduce_loss)) return fail(CE_EINVAL, "loss is NULL");
  const WsLayout w = ws_layout(N, 1, p->reduce_loss != 0, false);
  if (!ws || ws_bytes < w.total)
    return fail(CE_EWORKSPACE, "workspace of %zu bytes needed, %zu given", w.total, ws ? ws_bytes : (size_t)0);
  if (((uintptr_t)ws) % 256u) return fail(CE_EWORKSPACE, "workspace must be 256-byte aligned");

  char* wsb = static_cast<char*>(ws);
  auto* hdr = reinterpret_cast<vce::WsHeader*>(wsb);
  int32_t* n_out = n_valid ? n_valid : &hdr->n_valid;
  hipError_t e;
  if (N == 0) {  // nothing to combine: n = 0, and the mean of no rows is 0/0
    if ((e = vce::launch_zero_count(n_out, stream))) return hip_fail(e, "count launch");
    if (p->reduce_loss && (e = vce::launch_mean(nullptr, 0, mean_n(p, n_out), loss, stream)))
      return hip_fail(e, "mean launch");
    return CE_OK;
  }
  vce::CombineArgs a;
  a.stats = stats;
  a.S = S;
  a.N = N;
  a.d1 = d1;
  a.vocab_total = vocab_total;
  a.tgt = t->data;
  a.ts0 = t->s0;
  a.ts1 = t->s1;
  a.ignore_idx = p->ignore_idx;
  const Smoothing q = smoothing_of(p, vocab_total);
  a.q_o_d = q.q_o;
  a.q_t_d = q.q_t;
  a.row_loss = p->reduce_loss ? reinterpret_cast<float*>(wsb + w.row_loss) : loss;
  a.lse = lse;
  a.lse_aux = lse_aux;
  a.n_out = n_out;  // counted by the combine kernel's workgroup 0
  if ((e = vce::launch_combine(a, stream))) return hip_fail(e, "combine launch");
  if (p->reduce_loss && (e = vce::launch_mean(a.row_loss, N, mean_n(p, n_out), loss, stream)))
    return hip_fail(e, "mean launch");
  return CE_OK;
}

ce_status ce_shard_combine(const float* stats, int32_t S, int64_t d0, int64_t d1, int64_t vocab_total,
                           const ce_targets* t, const ce_params* p, float* loss, float* lse, int32_t* n_valid,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
  return ce_shard_combine_ex(stats, S, d0, d1, vocab_total, t, p, loss, lse, nullptr, n_valid, ws, ws_bytes, stream);
}

ce_status ce_workspace_init(void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!ws) return fail(CE_EINVAL, "workspace is NULL");
  if (((uintptr_t)ws) % 256u) return fail(CE_EWORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < vce::kWsHeaderBytes || ws_bytes % 8u)
    return fail(CE_EWORKSPACE, "workspace of %zu bytes: need a multiple of 8, at least %zu", ws_bytes,
                vce::kWsHeaderBytes);
  hipError_t e;
  if ((e = vce::launch_ws_init(ws, ws_bytes, stream))) return hip_fail(e, "workspace init launch");
  return CE_OK;
}

ce_status ce_workspace_check(void* ws, hipStream_t stream) {
  if (!ws) return fail(CE_EINVAL, "workspace is NULL");
  hipError_t e;
  if ((e = hipStreamSynchronize(stream))) return hip_fail(e, "stream synchronize");
  vce::WsHeader h;
  if ((e = hipMemcpy(&h, ws, sizeof h, hipMemcpyDeviceToHost))) return hip_fail(e, "workspace read");
  if (!h.status) return CE_OK;
  const uint32_t zero = 0;
  if ((e = hipMemcpy(ws, &zero, sizeof zero, hipMemcpyHostToDevice))) return hip_fail(e, "workspace status clear");
  if (h.status & 2u) return fail(CE_EWORKSPACE, "ce_fwd_bwd_fused ran on a workspace that ce_workspace_init has not prepared (or prepared smaller)");
  return fail(CE_EDEADLOCK, "a split row gave up waiting for its partner chunks");
}

ce_status ce_profile_start(int32_t capacity) {
  if (capacity < 1 || capacity > (1 << 20)) return fail(CE_EINVAL, "capacity out of range");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (g_prof_cap) return fail(CE_EINVAL, "profiling already started");
  g_prof_ev.assign(2 * (size_t)capacity, nullptr);
  for (auto& ev : g_prof_ev) {
    hipError_t e = hipEventCreate(&ev);
    if (e) {
      for (auto& x : g_prof_ev)
        if (x) (void)hipEventDestroy(x);
      g_prof_ev.clear();
      return hip_fail(e, "event create");
    }
  }
  g_prof_cap = capacity;
  g_prof_used = 0;
  return CE_OK;
}

ce_status ce_profile_stop(float* ms, int32_t cap, int32_t* count) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_cap) return fail(CE_EINVAL, "profiling was not started");
  ce_status st = CE_OK;
  int32_t n = 0;
  for (int32_t i = 0; i < g_prof_used; ++i) {
    hipError_t e = hipEventSynchronize(g_prof_ev[2 * i + 1]);
    float v = 0.f;
    if (!e) e = hipEventElapsedTime(&v, g_prof_ev[2 * i], g_prof_ev[2 * i + 1]);
    if (e && st == CE_OK) st = hip_fail(e, "event elapsed time");
    if (ms && n < cap) ms[n++] = v;
  }
  for (auto& ev : g_prof_ev) (void)hipEventDestroy(ev);
  g_prof_ev.clear();
  g_prof_cap = g_prof_used = 0;
  if (count) *count = n;
  return st;
}

}  // extern "C"
