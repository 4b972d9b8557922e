// Internal interface between the C ABI layer (ce_api.cpp) and the gfx950
// kernels (ce_kernels.hip).  Host-side only types; no torch, no allocation.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "ce.h"

namespace vce {

// Workspace header (first 256 bytes of every workspace).
constexpr int kMaxSlices = 16;
struct WsHeader {
  uint32_t status;                 // bit 0: a wait gave up; bit 1: the workspace was not initialised
  int32_t n_valid;                 // count of non-ignored rows when the caller passed no n_valid
  unsigned long long magic;        // kWsMagic once ce_workspace_init has run
  unsigned long long init_bytes;   // bytes ce_workspace_init cleared
  unsigned long long epoch;        // fused call: its low 32 bits tag the call's words (1 after init, never 0)
  // Test hook, never set by the library (ce_workspace_init zeroes it): when
  // it equals (row + 1) << 8 | chunk, that chunk of that split row leaves its
  // exchange words unpublished, so its partners' bounded waits give up.
  unsigned long long withhold;
  unsigned long long reserved[11];
  unsigned long long counts[kMaxSlices];  // fused call: tagged counts of non-ignored rows per target slice
};
constexpr size_t kWsHeaderBytes = 256;
static_assert(sizeof(WsHeader) == kWsHeaderBytes, "workspace header is 256 bytes");
// k_ws_init writes the header by word index: 1 = magic, 2 = init_bytes, 3 = epoch
static_assert(offsetof(WsHeader, magic) == 8 && offsetof(WsHeader, init_bytes) == 16, "header word layout");
static_assert(offsetof(WsHeader, epoch) == 24 && offsetof(WsHeader, counts) == 128, "header word layout");
static_assert(offsetof(WsHeader, withhold) == 32, "header word layout: the fused kernel reads it after the epoch");
constexpr unsigned long long kWsMagic = 0x43452d5753304331ull;

// Which template instance of the fused kernel a plan uses.
struct FusedShape {
  int threads;      // workgroup size T
  int vecs;         // 16-byte vectors held per thread P
};

struct RowLayout {
  char* x;                 // logits base (element (0,0,0))
  int32_t dtype;           // CE_F32 / CE_BF16
  int64_t d1, s0, s1;      // logical dim and element strides
  int64_t N;               // rows
  int64_t V;               // columns in this buffer (v_local)
  int64_t vocab_start, vocab_total;
  const int64_t* tgt;
  int64_t ts0, ts1;
  int64_t ignore_idx;
  // the smoothed target distribution: q_t at the target, q_o at every other column
  float q_o;               // a / V, or a / (V - 1)
  float q_to;              // q_t - q_o, the target logit's weight in the loss beyond q_o
  float q_rest;            // 1 - q_t: the target's gradient is s (q_rest - (1 - p_t))
};

struct FusedArgs {
  RowLayout L;
  int32_t K;               // chunks per row
  int32_t aligned;         // every row starts and ends on a 16-byte boundary (no head/tail)
  int64_t C;               // body vectors per chunk
  int32_t reduce;          // CE_REDUCE_NONE / MEAN (over non-ignored rows) / SUM
  const float* g;          // upstream gradient ([N] or [1]); NULL = 1
  int32_t* n_out;          // [1] count of non-ignored rows (nullable), written by the last item's workgroup
  float* row_loss;         // [N] loss output (no reduction)
  unsigned long long* row_loss_tagged;  // [N] tagged per-row losses (workspace; every mode)
  float* mean_out;         // [1] mean or sum of the losses, written by the workgroup of the last item
  WsHeader* hdr;
  unsigned long long* slots;  // [N][K][4] tagged exchange words (K > 1)
  int64_t slice_rows;      // rows per target slice; workgroup b < nslice counts slice b
  unsigned long long ws_bytes;  // workspace bytes this call uses (checked against the initialised size)
  int32_t nslice;
  // rows of at most kShortRow columns held whole (K = 1): statistics and
  // gradient in FP64 by one wave, with the distribution in double
  int32_t short_rows;
  double q_o_d, q_t_d;     // q_o and q_t
  unsigned long long* phase;  // [items][8] phase stamps (the instrumented build; NULL otherwise)
};
// Longest row the FP64 whole-row paths take (two columns per lane of a wave).
constexpr int64_t kShortRow = 128;

// The vocabulary shards of ce_shards_fwd_bwd_fused (a kernel argument):
// shard s's layout (buffer, strides, v_local, vocab_start); each shard row is
// cut into kper chunks, so a row has K = S * kper chunks.
constexpr int kMaxShards = 16;
struct ShardSet {
  int32_t S;
  int32_t kper;
  RowLayout L[kMaxShards];
};

enum StatsMode { kStatsForward = 0, kStatsShard = 1 };

struct StatsArgs {
  RowLayout L;
  int32_t mode;
  float* row_loss;  // forward: loss [N] or per-row scratch
  float* lse;       // forward: may be NULL
  float* lse_aux;   // forward: [N][2] (lse residual, 1 - p_t) or NULL
  float* stats;     // shard: [N][4]
  int32_t* n_out;   // forward: [1] count of non-ignored rows, written by workgroup 0 (may be NULL)
  // rows of at most kShortRow columns: one wave in FP64, the distribution in double
  int32_t short_rows;
  double q_o_d, q_t_d;
  unsigned long long* phase;  // [rows][8] phase stamps (the instrumented build; NULL otherwise)
};

struct BackwardArgs {
  RowLayout L;
  int32_t K;               // items per row: batches of T x PB vectors, one a workgroup (set by the launcher)
  const float* lse;
  const float* lse_aux;    // [N][2] (lse residual, 1 - p_t) or NULL: the lse alone
  int32_t reduce;          // CE_REDUCE_*
  const float* g;
  const int32_t* n_valid;  // read with CE_REDUCE_MEAN only
  // rows of at most kShortRow columns, one wave in FP64 (kShortRecompute:
  // unsharded rows recomputed whole; kShortFromLse: shard rows of a vocabulary
  // of at most kShortRow columns, from the handed-over lse)
  int32_t short_rows;
  double q_o_d, q_t_d;
};
enum { kShortNone = 0, kShortRecompute = 1, kShortFromLse = 2 };

struct ScaleArgs {
  RowLayout L;             // logits holding a staged gradient (targets unused)
  const float* g;          // [N] (per_row) or [1]
  int32_t per_row;
};

struct CombineArgs {
  const float* stats;
  int32_t S;
  int64_t N, d1, vocab_total;
  const int64_t* tgt;
  int64_t ts0, ts1, ignore_idx;
  double q_o_d, q_t_d;     // q_o and q_t (the loss is formed in FP64 and rounded once)
  float* row_loss;
  float* lse;
  float* lse_aux;   // [N][2] (lse residual, 1 - p_t) or NULL
  int32_t* n_out;   // [1] count of non-ignored rows, written by workgroup 0 (may be NULL)
};

// The allocation-free fused call's workspace: a file-scope device array of
// this many bytes in ce_kernels.hip, one per device, held until the process ends.
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
constexpr int kMaxDevices = 64;
// The device address of that array on the device of `stream` (NULL: the
// current device), looked up once per device with that device current; the
// first call on a device also enqueues the array's preparation (a fill
// kernel) on `stream`, and refuses a stream that is being captured.
hipError_t static_scratch(hipStream_t stream, void** out);

// Shape choice for the fused kernel (host side, no HIP calls).
FusedShape fused_shape_for(int64_t body_vecs_per_chunk);
int64_t max_body_vecs(int32_t dtype, int64_t V);
int32_t fused_auto_chunks(int32_t dtype, int64_t V);

// Launchers: enqueue on `stream`, return the hipError_t of the launch.
// n_out[0] = 0 (calls on no rows)
hipError_t launch_zero_count(int32_t* n_out, hipStream_t stream);
hipError_t launch_fused(const FusedArgs& a, FusedShape shape, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
// shapes 512 x 8 and 256 x {1, 2, 4, 8} only
hipError_t launch_fused_shards(const FusedArgs& a, const ShardSet& ss, FusedShape shape, hipStream_t stream,
                               hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_stats(const StatsArgs& a, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_backward(const BackwardArgs& a, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_combine(const CombineArgs& a, hipStream_t stream);
// out[0] = sum of row_loss / n_valid[0], or the plain sum when n_valid is NULL
hipError_t launch_mean(const float* row_loss, int64_t N, const int32_t* n_valid, float* out, hipStream_t stream);
hipError_t launch_ws_init(void* ws, size_t bytes, hipStream_t stream);
hipError_t launch_scale(const ScaleArgs& a, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_stream_ref(const void* src, void* dst, int64_t bytes, uint32_t flip, hipStream_t stream,
                             hipEvent_t ev0, hipEvent_t ev1);
// chunked linear + cross-entropy: n over all N rows (row r's target at tgt[r * ts]) into n_out, and
// with the mean scale[0] = g / n; then loss[0] = sum of parts (index order, FP64), / n for the mean
hipError_t launch_linear_prep(const int64_t* tgt, int64_t ts, int64_t N, int64_t ignore_idx, int32_t reduce,
                              const float* g, int32_t* n_out, float* scale, hipStream_t stream);
hipError_t launch_linear_finish(const float* parts, int64_t nparts, int32_t reduce, const int32_t* n, float* out,
                                hipStream_t stream);
// zeros in rows x cols of an FP32 matrix with row stride ld
hipError_t launch_fill_f32(float* p, int64_t rows, int64_t cols, int64_t ld, hipStream_t stream);

// One BF16 product on the library's MFMA kernel (ce_gemm.hip), FP32 accumulation:
//   C[M][N] (+)= sum_k A(m, k) B(n, k)
// A is [M][K] (a_kc: K contiguous) or [K][M]; B is [N][K] (b_kc) or [K][N]; leading dimensions in elements.
// out 0: C BF16, written; 1: C FP32, written; 2: C FP32, added to.  The layouts of the chunked head's three
// products are supported: (a_kc, b_kc, out) = (1, 1, 0) logits, (1, 0, 0) dh, (0, 0, 1 or 2) dW.
struct GemmBf16 {
  const void* A;
  int64_t lda;
  bool a_kc;
  const void* B;
  int64_t ldb;
  bool b_kc;
  void* C;
  int64_t ldc;
  int out;
  int M, N, K;
  // optional device scratch (16-byte aligned): a BF16 product whose output tiles would leave most compute
  // units idle splits its K range over FP32 partial planes here, summed in a fixed order afterwards
  void* scratch = nullptr;
  size_t scratch_bytes = 0;
};
// Whether launch_gemm_bf16 takes g: M, N, K >= 1; lda and ldb multiples of 8 and at least the contiguous
// extent; A and B 16-byte aligned (so no 16-byte chunk straddles a row's end); one of the head's layouts.
bool gemm_bf16_supported(const GemmBf16& g);
hipError_t launch_gemm_bf16(const GemmBf16& g, hipStream_t stream);

// The instrumented build's phase-stamp buffer when it holds `bytes`, else NULL
// (always NULL in the normal build).
unsigned long long* phase_buffer(size_t bytes);

// Shared by the entry points (ce_api.cpp): the calling thread's error detail,
// and the fused call's workspace need for N whole rows of V columns.
void set_last_error(const char* msg);
size_t fused_workspace_bytes(int64_t N, int32_t dtype, int64_t V, bool reduce);
// every check of ce_fwd_bwd_fused that depends on the logits' shape and the
// parameters (none on buffers), and the plan: chunks per row K, body vectors
// per chunk C, workgroup shape
ce_status fused_plan(const ce_logits* x, const ce_params* p, int32_t* K, int64_t* C, FusedShape* shape);

}  // namespace vce
