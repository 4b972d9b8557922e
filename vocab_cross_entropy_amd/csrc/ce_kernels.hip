// gfx950 kernels of the fused (vocabulary-parallel) cross-entropy library.
//
// Arithmetic (per row of logits x, target t, V = vocab_total, and a smoothed
// target distribution that puts q_t on the target and q_o on every other
// column: q_o = a / V, q_t = q_o + 1 - a for smoothing a over all classes,
// q_o = a / (V - 1), q_t = 1 - a over the other classes):
//   lse  = log sum_j exp(x_j)                       (FP32 accumulation)
//   loss = lse - (q_t - q_o) x_t - q_o sum_j x_j    (= -sum_j q_j (x_j - lse))
//   grad_j = s (exp(x_j - lse) - q_j)
// -- the log_softmax + NLL identity and the softmax-minus-onehot gradient of
// the CANN ops-nn fusion page ("fusion scheme", "backward", smoothing per its
// forward step 4 and "pitfall 3", or the uniform a/V of torch's
// F.cross_entropy), the in-place gradient staging of TransformerEngineNPU
// issue #29 (section 6), and the per-shard (max, sum-exp, target logit)
// exchange of hyper-parallel issue #269 (section 3.1) extended with the row
// sum that q_o > 0 needs.  The host passes q_o, q_t - q_o and 1 - q_t.
//
// Exponentials are taken in base 2 on the hardware v_exp_f32: with
// u = x * log2(e), lse = ln2 * (m2 + log2 sum_j 2^(u_j - m2)) for any m2, and
// m2 = fl(max_j x_j * log2 e) keeps every term <= 1 (the max-shift of the
// ops-nn page's "pitfall 1").
//
// Layout: logical row r = i0 * d1 + i1 starts at element i0*s0 + i1*s1; its
// columns are contiguous.  Each row is cut into a head of up to 15 bytes that
// precedes the first 16-byte boundary, a body of 16-byte vectors and a tail
// of fewer than 16 bytes, so every body access is one coalesced 128-bit load
// or store whatever the row's alignment.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "ce.h"
#include "ce_internal.h"

namespace vce {
namespace {

constexpr float kL = 1.44269504088896340736f;     // log2(e)
constexpr float kLn2 = 0.69314718055994530942f;  // ln(2)
// 1 / kL = kLn2 + kInvLlo exactly enough: kL is log2(e) rounded to FP32, and
// a base-2 log-sum-exp formed with it converts back to natural units by its
// own reciprocal.  Taking ln(2) alone leaves kL's rounding (1.3e-8 relative)
// on the whole lse, 0.13 ulp at lse = 48.
constexpr float kInvLlo = 7.348693209507928e-09f;

// natural lse from the base-2 split c_hi + c_lo, rounded once
__device__ __forceinline__ float lse_natural(float c_hi, float c_lo) {
  return __builtin_fmaf(c_hi, kLn2, __builtin_fmaf(c_hi, kInvLlo, c_lo * kLn2));
}
// Bound on polling iterations of one lane waiting for a partner chunk
// (each iteration sleeps ~128 cycles: ~0.2 s in total), after which the
// row is finished with NaN and the workspace status word is set.
constexpr uint32_t kSpinLimit = 1u << 22;
// Reuse path: the sum pass's terms (scaled by 2^kReuseShift to keep them in
// FP16's normal range) are kept as FP16 for the BF16 gradient, relative
// error 2^-11 next to the gradient's own 2^-9 rounding, inside the 2^-8 bar.
// Near p = q_o the gradient s (p - q_o) cancels and that FP16 error is
// absolute, s q_o 2^-11; the path is taken only while s q_o and q_o are
// small enough that this stays well under the 1e-7 floor (scaled by s).
constexpr int kReuseShift = 14;
constexpr float kReuseUnscale = 1.f / 16384.f;
constexpr float kReuseSA = 4e-5f;
constexpr float kReuseA = 5e-5f;
// and the FP16 error of a single term, |s| p 2^-11, stays below half the floor
constexpr float kReuseAbs = 5e-8f;
// The streaming kernels' instance for rows of at most 1024 vectors, the only
// one that rows of at most kShortRow columns get; it alone compiles their
// FP64 whole-row path.
constexpr int kShortT = 256, kShortPB = 4;

// Phase stamps, in the instrumented build only (-DCE_PHASE_CLOCK, libce_phases.so):
// thread 0 of a workgroup stores the real-time counter (100 MHz) into
// slot i of its record; the normal build compiles them out.
#ifdef CE_PHASE_CLOCK
#define CE_STAMP(buf, rec, i)                                                   \
  do {                                                                          \
    if ((buf) && threadIdx.x == 0) (buf)[(size_t)(rec) * 8u + (i)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
#else
#define CE_STAMP(buf, rec, i) \
  do {                        \
  } while (0)
#endif

template <int DT>
struct ElemT;
template <>
struct ElemT<CE_BF16> {
  static constexpr int E = 8;   // elements per 16-byte vector
  static constexpr int EB = 2;  // bytes per element
};
template <>
struct ElemT<CE_F32> {
  static constexpr int E = 4;
  static constexpr int EB = 4;
};

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// FP32 pair -> packed BF16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  f2 in = {lo, hi};
  b2 out = __builtin_convertvector(in, b2);
  return __builtin_bit_cast(uint32_t, out);
}

// Raw buffer accesses with a byte range: a load past the range returns zero
// and a store past it is dropped by the hardware, so partly filled vector
// slots need no branch (a branch around each load would serialise them).
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit element format

// A range of `bytes` (below 4 GiB: the host refuses longer rows) starting at p;
// the hardware reads the count as unsigned, so the narrowing keeps its bits.
__device__ __forceinline__ Rsrc make_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)(uint32_t)bytes, kRsrcWord3);
}
// Cache policy of the 16-byte loads and stores (the buffer instructions'
// cache-policy operand).  kStream sets the non-temporal bit: the line is
// touched once, so the caches give it the lowest priority to stay.  The
// fused, statistics and backward kernels take it for the logits they stream.
// On the 4 x 2048 x 128000 BF16 fused step: 675 against 735 us with loads and
// stores marked, 706 with the stores alone, 714 with the loads alone; the
// forward + backward pair: 1,151 against 1,174 us.
constexpr int kCacheDefault = 0, kCacheStream = 2;
template <int CP = kCacheDefault>
__device__ __forceinline__ uint4 bload16(Rsrc r, uint32_t off) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, CP);
  return make_uint4(v.x, v.y, v.z, v.w);
}
template <int CP = kCacheDefault>
__device__ __forceinline__ void bstore16(const uint4& v, Rsrc r, uint32_t off) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(w, r, (int)off, 0, CP);
}
// one element (index j) of a range-checked buffer, widened to FP32 (0 outside)
template <int DT>
__device__ __forceinline__ float bload_elem(Rsrc r, int j) {
  if constexpr (DT == CE_BF16) {
    return __uint_as_float((uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, j * 2, 0, 0) << 16);
  } else {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, j * 4, 0, 0));
  }
}
template <int DT>
__device__ __forceinline__ void bstore_elem(float g, Rsrc r, int j) {
  if constexpr (DT == CE_BF16) {
    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)(pack_bf16(g, 0.f) & 0xffffu), r, j * 2, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(g), r, j * 4, 0, 0);
  }
}

// FP32 pair -> packed FP16 pair, round to nearest even (v_cvt_pk_f16_f32).
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  f2 in = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(in, h2));
}
// A vector's terms packed to FP16 pairs (the staging of BF16 gradients; FP32
// rows never stage, their instance only needs to compile).
template <int DT>
__device__ __forceinline__ uint4 pack_terms_f16(const float (&t)[ElemT<DT>::E]) {
  if constexpr (DT == CE_BF16)
    return make_uint4(pack_f16(t[0], t[1]), pack_f16(t[2], t[3]), pack_f16(t[4], t[5]), pack_f16(t[6], t[7]));
  else
    return make_uint4(pack_f16(t[0], t[1]), pack_f16(t[2], t[3]), 0u, 0u);
}

// fma(FP16 half of w widened to FP32, k, c) in one v_fma_mix_f32
// (op_sel_hi marks operand 0 as FP16, op_sel picks its high half).
__device__ __forceinline__ float fma_mix_lo(uint32_t w, float k, float c) {
  float d;
  asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(d) : "v"(w), "v"(k), "v"(c));
  return d;
}
__device__ __forceinline__ float fma_mix_hi(uint32_t w, float k, float c) {
  float d;
  asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(w), "v"(k), "v"(c));
  return d;
}

template <int DT>
__device__ __forceinline__ void unpack(const uint4& v, float (&f)[ElemT<DT>::E]) {
  if constexpr (DT == CE_BF16) {
    f[0] = bf_lo(v.x); f[1] = bf_hi(v.x);
    f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
    f[4] = bf_lo(v.z); f[5] = bf_hi(v.z);
    f[6] = bf_lo(v.w); f[7] = bf_hi(v.w);
  } else {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
}

template <int DT>
__device__ __forceinline__ uint4 pack(const float (&f)[ElemT<DT>::E]) {
  if constexpr (DT == CE_BF16) {
    return make_uint4(pack_bf16(f[0], f[1]), pack_bf16(f[2], f[3]), pack_bf16(f[4], f[5]), pack_bf16(f[6], f[7]));
  } else {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3]));
  }
}

template <int DT>
__device__ __forceinline__ float load_elem(const char* base, int64_t j) {
  if constexpr (DT == CE_BF16) {
    return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(base)[j] << 16);
  } else {
    return reinterpret_cast<const float*>(base)[j];
  }
}

template <int DT>
__device__ __forceinline__ void store_elem(char* base, int64_t j, float g) {
  if constexpr (DT == CE_BF16) {
    reinterpret_cast<uint16_t*>(base)[j] = (uint16_t)(pack_bf16(g, 0.f) & 0xffffu);
  } else {
    reinterpret_cast<float*>(base)[j] = g;
  }
}

template <int DT>
__device__ __forceinline__ float extract(const uint4& v, int e) {
  float f[ElemT<DT>::E];
  unpack<DT>(v, f);
  float r = f[0];
#pragma unroll
  for (int i = 1; i < ElemT<DT>::E; ++i) r = (e == i) ? f[i] : r;
  return r;
}

// Register barrier: the compiler must assume v changed, so the unpacked
// floats of one sweep are recomputed (one shift or mask each) in the next
// instead of being kept alive, which would double the registers a chunk
// needs.  Emits no instruction.
__device__ __forceinline__ void launder(uint4& v) {
  asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

// The largest of three floats in one v_max3_f32.  fmaxf on values that come
// from integer unpacking makes the compiler quiet each operand first (one
// v_max_f32 x, x per element), which doubled the max pass's instructions.  A
// NaN element still makes the row NaN: the sum pass's exponential carries it.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float d;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
  return d;
}

// max(m, elements of v)
template <int DT>
__device__ __forceinline__ float vec_max(const uint4& v, float m) {
  if constexpr (DT == CE_BF16) {
    m = max3(m, bf_lo(v.x), bf_hi(v.x));
    m = max3(m, bf_lo(v.y), bf_hi(v.y));
    m = max3(m, bf_lo(v.z), bf_hi(v.z));
    return max3(m, bf_lo(v.w), bf_hi(v.w));
  } else {
    m = max3(m, __uint_as_float(v.x), __uint_as_float(v.y));
    return max3(m, __uint_as_float(v.z), __uint_as_float(v.w));
  }
}

// sum of the elements of v (BF16 pairs through v_dot2_f32_bf16 with (1, 1))
template <int DT>
__device__ __forceinline__ float vec_sum(const uint4& v) {
  if constexpr (DT == CE_BF16) {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const b2 one = __builtin_bit_cast(b2, 0x3f803f80u);
    float acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, v.x), one, 0.f, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, v.y), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, v.z), one, acc, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, v.w), one, acc, false);
  } else {
    return (__uint_as_float(v.x) + __uint_as_float(v.y)) + (__uint_as_float(v.z) + __uint_as_float(v.w));
  }
}

// v with element e replaced by -inf
template <int DT>
__device__ __forceinline__ uint4 with_neg_inf(uint4 v, int e) {
  if constexpr (DT == CE_BF16) {
    const int q = e >> 1;
    const bool hi = e & 1;
    auto put = [&](uint32_t w) { return hi ? ((w & 0x0000ffffu) | 0xff800000u) : ((w & 0xffff0000u) | 0x0000ff80u); };
    if (q == 0) v.x = put(v.x);
    if (q == 1) v.y = put(v.y);
    if (q == 2) v.z = put(v.z);
    if (q == 3) v.w = put(v.w);
  } else {
    if (e == 0) v.x = 0xff800000u;
    if (e == 1) v.y = 0xff800000u;
    if (e == 2) v.z = 0xff800000u;
    if (e == 3) v.w = 0xff800000u;
  }
  return v;
}

// exp(x - lse) from the base-2 lse split c_hi + c_lo.  For BF16 gradients the
// low part is far below their rounding and is dropped.
template <int DT>
__device__ __forceinline__ float softmax_term(float x, float c_hi, float c_lo) {
  if constexpr (DT == CE_BF16) {
    return ex2(__builtin_fmaf(x, kL, -c_hi));
  } else {
    return ex2(__builtin_fmaf(x, kL, -c_hi) - c_lo);
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Workgroup reductions in a fixed order (deterministic, uniform result).
template <int T>
__device__ __forceinline__ float block_max(float v, float (*sh)[4]) {
  v = wave_max(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) sh[w][0] = v;
  __syncthreads();
  float r = sh[0][0];
#pragma unroll
  for (int i = 1; i < T / 64; ++i) r = fmaxf(r, sh[i][0]);
  __syncthreads();
  return r;
}

template <int T>
__device__ __forceinline__ void block_sum3(float& a, float& b, float& c, float (*sh)[4]) {
  a = wave_sum(a);
  b = wave_sum(b);
  c = wave_sum(c);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sh[w][0] = a;
    sh[w][1] = b;
    sh[w][2] = c;
  }
  __syncthreads();
  a = sh[0][0];
  b = sh[0][1];
  c = sh[0][2];
#pragma unroll
  for (int i = 1; i < T / 64; ++i) {
    a += sh[i][0];
    b += sh[i][1];
    c += sh[i][2];
  }
  __syncthreads();
}

// Geometry of one logical row.
template <int DT>
struct Row {
  char* base;     // element 0
  int64_t h;      // head elements before the first 16-byte boundary
  int64_t nv;     // body vectors
  int tn;         // tail elements
  uint4* body;    // first body vector
  char* tail;     // first tail element
  int64_t t;      // target (global index)
};

template <int DT, bool HT = true>
__device__ __forceinline__ Row<DT> row_geometry(const RowLayout& L, int64_t r) {
  constexpr int E = ElemT<DT>::E, EB = ElemT<DT>::EB;
  Row<DT> g;
  const int64_t i0 = r / L.d1, i1 = r - i0 * L.d1;
  g.t = L.tgt[i0 * L.ts0 + i1 * L.ts1];
  g.base = L.x + (i0 * L.s0 + i1 * L.s1) * EB;
  int64_t h = HT ? (int64_t)(((16u - ((uint32_t)(uintptr_t)g.base & 15u)) & 15u) / EB) : 0;
  g.h = h > L.V ? L.V : h;
  g.nv = (L.V - g.h) / E;
  g.tn = (int)(L.V - g.h - g.nv * E);
  g.body = reinterpret_cast<uint4*>(g.base + g.h * EB);
  g.tail = g.base + (g.h + g.nv * E) * EB;
  return g;
}

// Row r's span without its target (for scaling a staged gradient).
template <int DT>
__device__ __forceinline__ Row<DT> row_span(const RowLayout& L, int64_t r) {
  constexpr int E = ElemT<DT>::E, EB = ElemT<DT>::EB;
  Row<DT> g;
  const int64_t i0 = r / L.d1, i1 = r - i0 * L.d1;
  g.t = 0;
  g.base = L.x + (i0 * L.s0 + i1 * L.s1) * EB;
  const int64_t h = (int64_t)(((16u - ((uint32_t)(uintptr_t)g.base & 15u)) & 15u) / EB);
  g.h = h > L.V ? L.V : h;
  g.nv = (L.V - g.h) / E;
  g.tn = (int)(L.V - g.h - g.nv * E);
  g.body = reinterpret_cast<uint4*>(g.base + g.h * EB);
  g.tail = g.base + (g.h + g.nv * E) * EB;
  return g;
}

// lse - (q_t - q_o) x_t - q_o sum_j x_j, leaving out a term whose weight is 0
// (0 log 0 = 0): a masked class (a logit of -inf) with no smoothing weight
// keeps the loss finite, as in torch's F.cross_entropy.
__device__ __forceinline__ float row_loss_of(float lse, float q_to, float y, float q_o, float r) {
  float l = lse;
  if (q_to != 0.f) l -= q_to * y;
  if (q_o != 0.f) l -= q_o * r;
  return l;
}

// Upstream gradient scale s of row r: g_r, g / n (mean) or g (sum).
__device__ __forceinline__ float grad_scale(int32_t reduce, const float* g, const int32_t* n_valid, int64_t r) {
  if (reduce == CE_REDUCE_MEAN) return (g ? g[0] : 1.f) / (float)(*n_valid);
  if (reduce == CE_REDUCE_SUM) return g ? g[0] : 1.f;
  return g ? g[r] : 1.f;
}

// n = #{rows whose target is not ignore_idx}, counted by one workgroup of T
// threads (the caller's workgroup 0; nothing else in its kernel needs n, so
// no other workgroup waits for it).  Returned in every thread.
template <int T>
__device__ int32_t block_count_targets(const int64_t* tgt, int64_t ts0, int64_t ts1, int64_t d1, int64_t N,
                                       int64_t ignore_idx) {
  __shared__ int csh[T / 64];
  int cnt = 0;
#pragma unroll 4
  for (int64_t r = threadIdx.x; r < N; r += T) {
    const int64_t i0 = r / d1, i1 = r - i0 * d1;
    cnt += tgt[i0 * ts0 + i1 * ts1] != ignore_idx;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
  if ((threadIdx.x & 63) == 0) csh[threadIdx.x >> 6] = cnt;
  __syncthreads();
  int n = 0;
#pragma unroll
  for (int i = 0; i < T / 64; ++i) n += csh[i];
  __syncthreads();
  return n;
}

// --------------------------------------------------------------------------
// Calls on no rows: n = 0 (the mean of no rows is then 0/0).
__global__ __launch_bounds__(64) void k_zero_count(int32_t* n_out) {
  if (threadIdx.x == 0) n_out[0] = 0;
}

// --------------------------------------------------------------------------
// Words the fused kernel's workgroups exchange are 64 bits: the call's tag
// in the high half, a 32-bit payload in the low half, written and read with
// relaxed agent-scope atomics.  The tag is the low half of the workspace's
// epoch word, which the last workgroup of each call advances (never to a
// value whose low half is 0), so a word left by an earlier call (or the
// zeros of ce_workspace_init) never passes for this call's, the workspace
// needs no clearing between calls, and a call replayed from a captured graph
// (same kernel arguments) still gets a fresh tag.
__device__ __forceinline__ unsigned long long tagged(uint32_t tag, uint32_t payload) {
  return ((unsigned long long)tag << 32) | payload;
}
__device__ __forceinline__ void publish(unsigned long long* p, uint32_t tag, uint32_t payload) {
  __hip_atomic_store(p, tagged(tag, payload), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long poll(const unsigned long long* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Publish a fused row's loss: chunk 0 of each row publishes a tagged word
// (fire-and-forget, no round trip before the workgroup exits), which the
// last workgroup collects for the mean and, in both modes, as proof that
// every workgroup has read the epoch; without reduction it also goes
// straight to loss[r].
template <int T>
__device__ __forceinline__ void publish_row_loss(const FusedArgs& a, uint32_t tag, int64_t r, float loss,
                                                 bool chunk0) {
  if (!chunk0 || threadIdx.x != 0) return;
  if (!a.reduce) a.row_loss[r] = loss;
  publish(a.row_loss_tagged + r, tag, __float_as_uint(loss));
}

// n = #{rows whose target is not ignore_idx}, counted inside the fused kernel:
// workgroup b < nslice counts rows [b * slice_rows, (b + 1) * slice_rows)
// before anything else and publishes a tagged count in the header.  Those
// workgroups start first and wait for nothing, so the counts always arrive.
template <int T>
__device__ void count_slice(const FusedArgs& a, uint32_t tag, int64_t b) {
  __shared__ int csh[T / 64];
  const RowLayout& L = a.L;
  const int64_t r0 = b * a.slice_rows;
  const int64_t r1 = r0 + a.slice_rows < L.N ? r0 + a.slice_rows : L.N;
  int cnt = 0;
  for (int64_t r = r0 + threadIdx.x; r < r1; r += T) {
    const int64_t i0 = r / L.d1, i1 = r - i0 * L.d1;
    cnt += L.tgt[i0 * L.ts0 + i1 * L.ts1] != L.ignore_idx;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o);
  if ((threadIdx.x & 63) == 0) csh[threadIdx.x >> 6] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0;
    for (int i = 0; i < T / 64; ++i) n += csh[i];
    publish(&a.hdr->counts[b], tag, (uint32_t)n);
  }
}

// The slice counts as seen by one wave: lane q < nslice holds count q's word,
// read with an agent-scope load (issued early, its round trip overlaps other
// loads); lanes whose word does not carry this call's tag yet poll it again,
// bounded.  (A plain, cached load could keep a stale line in an XCD's L2.)
__device__ __forceinline__ unsigned long long count_word_early(const FusedArgs& a) {
  const int lane = threadIdx.x & 63;
  return lane < a.nslice ? poll(&a.hdr->counts[lane]) : 0ull;
}
__device__ int32_t wave_count(const FusedArgs& a, uint32_t tag, unsigned long long w, bool* ok) {
  const int lane = threadIdx.x & 63;
  const bool mine = lane < a.nslice;
  bool ready = !mine || (uint32_t)(w >> 32) == tag;
  uint32_t spins = 0;
  while (!__all(ready) && spins <= kSpinLimit) {
    if (!ready) {
      w = poll(&a.hdr->counts[lane]);
      ready = (uint32_t)(w >> 32) == tag;
    }
    ++spins;
    __builtin_amdgcn_s_sleep(2);
  }
  *ok = __all(ready);
  int c = mine ? (int)(uint32_t)w : 0;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) c += __shfl_xor(c, o);
  return c;
}

// The last item's workgroup finishes the call once its own item is done: it
// starts after every other workgroup of the launch (in-order dispatch, see
// k_fused), none of which waits for it, so every tagged word arrives.  It
// writes n and, with the mean, the N losses summed in index order in FP64
// (deterministic).  Last, it advances the epoch: every workgroup that used
// this call's tag has read it by then (its words fed a row loss, a count or
// both), so the next call's tag is set only after this call is done with it.
// Every row's tagged loss, summed in index order in FP64 by this workgroup
// (thread-partial sums; the caller combines them in a fixed order).  Words
// that have not arrived are polled again, bounded.
template <int T>
__device__ double poll_row_losses(const FusedArgs& a, uint32_t tag, bool* gave_up_out) {
  // independent loads in flight per thread (more would raise the kernel's register need)
  constexpr int U = 8;
  double acc = 0.0;
  uint32_t spins = 0;
  bool gave_up = false;
  for (int64_t base = 0; base < a.L.N; base += (int64_t)T * U) {
    unsigned long long w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + (int64_t)u * T + threadIdx.x;
      w[u] = i < a.L.N ? poll(a.row_loss_tagged + i) : tagged(tag, 0u);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + (int64_t)u * T + threadIdx.x;
      while ((uint32_t)(w[u] >> 32) != tag && !gave_up) {
        if (++spins > kSpinLimit) {
          gave_up = true;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
        w[u] = poll(a.row_loss_tagged + i);
      }
      acc += gave_up ? __builtin_nan("") : (double)__uint_as_float((uint32_t)w[u]);
    }
  }
  *gave_up_out = gave_up;
  return acc;
}

// Advance the workspace's epoch (skipping values whose low half is 0); the
// caller has seen every word tagged with this call's tag.
__device__ __forceinline__ void advance_epoch(const FusedArgs& a) {
  unsigned long long next = a.hdr->epoch + 1;  // this call's epoch: nothing has written it since
  if ((uint32_t)next == 0u) ++next;
  __hip_atomic_store(&a.hdr->epoch, next, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The last item's workgroup finishes the call once its own item is done: it
// starts after every other workgroup of the launch (in-order dispatch, see
// k_fused), none of which waits for it, so every tagged word arrives.  It
// writes n and, with a reduction, the N losses summed in index order in FP64
// (deterministic), divided by n for the mean.  Last, it advances the epoch:
// every workgroup that used this call's tag has read it by then (its words
// fed a row loss, a count or both), so the next call's tag is set only after
// this call is done with it.
// (Reduced and unreduced calls keep separate tails: sharing the mean's tail measurably
// raised the whole kernel's register allocation.)
template <int T>
__device__ void fused_finish(const FusedArgs& a, uint32_t tag, bool ws_ok) {
  __shared__ double s_sum[T / 64];
  // In a workspace ce_workspace_init never prepared (ws_ok false), stale
  // words can carry the "tag" (both are whatever the memory held), so the
  // counts and row losses read here mean nothing: n is then -1 and the mean
  // or sum NaN, like every row's loss and gradient.
  bool cnt_ok = true;
  const int32_t n = wave_count(a, tag, count_word_early(a), &cnt_ok);
  if (threadIdx.x == 0) {
    if (!cnt_ok) atomicOr(&a.hdr->status, 1u);
    if (a.n_out) a.n_out[0] = ws_ok ? n : -1;
  }
  bool gave_up = false;
  if (!a.reduce) {
    (void)poll_row_losses<T>(a, tag, &gave_up);
    if (gave_up) atomicOr(&a.hdr->status, 1u);
    __syncthreads();
    if (threadIdx.x == 0) advance_epoch(a);
    return;
  }
  double acc = poll_row_losses<T>(a, tag, &gave_up);
  if (gave_up) atomicOr(&a.hdr->status, 1u);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) s_sum[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
    for (int i = 0; i < T / 64; ++i) tot += s_sum[i];
    // N >= 1 here; n = 0 gives 0/0 = NaN
    if (!ws_ok)
      a.mean_out[0] = __builtin_nanf("");
    else if (a.reduce == CE_REDUCE_SUM)
      a.mean_out[0] = (float)tot;
    else
      a.mean_out[0] = cnt_ok ? (float)(tot / (double)n) : __builtin_nanf("");
    advance_epoch(a);
  }
}

// --------------------------------------------------------------------------
// A whole row of at most kShortRow = 128 columns, in FP64, by one wave (two
// columns per lane: columns lane and lane + 64): max, the sum of exp(x - max)
// over the columns other than the target, the target logit and the row sum
// by wave reductions, then loss and gradient s (p_j - q_j) rounded once to
// the output.  Rows this short cost a launch whatever the arithmetic, and
// FP32 cannot hold the gradient where p_j sits close to a large q_j (few
// columns, heavy smoothing: q_o = a / V reaches 1/128 at 128 columns): one
// FP32 rounding of p already exceeds the FP32 gradient's absolute floor there.
__device__ __forceinline__ double wave_max_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// (m, d, y, r) of a row held by one wave, two columns per lane: x0 is column
// lane, x1 column lane + 64 (in0 / in1: inside the row); tl is the target's
// column in this buffer (outside [0, 128): not here, y = 0).  d leaves the
// target's term out.  Uniform over the wave.
struct Stats64 {
  double m, d, y, r;
};
__device__ __forceinline__ Stats64 wave_stats64(double x0, bool in0, double x1, bool in1, int64_t tl) {
  const int lane = threadIdx.x & 63;
  const bool t0 = in0 && tl == lane, t1 = in1 && tl == lane + 64;
  Stats64 st;
  st.m = wave_max_d(fmax(in0 ? x0 : -INFINITY, in1 ? x1 : -INFINITY));
  st.d = wave_sum_d((in0 && !t0 ? exp(x0 - st.m) : 0.0) + (in1 && !t1 ? exp(x1 - st.m) : 0.0));
  st.y = wave_sum_d(t0 ? x0 : (t1 ? x1 : 0.0));
  st.r = wave_sum_d((in0 ? x0 : 0.0) + (in1 ? x1 : 0.0));
  return st;
}
// lse of a whole row from its wave statistics, the target's term restored
__device__ __forceinline__ double lse_of64(const Stats64& st) {
  return st.m + log(st.d + (st.y == -INFINITY ? 0.0 : exp(st.y - st.m)));
}
// lse - (q_t - q_o) y - q_o r, leaving out a term whose weight is 0 (as row_loss_of)
__device__ __forceinline__ double row_loss64(double lse, double q_o, double q_t, double y, double r) {
  double loss = lse;
  if (q_t != q_o) loss -= (q_t - q_o) * y;
  if (q_o != 0.0) loss -= q_o * r;
  return loss;
}

// The arithmetic of a short row held by wave 0 (columns lane and lane + 64,
// global index = local index): publishes the row's loss and returns the
// lane's two gradients.
template <int T>
__device__ void short_row_grad(const FusedArgs& a, uint32_t tag, int64_t r, int64_t t, double x0, bool in0,
                               double x1, bool in1, double* g0, double* g1) {
  const int lane = threadIdx.x;
  const RowLayout& L = a.L;
  const bool ws_ok = (a.hdr->magic == kWsMagic) & (a.hdr->init_bytes >= a.ws_bytes);
  const bool tvalid = t >= 0 && t < L.vocab_total;

  // s = g_r, g / n (the mean; n from the slice counts) or g (the sum)
  double s = a.g ? (double)a.g[a.reduce ? 0 : r] : 1.0;
  if (a.reduce == CE_REDUCE_MEAN) {
    bool ok;
    const int32_t n = wave_count(a, tag, count_word_early(a), &ok);
    s = ok ? s / (double)n : __builtin_nan("");
  }
  if (!ws_ok) {
    s = __builtin_nan("");
    if (lane == 0) atomicOr(&a.hdr->status, 2u);
  }

  const Stats64 st = wave_stats64(x0, in0, x1, in1, tvalid ? t : -1);
  const double lse = lse_of64(st);
  const double loss = row_loss64(lse, a.q_o_d, a.q_t_d, st.y, st.r);
  publish_row_loss<T>(a, tag, r, tvalid && ws_ok ? (float)loss : __uint_as_float(0x7fc00000u), true);
  const double q0 = lane == t ? a.q_t_d : a.q_o_d, q1 = lane + 64 == t ? a.q_t_d : a.q_o_d;
  *g0 = tvalid ? s * (exp(x0 - lse) - q0) : __builtin_nan("");
  *g1 = tvalid ? s * (exp(x1 - lse) - q1) : __builtin_nan("");
}

template <int DT, int T>
__device__ void fused_short_row(const FusedArgs& a, uint32_t tag, int64_t r, const Row<DT>& g) {
  const int lane = threadIdx.x;
  if (lane >= 64) return;  // wave 0 holds the row
  const Rsrc rx = make_rsrc(g.base, a.L.V * ElemT<DT>::EB);  // lanes past the row read 0, their stores drop
  const bool in0 = lane < a.L.V, in1 = lane + 64 < a.L.V;
  const double x0 = (double)bload_elem<DT>(rx, lane), x1 = (double)bload_elem<DT>(rx, lane + 64);
  double g0, g1;
  short_row_grad<T>(a, tag, r, g.t, x0, in0, x1, in1, &g0, &g1);
  bstore_elem<DT>((float)g0, rx, lane);
  bstore_elem<DT>((float)g1, rx, lane + 64);
}

// The same for a short row held as vocabulary shards: lane j gathers global
// columns j and j + 64 from the shards that hold them (per-lane addresses, so
// plain loads and stores rather than one buffer range).  Ignored rows store
// +0.0 in every shard's piece, loss 0.
template <int DT, int T>
__device__ void fused_short_row_shards(const FusedArgs& a, uint32_t tag, int64_t r, int64_t t, const ShardSet* ss) {
  constexpr int EB = ElemT<DT>::EB;
  const int lane = threadIdx.x;
  if (lane >= 64) return;
  const int64_t i0 = r / a.L.d1, i1 = r - i0 * a.L.d1;
  char* p0 = nullptr;
  char* p1 = nullptr;
  for (int k = 0; k < ss->S; ++k) {
    const RowLayout& Ls = ss->L[k];
    char* rowp = Ls.x + (i0 * Ls.s0 + i1 * Ls.s1) * EB;
    if (lane >= Ls.vocab_start && lane < Ls.vocab_start + Ls.V) p0 = rowp + (lane - Ls.vocab_start) * EB;
    if (lane + 64 >= Ls.vocab_start && lane + 64 < Ls.vocab_start + Ls.V) p1 = rowp + (lane + 64 - Ls.vocab_start) * EB;
  }
  const bool in0 = p0 != nullptr, in1 = p1 != nullptr;
  if (t == a.L.ignore_idx) {
    if (in0) store_elem<DT>(p0, 0, 0.f);
    if (in1) store_elem<DT>(p1, 0, 0.f);
    publish_row_loss<T>(a, tag, r, 0.f, true);
    return;
  }
  const double x0 = in0 ? (double)load_elem<DT>(p0, 0) : 0.0;
  const double x1 = in1 ? (double)load_elem<DT>(p1, 0) : 0.0;
  double g0, g1;
  short_row_grad<T>(a, tag, r, t, x0, in0, x1, in1, &g0, &g1);
  if (in0) store_elem<DT>(p0, 0, (float)g0);
  if (in1) store_elem<DT>(p1, 0, (float)g1);
}

// --------------------------------------------------------------------------
// Fused forward + backward.  One workgroup per (row, chunk); the chunk's
// body vectors live in registers (P per thread) between the statistics pass
// and the gradient pass, so the logits are read from HBM once and the
// gradient is written once.  With K > 1 chunks per row, every chunk publishes
// (m2, d_excl, y, r) as tagged 64-bit words, waits for its partners, and all
// chunks combine the K tuples in chunk order, so they agree bit for bit on
// the row's lse.  Item = blockIdx.x, and the K chunks of a row are K
// consecutive workgroups.  The hardware dispatcher starts the workgroups of
// a launch in increasing index order (round robin over the XCDs, in order
// within each), so a chunk that waits for a partner waits for a workgroup
// that is running or will start as soon as any running one, whose partners
// have all started, finishes.  An atomic ticket would give the same
// guarantee without that ordering, but its round trip at every workgroup's
// start measured 3% of the kernel on 128000-column rows.  Every wait is
// bounded: a partner that never arrives makes the chunk give up with NaN
// results and a status word, never a hang.
//
// The target's own term is kept out of the sum-exp (its register copy is
// set to -inf after the max pass and its term is rebuilt from the target
// logit), so that 1 - p_t = D_excl / D stays accurate when the target holds
// almost all of the probability; its gradient is stored separately after the
// vector stores.
// HT: rows may have head/tail elements (a row start or end off a 16-byte
// boundary).  When every row is aligned the host launches HT = false, which
// keeps the two scalar element registers out of the chunk's register budget.
// SH: the row's K chunks are kper sub-chunks of each of ss->S vocabulary
// shards (separate buffers, each with its own layout and vocab_start), the
// single-read form of the shard flow; chunk k is sub-chunk k mod kper of
// shard k / kper.  Without SH they are K consecutive pieces of one buffer.
template <int DT, int T, int P, bool HT, bool SH>
__device__ __forceinline__ void fused_item(const FusedArgs& a, const ShardSet* ss) {
  constexpr int E = ElemT<DT>::E;
  __shared__ float sh[T / 64][4];
  __shared__ float xs[64 * 4];
  __shared__ int sh_n;
  const int tid = threadIdx.x;
  const RowLayout& L = a.L;  // targets, rows, ignore_idx, vocabulary and smoothing: common to all shards
  // A new workgroup's waves take issue priority over the running ones on
  // their SIMD until the chunk loads are out: its memory requests go in flight
  // sooner, while the others' arithmetic loses little (on the 4 x 2048 x
  // 128000 BF16 workload about 2% of the kernel's time, in interleaved runs).
  __builtin_amdgcn_s_setprio(3);
  const int K = a.K;

  const int64_t item = blockIdx.x;
  CE_STAMP(a.phase, item, 0);
  // the workspace's init record and epoch, with scalar loads (constant
  // address space: nothing writes them before this call's last workgroup
  // finishes); the epoch's low half is this call's tag
  typedef const __attribute__((address_space(4))) unsigned long long* ConstU64;
  const ConstU64 wsrec = (ConstU64)(&a.hdr->magic);  // magic, init_bytes, epoch, withhold
  const uint32_t tag = (uint32_t)wsrec[2];
  const bool ws_ok = (wsrec[0] == kWsMagic) & (wsrec[1] >= a.ws_bytes);
  const unsigned long long withhold = wsrec[3];  // the test hook (0 in every prepared workspace)
  if (item < a.nslice) count_slice<T>(a, tag, item);
  const int64_t last_item = L.N * K - 1;
  const int64_t r = item / K;
  const int k = (int)(item - r * K);
  if (r >= L.N) return;

  int kb = k, kper = K;  // this chunk's place in its buffer
  const RowLayout* Lb = &a.L;
  if constexpr (SH) {
    kper = ss->kper;
    const int sidx = k / kper;
    kb = k - sidx * kper;
    Lb = &ss->L[sidx];
  }
  const Row<DT> g = row_geometry<DT, HT>(*Lb, r);
  const int64_t cb = (int64_t)kb * a.C;
  const int64_t cend = g.nv < cb + a.C ? g.nv : cb + a.C;
  const int nvc = cend > cb ? (int)(cend - cb) : 0;
  uint4* body = g.body + cb;
  const bool first = (kb == 0), last = (kb == kper - 1);  // the buffer's head and tail
  const bool row_first = (k == 0);                      // the row's loss is published once

  if (SH && P == 1 && a.short_rows) {  // a vocabulary of at most kShortRow columns across the shards
    if constexpr (SH && P == 1) fused_short_row_shards<DT, T>(a, tag, r, g.t, ss);
  } else if (g.t == L.ignore_idx) {  // ignored row: +0.0 gradient, loss 0, nothing read
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    for (int i = tid; i < nvc; i += T) body[i] = z;
    if (HT) {
      if (first && tid < g.h) store_elem<DT>(g.base, tid, 0.f);
      if (last && tid < g.tn) store_elem<DT>(g.tail, tid, 0.f);
    }
    publish_row_loss<T>(a, tag, r, 0.f, row_first);
  } else if (P == 1 && a.short_rows) {
    if constexpr (P == 1) fused_short_row<DT, T>(a, tag, r, g);
  } else {

    // ---- the single read of this chunk (slots past the chunk read as zero
    // and are masked below; their stores are dropped)
    const Rsrc rb = make_rsrc(body, (int64_t)nvc * 16);
    const Rsrc rh = make_rsrc(g.base, HT && first ? g.h * ElemT<DT>::EB : 0);
    const Rsrc rt = make_rsrc(g.tail, HT && last ? (int64_t)g.tn * ElemT<DT>::EB : 0);
    // The slice counts (wave 0, an agent-scope load to memory) go out before
    // the chunk loads, so their round trip overlaps them; the upstream
    // gradient after.  The initialisation record came in with scalar loads,
    // which keeps it out of the vector loads' in-order completion count, and
    // is combined without branches, so no wait is placed before the chunk is
    // in flight.
    const unsigned long long cw = (a.reduce == CE_REDUCE_MEAN && tid < 64) ? count_word_early(a) : 0ull;
    uint4 v[P];
#pragma unroll
    for (int j = 0; j < P; ++j) v[j] = bload16<kCacheStream>(rb, (uint32_t)(j * T + tid) * 16u);
    CE_STAMP(a.phase, item, 1);
    __builtin_amdgcn_s_setprio(0);
    const float g_up = a.g ? a.g[a.reduce ? 0 : r] : 1.f;

    const bool hv = HT && first && tid < g.h, tv = HT && last && tid < g.tn;
    float hx = -INFINITY, tx = -INFINITY;
    if (HT) {
      hx = bload_elem<DT>(rh, tid);
      tx = bload_elem<DT>(rt, tid);
      hx = hv ? hx : -INFINITY;
      tx = tv ? tx : -INFINITY;
    }

    // ---- where the target sits (uniform): head, body (chunk, vector, lane,
    // element) or tail; only the chunk that holds it has own_tid >= 0
    const bool tvalid = g.t >= 0 && g.t < L.vocab_total;
    const int64_t tl = g.t - Lb->vocab_start;
    // a shard owns the target only when it lies in the shard's own columns
    // (one unsharded buffer holds every valid target)
    const bool tin = SH ? (tvalid && tl >= 0 && tl < Lb->V) : tvalid;
    int own_tid = -1, own_j = 0, own_e = 0;
    if (tin) {
      if (tl < g.h) {
        if (first) own_tid = (int)tl;
      } else {
        const int64_t c = tl - g.h;
        if (c < g.nv * E) {
          const int64_t vec = c / E;
          if (vec >= cb && vec < cend) {
            const int vi = (int)(vec - cb);
            own_j = vi / T;
            own_tid = vi - own_j * T;
            own_e = (int)(c - vec * E);
          }
        } else if (last) {
          own_tid = (int)(c - g.nv * E);
        }
      }
    }
    const int own_where = own_tid < 0 ? 0 : (tl < g.h ? 1 : (tl - g.h < g.nv * E ? 2 : 3));

    // ---- max, and the row sum that the smoothing term needs
    const bool smooth = L.q_o != 0.f;
    float m = fmaxf(hx, tx);
    float rs = (hv ? hx : 0.f) + (tv ? tx : 0.f);
    if (smooth) {
#pragma unroll
      for (int j = 0; j < P; ++j) {
        const float mj = vec_max<DT>(v[j], m);
        m = (j * T + tid < nvc) ? mj : m;
        rs += vec_sum<DT>(v[j]);  // slots past the chunk hold zeros
      }
    } else {
#pragma unroll
      for (int j = 0; j < P; ++j) {
        const float mj = vec_max<DT>(v[j], m);
        m = (j * T + tid < nvc) ? mj : m;
      }
    }
    const float m_loc = m;  // this thread's own maximum (bounds its largest softmax term)
    if (a.reduce == CE_REDUCE_MEAN && tid < 64) {  // n, handed to the other waves by block_max's barrier
      bool ok;
      const int32_t n = wave_count(a, tag, cw, &ok);
      if (tid == 0) sh_n = ok ? n : -1;
    }
    m = block_max<T>(m, sh);
    CE_STAMP(a.phase, item, 2);
    // s = g / n with the mean, g with the sum, g_r without; NaN (loud) when a
    // count never arrived or the workspace was not initialised
    float s_up = g_up;
    if (a.reduce == CE_REDUCE_MEAN) s_up = sh_n >= 0 ? g_up / (float)sh_n : __builtin_nanf("");
    if (!ws_ok) {
      s_up = __builtin_nanf("");
      if (tid == 0) atomicOr(&a.hdr->status, 2u);
    }
    const float m2 = m * kL;
    const float msub = (m == -INFINITY) ? 0.f : m2;
#pragma unroll
    for (int j = 0; j < P; ++j) launder(v[j]);

    // ---- the owning lane takes the target logit out of its registers
    float y = 0.f;
    if (own_tid >= 0 && (__builtin_amdgcn_readfirstlane(tid) >> 6) == (own_tid >> 6)) {  // the owning wave only
      if (tid == own_tid) {
        if (own_where == 1) {
          y = hx;
          hx = -INFINITY;
        } else if (own_where == 3) {
          y = tx;
          tx = -INFINITY;
        } else {
#pragma unroll
          for (int j = 0; j < P; ++j)
            if (j == own_j) {
              y = extract<DT>(v[j], own_e);
              v[j] = with_neg_inf<DT>(v[j], own_e);
            }
        }
      }
    }

    // ---- sum of 2^(x log2e - m2) over everything but the target.
    // On the reuse path (BF16 gradients, see kReuseSA) each term, scaled by
    // 2^14, is also packed to FP16 into the registers that held the pair of
    // logits, and the gradient pass reads it back instead of recomputing it.
    // Per wave: every lane's largest term is below |s| p_max 2^-11 <= kReuseAbs, with
    // p_j <= e^(x_j - chunk max) because lse >= every chunk's max; a wave
    // holding a large softmax value keeps its logits and the exact path.
    const bool reuse_row = DT == CE_BF16 && fabsf(s_up) * L.q_o <= kReuseSA && L.q_o <= kReuseA;
    const bool big_lane = fabsf(s_up) * ex2((m_loc - m) * kL) * (1.f / 2048.f) > kReuseAbs;
    const bool reuse = reuse_row && !__any(big_lane);
    float d0 = ex2(__builtin_fmaf(hx, kL, -msub)) + ex2(__builtin_fmaf(tx, kL, -msub)), d1 = 0.f;
    if (reuse) {
      const float msc = msub - (float)kReuseShift;
      float q0 = 0.f, q1 = 0.f;
#pragma unroll
      for (int j = 0; j < P; ++j) {
        float f[E];
        unpack<DT>(v[j], f);
        const float mj = (j * T + tid < nvc) ? msc : INFINITY;  // 2^-inf = 0 for slots past the chunk
        float t[E];
#pragma unroll
        for (int e = 0; e < E; ++e) t[e] = ex2(__builtin_fmaf(f[e], kL, -mj));
#pragma unroll
        for (int e = 0; e < E; e += 2) {
          q0 += t[e];
          q1 += t[e + 1];
        }
        v[j] = pack_terms_f16<DT>(t);
      }
      d0 += (q0 + q1) * kReuseUnscale;  // exact power-of-two rescale
    } else {
#pragma unroll
      for (int j = 0; j < P; ++j) {
        float f[E];
        unpack<DT>(v[j], f);
        const float mj = (j * T + tid < nvc) ? msub : INFINITY;  // 2^-inf = 0 for slots past the chunk
#pragma unroll
        for (int e = 0; e < E; e += 2) {
          d0 += ex2(__builtin_fmaf(f[e], kL, -mj));
          d1 += ex2(__builtin_fmaf(f[e + 1], kL, -mj));
        }
      }
    }
    float d = d0 + d1;
#pragma unroll
    for (int j = 0; j < P; ++j) launder(v[j]);
    block_sum3<T>(d, y, rs, sh);
    CE_STAMP(a.phase, item, 3);

    // ---- exchange between the chunks of a split row
    float M2 = m2, D = d, Y = y, R = rs;
    if (K > 1) {
      unsigned long long* row_slots = a.slots + (size_t)r * (size_t)K * 4u;
      if (tid == 0 && withhold != ((((unsigned long long)r + 1u) << 8) | (unsigned)k)) {
        const float mine[4] = {m2, d, y, rs};
#pragma unroll
        for (int q = 0; q < 4; ++q)
          publish(row_slots + 4 * k + q, tag, __float_as_uint(mine[q]));
      }
      if (tid < 64) {
        uint32_t spins = 0;
        bool gave_up = false;
        for (int w = tid; w < 4 * K; w += 64) {
          unsigned long long val = 0ull;
          for (;;) {
            val = poll(row_slots + w);
            if ((uint32_t)(val >> 32) == tag) break;
            if (++spins > kSpinLimit) {
              gave_up = true;
              break;
            }
            __builtin_amdgcn_s_sleep(2);
          }
          xs[w] = gave_up ? __uint_as_float(0x7fc00000u) : __uint_as_float((uint32_t)val);
        }
        if (gave_up) atomicOr(&a.hdr->status, 1u);
      }
      __syncthreads();
      M2 = -INFINITY;
      for (int q = 0; q < K; ++q) M2 = fmaxf(M2, xs[4 * q]);
      D = 0.f;
      Y = 0.f;
      R = 0.f;
      for (int q = 0; q < K; ++q) {
        const float mq = xs[4 * q];
        D += (mq == -INFINITY) ? 0.f : xs[4 * q + 1] * ex2(mq - M2);
        Y += xs[4 * q + 2];
        R += xs[4 * q + 3];
      }
    }

    CE_STAMP(a.phase, item, 4);
    // ---- sum with the target term restored, lse (base 2, split into hi + lo
    // by an exact two-sum), loss
    const float e_t = tvalid ? ex2(__builtin_fmaf(Y, kL, -M2)) : 0.f;
    const float Dt = D + e_t;
    const float lgD = lg2(Dt);
    const float c_hi = M2 + lgD;
    const float bb = c_hi - M2;
    const float c_lo = (M2 - (c_hi - bb)) + (lgD - bb);
    const float lse = lse_natural(c_hi, c_lo);
    const float row_loss = tvalid && ws_ok ? row_loss_of(lse, L.q_to, Y, L.q_o, R) : __uint_as_float(0x7fc00000u);

    // ---- gradient from the registers, written over the logits.  The store
    // offsets are recomputed from an opaque copy of the thread index, so the
    // compiler does not keep the P load offsets alive through the passes.
    int tid_st = tid;
    asm volatile("" : "+v"(tid_st));
    const float s = tvalid ? s_up : __uint_as_float(0x7fc00000u);
    const float b = -s * L.q_o;
    if (reuse) {
      // p = 2^(x log2e - msub) / D * 2^(msub - M2); the registers hold that first factor times 2^14
      const float kr = s * ex2(msub - M2 - (float)kReuseShift) / Dt;
#pragma unroll
      for (int j = 0; j < P; ++j) {
        const uint32_t w[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) o[q] = pack_bf16(fma_mix_lo(w[q], kr, b), fma_mix_hi(w[q], kr, b));
        bstore16<kCacheStream>(make_uint4(o[0], o[1], o[2], o[3]), rb, (uint32_t)(j * T + tid_st) * 16u);
      }
    } else {
#pragma unroll
      for (int j = 0; j < P; ++j) {
        float f[E];
        unpack<DT>(v[j], f);
        float gr[E];
#pragma unroll
        for (int e = 0; e < E; ++e) gr[e] = __builtin_fmaf(softmax_term<DT>(f[e], c_hi, c_lo), s, b);
        bstore16<kCacheStream>(pack<DT>(gr), rb, (uint32_t)(j * T + tid_st) * 16u);
      }
    }
    if (HT) {
      bstore_elem<DT>(__builtin_fmaf(softmax_term<DT>(hx, c_hi, c_lo), s, b), rh, tid);
      bstore_elem<DT>(__builtin_fmaf(softmax_term<DT>(tx, c_hi, c_lo), s, b), rt, tid);
    }
    CE_STAMP(a.phase, item, 5);
    // target element: s (p_t - q_t), stored by the lane that just wrote its
    // vector (same-thread order keeps this store last).  Where p_t > 1/2 it is
    // s ((1 - q_t) - (1 - p_t)) with 1 - p_t = D_excl / D, so p_t near 1 does not
    // cancel; below, s ((p_t - q_o) - (q_t - q_o)) with p_t = e_t / D, so that
    // q_t and p_t both far below 1 (smoothing near 1) do not cancel either.
    if (tid == own_tid) {
      const float ex = D / Dt;
      const float g_t = s * (ex < 0.5f ? L.q_rest - ex : (e_t / Dt - L.q_o) - L.q_to);
      if (own_where == 1)
        bstore_elem<DT>(g_t, rh, tid);
      else if (own_where == 3)
        bstore_elem<DT>(g_t, rt, tid);
      else
        bstore_elem<DT>(g_t, rb, (own_j * T + tid) * E + own_e);
    }
    publish_row_loss<T>(a, tag, r, row_loss, row_first);
  }
  CE_STAMP(a.phase, item, 6);
  // one call site for both kinds of row (two inlined copies of the finish
  // measurably raised the register allocation of the whole kernel)
  if (item == last_item) {
    fused_finish<T>(a, tag, ws_ok);
    CE_STAMP(a.phase, item, 7);
  }
}

// The BF16 512 x 8 instances are held to 8 waves per SIMD (four workgroups a
// CU; FP32's reach 8 by themselves).  That spills about 35 scalar registers to
// vector lanes (the kernel needs 102 for 7 waves), and still wins: 1024 rows of 32000 columns then run in
// one resident round, 27.3-27.4 against 28.8-29.3 us, and the split rows
// that take this shape gain 1-2% (152064 columns: 818-820 against 828-829 us;
// 256000: 1,308-1,314 against 1,333-1,337).  The 256-thread instances lose
// from it (8192 rows of 128000: 668 against 654 us; 1024 of 8192: 15.5
// against 14.2) and keep the default.
template <int DT, int T, int P, bool HT>
__global__ __launch_bounds__(T)
__attribute__((amdgpu_waves_per_eu((DT == CE_BF16 && T == 512 && P == 8) ? 8 : 4, 8))) void k_fused(FusedArgs a) {
  fused_item<DT, T, P, HT, false>(a, nullptr);
}

// The shard flow in one launch: each shard's piece of a row is read once
// into registers, the shards exchange (max, sum-exp, target logit, row sum)
// through the workspace's tagged words like the chunks of a split row, and
// each writes its gradient in place.  Shards may start and end anywhere, so
// head and tail elements are always handled.
template <int DT, int T, int P>
__global__ __launch_bounds__(T) __attribute__((amdgpu_waves_per_eu(4, 8))) void k_fused_shards(FusedArgs a,
                                                                                                ShardSet ss) {
  fused_item<DT, T, P, true, true>(a, &ss);
}

// --------------------------------------------------------------------------
// The natural lse c / kL of a base-2 log-sum-exp c = c_hi + c_lo, split into
// its FP32 rounding and the residual: lse_hi + lse_lo carries the sum's own
// precision, and the separate backward rebuilds c from the pair.
__device__ __forceinline__ void lse_pair(float c_hi, float c_lo, float* lse_hi, float* lse_lo) {
  const float hi = lse_natural(c_hi, c_lo);
  // c - hi kL: hi kL is within an ulp of c_hi, so the fma's difference is exact
  const float rc = __builtin_fmaf(-hi, kL, c_hi) + c_lo;
  *lse_hi = hi;
  *lse_lo = rc * kLn2;  // rc / kL to far below the FP32 rounding of lse
}

// Streaming statistics of whole rows (forward) or of shard rows.  Each thread
// keeps an online (max, sum) pair, rescaled once per batch of PB vectors.  The
// max covers every column; the sum leaves out the row's target (its lane sets
// its register copy to -inf after the batch's max), so that 1 - p_t = d / (d +
// e^(x_t - m)) keeps its digits when the target holds nearly all the
// probability; the forward restores the term from the target logit, the
// shard statistics leave it to the combine.
template <int DT, int T>
__device__ void stats_short_row(const StatsArgs& a, int64_t r, const Row<DT>& g, bool tvalid, bool owns, int64_t tl) {
  const int lane = threadIdx.x;
  const RowLayout& L = a.L;
  const Rsrc rx = make_rsrc(g.base, L.V * ElemT<DT>::EB);
  const bool in0 = lane < L.V, in1 = lane + 64 < L.V;
  const double x0 = (double)bload_elem<DT>(rx, lane), x1 = (double)bload_elem<DT>(rx, lane + 64);
  const Stats64 st = wave_stats64(x0, in0, x1, in1, owns ? tl : -1);
  if (lane != 0) return;
  if (a.mode == kStatsForward) {
    const double D = st.d + (st.y == -INFINITY ? 0.0 : exp(st.y - st.m));
    const double lse = st.m + log(D);
    const double loss = row_loss64(lse, a.q_o_d, a.q_t_d, st.y, st.r);
    const float lse_hi = (float)lse;
    a.row_loss[r] = tvalid ? (float)loss : __uint_as_float(0x7fc00000u);
    if (a.lse) a.lse[r] = tvalid ? lse_hi : __uint_as_float(0x7fc00000u);
    if (a.lse_aux)
      reinterpret_cast<float2*>(a.lse_aux)[r] =
          tvalid ? make_float2((float)(lse - (double)lse_hi), (float)(st.d / D)) : make_float2(NAN, NAN);
  } else {
    reinterpret_cast<float4*>(a.stats)[r] = make_float4((float)st.m, (float)st.d, (float)st.y, (float)st.r);
  }
}

template <int DT, int T, int PB>
__global__ __launch_bounds__(T) void k_stats(StatsArgs a) {
  constexpr int E = ElemT<DT>::E, EB = ElemT<DT>::EB;
  __shared__ float sh[T / 64][4];
  const int tid = threadIdx.x;
  const RowLayout& L = a.L;
  if (blockIdx.x == 0 && a.n_out) {
    const int32_t n = block_count_targets<T>(L.tgt, L.ts0, L.ts1, L.d1, L.N, L.ignore_idx);
    if (tid == 0) a.n_out[0] = n;
  }
  for (int64_t r = blockIdx.x; r < L.N; r += gridDim.x) {
    CE_STAMP(a.phase, r, 0);
    const Row<DT> g = row_geometry<DT>(L, r);
    if (g.t == L.ignore_idx) {
      if (tid == 0) {
        if (a.mode == kStatsForward) {
          a.row_loss[r] = 0.f;
          if (a.lse) a.lse[r] = 0.f;
          if (a.lse_aux) reinterpret_cast<float2*>(a.lse_aux)[r] = make_float2(0.f, 0.f);
        } else {
          reinterpret_cast<float4*>(a.stats)[r] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
      }
      continue;
    }
    const bool tvalid = g.t >= 0 && g.t < L.vocab_total;
    const int64_t tl = g.t - L.vocab_start;
    const bool owns = tvalid && tl >= 0 && tl < L.V;
    if constexpr (T == kShortT && PB == kShortPB) {  // the instance rows of at most kShortRow columns get
      if (a.short_rows) {  // whole rows of at most kShortRow columns: wave 0, FP64
        if (tid < 64) stats_short_row<DT, T>(a, r, g, tvalid, owns, tl);
        continue;
      }
    }
    const Rsrc rb = make_rsrc(g.body, g.nv * 16);
    const Rsrc rh = make_rsrc(g.base, g.h * EB);
    const Rsrc rt = make_rsrc(g.tail, (int64_t)g.tn * EB);
    const Rsrc ry = make_rsrc(g.base, owns && tid == 0 ? L.V * EB : 0);
    float y = bload_elem<DT>(ry, owns ? (int)tl : 0);
    const bool hv = tid < g.h, tv = tid < g.tn;
    float hx = bload_elem<DT>(rh, tid);
    float tx = bload_elem<DT>(rt, tid);
    hx = hv ? hx : -INFINITY;
    tx = tv ? tx : -INFINITY;
    float m = fmaxf(hx, tx);
    float m2 = m * kL;
    float msub = (m == -INFINITY) ? 0.f : m2;
    float rs = (hv ? hx : 0.f) + (tv ? tx : 0.f);
    // the target's place in the row: head lane, body vector (element te) or tail lane
    int64_t tvec = -1;
    int te = 0;
    if (owns) {
      if (tl < g.h) {
        if (tid == tl) hx = -INFINITY;
      } else if (tl - g.h < g.nv * E) {
        tvec = (tl - g.h) / E;
        te = (int)(tl - g.h - tvec * E);
      } else if (tid == tl - g.h - g.nv * E) {
        tx = -INFINITY;
      }
    }
    float d = ex2(__builtin_fmaf(hx, kL, -msub)) + ex2(__builtin_fmaf(tx, kL, -msub));
    for (int64_t base = 0; base < g.nv; base += (int64_t)T * PB) {
      uint4 v[PB];
#pragma unroll
      for (int j = 0; j < PB; ++j) v[j] = bload16<kCacheStream>(rb, (uint32_t)(base + j * T + tid) * 16u);
      if (base == 0) CE_STAMP(a.phase, r, 1);
      float bm = -INFINITY;
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        const float mj = vec_max<DT>(v[j], bm);
        bm = (base + j * T + tid < g.nv) ? mj : bm;
        rs += vec_sum<DT>(v[j]);  // zeros past the row
      }
      if (bm > m) {
        const float bm2 = bm * kL;
        d *= ex2(m2 - bm2);
        m = bm;
        m2 = bm2;
        msub = m2;
      }
      // The sum pass unpacks again rather than keep the max pass's floats: 96 instead of 130-137
      // VGPRs, two 512-thread workgroups a CU instead of one (8192 rows of 128000 BF16 columns:
      // 303-305 against 366-373 us).
#pragma unroll
      for (int j = 0; j < PB; ++j) launder(v[j]);
      // the batch holding the target vector (uniform test): its lane drops the target from the sum
      const int64_t tq = tvec - base;
      if (tq >= 0 && tq < (int64_t)T * PB) {
        const int own_j = (int)(tq / T);
        if (tid == (int)(tq - (int64_t)own_j * T)) {
#pragma unroll
          for (int j = 0; j < PB; ++j)
            if (j == own_j) v[j] = with_neg_inf<DT>(v[j], te);
        }
      }
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        float f[E];
        unpack<DT>(v[j], f);
        const float mj = (base + j * T + tid < g.nv) ? msub : INFINITY;
#pragma unroll
        for (int e = 0; e < E; ++e) d += ex2(__builtin_fmaf(f[e], kL, -mj));
      }
    }
    const float M = block_max<T>(m, sh);
    CE_STAMP(a.phase, r, 2);
    const float M2 = M * kL;
    float dadj = (m == -INFINITY) ? 0.f : d * ex2(m2 - M2);
    block_sum3<T>(dadj, y, rs, sh);
    if (tid == 0) {
      if (a.mode == kStatsForward) {
        // the target's term restored: D = d_excl + 2^(y log2e - M2)
        const float e_t = (owns && y != -INFINITY) ? ex2(__builtin_fmaf(y, kL, -M2)) : 0.f;
        const float Dt = dadj + e_t;
        const float lgD = lg2(Dt);
        const float c_hi = M2 + lgD;
        const float bb = c_hi - M2;
        const float c_lo = (M2 - (c_hi - bb)) + (lgD - bb);
        float lse, lse_lo;
        lse_pair(c_hi, c_lo, &lse, &lse_lo);
        const float loss = row_loss_of(lse, L.q_to, y, L.q_o, rs);
        a.row_loss[r] = tvalid ? loss : __uint_as_float(0x7fc00000u);
        if (a.lse) a.lse[r] = tvalid ? lse : __uint_as_float(0x7fc00000u);
        if (a.lse_aux)
          reinterpret_cast<float2*>(a.lse_aux)[r] = tvalid ? make_float2(lse_lo, dadj / Dt) : make_float2(NAN, NAN);
      } else {
        // natural-units sum: sum exp(x - M) = dadj * 2^(M2 - M log2e)
        const float dn = (M == -INFINITY) ? 0.f : dadj * ex2(-__builtin_fmaf(M, kL, -M2));
        reinterpret_cast<float4*>(a.stats)[r] = make_float4(M, dn, y, rs);
      }
    }
    CE_STAMP(a.phase, r, 3);
  }
}

// --------------------------------------------------------------------------
// Streaming in-place backward from the forward's hand-off; works on shards.
// With lse_aux the row's lse is the pair lse + lse_aux[r][0] and its target
// gradient takes the fused kernel's form: s ((1 - q_t) - (1 - p_t)) from the
// handed-over 1 - p_t = lse_aux[r][1] where that is below 1/2, else
// s ((p_t - q_o) - (q_t - q_o)).  With the lse alone, 1 - p_t comes from
// expm1(x_t - lse) instead, resolved only to the FP32 lse's own precision.
// Unsharded rows of at most kShortRow columns are recomputed whole by one
// wave in FP64 (the fused kernel's short-row arithmetic); lse is not read.
// A workgroup takes one item: batch k (T x PB body vectors) of row r, item
// r K + k, so that a long row's batches run in K workgroups at once rather
// than one after another in one (8192 rows of 128000 BF16 columns, K = 4:
// 670-678 against 734-739 us); chunk 0 also takes the row's head and tail.
template <int DT, int T, int PB>
__global__ __launch_bounds__(T) void k_backward(BackwardArgs a) {
  constexpr int E = ElemT<DT>::E, EB = ElemT<DT>::EB;
  const int tid = threadIdx.x;
  const RowLayout& L = a.L;
  const int64_t K = a.K, items = L.N * K;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int64_t r = it / K, k = it - r * K;
    const Row<DT> g = row_geometry<DT>(L, r);
    const int64_t cb = k * (int64_t)(T * PB);  // this item's first body vector
    const int64_t ce = g.nv < cb + T * PB ? g.nv : cb + T * PB;
    if (g.t == L.ignore_idx) {
      const uint4 z = make_uint4(0u, 0u, 0u, 0u);
      for (int64_t i = cb + tid; i < ce; i += T) g.body[i] = z;
      if (k == 0 && tid < g.h) store_elem<DT>(g.base, tid, 0.f);
      if (k == 0 && tid < g.tn) store_elem<DT>(g.tail, tid, 0.f);
      continue;
    }
    const bool tvalid = g.t >= 0 && g.t < L.vocab_total;
    const int64_t tl = tvalid ? g.t - L.vocab_start : -1;  // may fall outside this shard
    float s = grad_scale(a.reduce, a.g, a.n_valid, r);
    if (!tvalid) s = __uint_as_float(0x7fc00000u);
    if (T == kShortT && PB == kShortPB && a.short_rows) {  // the instance rows of at most kShortRow columns get
      // one wave, two columns per lane, FP64: the whole row recomputed (unsharded), or the shard's
      // columns from the handed-over lse (a vocabulary of at most kShortRow columns)
      if (tid < 64) {
        const Rsrc rx = make_rsrc(g.base, L.V * EB);
        const bool in0 = tid < L.V, in1 = tid + 64 < L.V;
        const double x0 = (double)bload_elem<DT>(rx, tid), x1 = (double)bload_elem<DT>(rx, tid + 64);
        double lse;
        float rest = 2.f;  // 1 - p_t from the hand-off (2: not given)
        if (a.short_rows == kShortRecompute) {
          lse = lse_of64(wave_stats64(x0, in0, x1, in1, tl));
        } else {
          const float2 aux = a.lse_aux ? reinterpret_cast<const float2*>(a.lse_aux)[r] : make_float2(0.f, 2.f);
          lse = (double)a.lse[r] + (double)aux.x;
          rest = aux.y;
        }
        const double sd = a.reduce == CE_REDUCE_MEAN ? (a.g ? (double)a.g[0] : 1.0) / (double)(*a.n_valid) : (double)s;
        // s (p - q); at a target holding more than half the probability, s ((1 - q_t) - (1 - p_t)) from the
        // handed-over 1 - p_t, which keeps the digits that p_t - 1 would lose
        auto grad64 = [&](double x, int64_t col) {
          if (col != tl) return sd * (exp(x - lse) - a.q_o_d);
          return rest < 0.5f ? sd * ((1.0 - a.q_t_d) - (double)rest) : sd * (exp(x - lse) - a.q_t_d);
        };
        bstore_elem<DT>(tvalid ? (float)grad64(x0, tid) : s, rx, tid);
        bstore_elem<DT>(tvalid ? (float)grad64(x1, tid + 64) : s, rx, tid + 64);
      }
      continue;
    }
    const float lse = a.lse[r];
    float2 aux = make_float2(0.f, 2.f);  // no hand-off: 1 - p_t unknown (never below 1/2)
    if (a.lse_aux) aux = reinterpret_cast<const float2*>(a.lse_aux)[r];
    const float c_hi = lse * kL;
    const float c_lo = __builtin_fmaf(lse, kL, -c_hi) + aux.x * kL;
    const float b = -s * L.q_o;
    // target: s (p_t - q_t) without subtracting numbers near 1 (see above)
    auto target_grad = [&](float x, float p) {
      if (a.lse_aux) return s * (aux.y < 0.5f ? L.q_rest - aux.y : (p - L.q_o) - L.q_to);
      return s * (p > 0.5f ? expm1f(x - lse) + L.q_rest : (p - L.q_o) - L.q_to);
    };
    const Rsrc rb = make_rsrc(g.body, g.nv * 16);
    const Rsrc rh = make_rsrc(g.base, k == 0 ? g.h * EB : 0);
    const Rsrc rt = make_rsrc(g.tail, k == 0 ? (int64_t)g.tn * EB : 0);
    {
      // head and tail elements, chunk 0 (range-checked: lanes past them, and other chunks, do nothing)
      const float hx = bload_elem<DT>(rh, tid);
      const float tx = bload_elem<DT>(rt, tid);
      const float ph = ex2(__builtin_fmaf(hx, kL, -c_hi) - c_lo), pt = ex2(__builtin_fmaf(tx, kL, -c_hi) - c_lo);
      float gh = __builtin_fmaf(ph, s, b);
      float gt = __builtin_fmaf(pt, s, b);
      if (tl == tid) gh = target_grad(hx, ph);
      if (tl == g.h + g.nv * E + tid) gt = target_grad(tx, pt);
      bstore_elem<DT>(gh, rh, tid);
      bstore_elem<DT>(gt, rt, tid);
    }
    for (int64_t base = cb; base < ce; base += (int64_t)T * PB) {  // one batch
      uint4 v[PB];
#pragma unroll
      for (int j = 0; j < PB; ++j) v[j] = bload16<kCacheStream>(rb, (uint32_t)(base + j * T + tid) * 16u);
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        const int64_t i = base + j * T + tid;
        float f[E];
        unpack<DT>(v[j], f);
        float pr[E], gr[E];
#pragma unroll
        for (int e = 0; e < E; ++e) {
          pr[e] = ex2(__builtin_fmaf(f[e], kL, -c_hi) - c_lo);
          gr[e] = __builtin_fmaf(pr[e], s, b);
        }
        const uint64_t off = (uint64_t)(tl - (g.h + i * E));
        if (off < (uint64_t)E) {
#pragma unroll
          for (int e = 0; e < E; ++e) gr[e] = (e == (int)off) ? target_grad(f[e], pr[e]) : gr[e];
        }
        bstore16<kCacheStream>(pack<DT>(gr), rb, (uint32_t)i * 16u);  // dropped past the row
      }
    }
  }
}

// --------------------------------------------------------------------------
// Combine of S shards' (m, d, y, r): one thread per row, shards in order.
// Each d leaves out the row's target (only its owner holds it); the combine
// restores that term from the gathered target logit:
//   M = max_s m_s, D_excl = sum_s d_s e^(m_s - M), D = D_excl + e^(x_t - M),
//   lse = M + log D, 1 - p_t = D_excl / D,
// in FP64 and rounded once: the backward rebuilds every p_j from lse (and the
// residual lse_aux[r][0]), and with few columns (p_j large) each FP32 rounding
// along the way would show in the gradient.
__global__ __launch_bounds__(256) void k_combine(CombineArgs a) {
  if (blockIdx.x == 0 && a.n_out) {
    const int32_t n = block_count_targets<256>(a.tgt, a.ts0, a.ts1, a.d1, a.N, a.ignore_idx);
    if (threadIdx.x == 0) a.n_out[0] = n;
  }
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= a.N) return;
  const int64_t i0 = r / a.d1, i1 = r - i0 * a.d1;
  const int64_t t = a.tgt[i0 * a.ts0 + i1 * a.ts1];
  if (t == a.ignore_idx) {
    a.row_loss[r] = 0.f;
    if (a.lse) a.lse[r] = 0.f;
    if (a.lse_aux) reinterpret_cast<float2*>(a.lse_aux)[r] = make_float2(0.f, 0.f);
    return;
  }
  const float4* st = reinterpret_cast<const float4*>(a.stats);
  double M = -INFINITY;
  for (int s = 0; s < a.S; ++s) M = fmax(M, (double)st[(int64_t)s * a.N + r].x);
  double Dx = 0.0, Y = 0.0, R = 0.0;
  for (int s = 0; s < a.S; ++s) {
    const float4 q = st[(int64_t)s * a.N + r];
    Dx += (q.x == -INFINITY) ? 0.0 : (double)q.y * exp((double)q.x - M);
    Y += (double)q.z;
    R += (double)q.w;
  }
  const double D = Dx + (Y == -INFINITY ? 0.0 : exp(Y - M));
  const double lse = M + log(D);
  const float lse_hi = (float)lse;
  const bool tvalid = t >= 0 && t < a.vocab_total;
  const float nan = __uint_as_float(0x7fc00000u);
  a.row_loss[r] = tvalid ? (float)row_loss64(lse, a.q_o_d, a.q_t_d, Y, R) : nan;
  if (a.lse) a.lse[r] = tvalid ? lse_hi : nan;
  if (a.lse_aux)
    reinterpret_cast<float2*>(a.lse_aux)[r] =
        tvalid ? make_float2((float)(lse - (double)lse_hi), (float)(Dx / D)) : make_float2(nan, nan);
}

// --------------------------------------------------------------------------
// Mean over non-ignored rows (or the plain sum when n_valid is NULL): sum of
// per-row losses in FP64, fixed order.
__global__ __launch_bounds__(1024) void k_mean(const float* row_loss, int64_t N, const int32_t* n_valid, float* out) {
  __shared__ double sh[16];
  double s = 0.0;
#pragma unroll 8
  for (int64_t i = threadIdx.x; i < N; i += 1024) s += (double)row_loss[i];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
    for (int i = 0; i < 16; ++i) tot += sh[i];
    out[0] = n_valid ? (float)(tot / (double)(*n_valid)) : (float)tot;  // n = 0 gives 0/0 = NaN
  }
}

template <int DT, int T, int P>
hipError_t launch_fused_t(const FusedArgs& a, int64_t grid, hipStream_t stream) {
  if (a.aligned)
    hipLaunchKernelGGL((k_fused<DT, T, P, false>), dim3((uint32_t)grid), dim3(T), 0, stream, a);
  else
    hipLaunchKernelGGL((k_fused<DT, T, P, true>), dim3((uint32_t)grid), dim3(T), 0, stream, a);
  return hipGetLastError();
}

template <int DT>
hipError_t launch_fused_dt(const FusedArgs& a, FusedShape shape, int64_t grid, hipStream_t stream) {
  if (shape.threads == 1024 && shape.vecs == 16) return launch_fused_t<DT, 1024, 16>(a, grid, stream);
  if (shape.threads == 512 && shape.vecs == 16) return launch_fused_t<DT, 512, 16>(a, grid, stream);
  if (shape.threads == 512 && shape.vecs == 8) return launch_fused_t<DT, 512, 8>(a, grid, stream);
  if (shape.threads == 256) {
    switch (shape.vecs) {
      case 1: return launch_fused_t<DT, 256, 1>(a, grid, stream);
      case 2: return launch_fused_t<DT, 256, 2>(a, grid, stream);
      case 4: return launch_fused_t<DT, 256, 4>(a, grid, stream);
      case 8: return launch_fused_t<DT, 256, 8>(a, grid, stream);
      default: break;
    }
  }
  return hipErrorInvalidValue;
}

template <int DT>
hipError_t launch_fused_shards_dt(const FusedArgs& a, const ShardSet& ss, FusedShape shape, int64_t grid,
                                  hipStream_t stream) {
  const dim3 g((uint32_t)grid);
  if (shape.threads == 512 && shape.vecs == 8)
    hipLaunchKernelGGL((k_fused_shards<DT, 512, 8>), g, dim3(512), 0, stream, a, ss);
  else if (shape.threads == 256 && shape.vecs == 8)
    hipLaunchKernelGGL((k_fused_shards<DT, 256, 8>), g, dim3(256), 0, stream, a, ss);
  else if (shape.threads == 256 && shape.vecs == 4)
    hipLaunchKernelGGL((k_fused_shards<DT, 256, 4>), g, dim3(256), 0, stream, a, ss);
  else if (shape.threads == 256 && shape.vecs == 2)
    hipLaunchKernelGGL((k_fused_shards<DT, 256, 2>), g, dim3(256), 0, stream, a, ss);
  else if (shape.threads == 256 && shape.vecs == 1)
    hipLaunchKernelGGL((k_fused_shards<DT, 256, 1>), g, dim3(256), 0, stream, a, ss);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

constexpr int kStreamT = 256;   // k_scale: threads per row
constexpr int kStreamPB = 4;    //          16-byte vectors per thread per batch
// Long rows: k_stats reads 512 threads x 8 vectors per batch, k_backward
// 1024 x 4; on 8192 rows of 128000 BF16 columns these measured 365-370 us
// (5.7 TB/s read) and 718-723 us (5.8 TB/s read + write), against 396 and
// 773 us at 256 x 4.  (k_stats keeps the max pass's unpacked floats for the
// sum pass, 126 VGPRs; a register barrier that re-unpacks instead, 85 VGPRs,
// measured slower.)  Rows of at most 1024 or 2048 vectors take a workgroup
// whose batch they fill.
int row_vectors(const RowLayout& L) { return (int)((L.V * (L.dtype == CE_BF16 ? 2 : 4) + 15) / 16); }

int64_t stream_grid(int64_t N) { return N < (1 << 20) ? N : (1 << 20); }

}  // namespace

// Shapes available to the fused kernel, smallest capacity first.
// (512, 8) covers 2049..4096 vectors with 8 waves a workgroup (56 VGPRs; for
// BF16 held to 8 waves per SIMD, see k_fused), which measured faster than
// (256, 16) (90 VGPRs, 5 waves per SIMD).
static const FusedShape kShapes[] = {{256, 1}, {256, 2}, {256, 4}, {256, 8}, {512, 8}, {512, 16}, {1024, 16}};

FusedShape fused_shape_for(int64_t vecs) {
  for (const FusedShape& s : kShapes)
    if ((int64_t)s.threads * s.vecs >= vecs) return s;
  return FusedShape{0, 0};
}

int64_t max_body_vecs(int32_t dtype, int64_t V) { return V / (dtype == CE_BF16 ? 8 : 4); }

// Rows of up to 4096 vectors stay whole.  Longer rows are split into K
// chunks held by 256 x 8 (2048 vectors) or 512 x 8 (4096 vectors)
// workgroups; K is the one between ceil(nv / 4096) and ceil(nv / 2048) whose
// chunks fill their workgroup's registers best.  How full the registers are
// matters most (8192 BF16 rows of 100000 columns: 7 chunks at 87% beat 4 at
// 76% by 8%).  Between options within 1% of each other, BF16 takes the
// 256-thread chunks as long as K stays at most 8, FP32 the fewer chunks.
// BF16 needs 102 scalar registers, 7 waves per SIMD: seven 4-wave workgroups
// a CU fill them, where 8-wave workgroups run three a CU, or four held to 8
// waves with spilled scalars; either way the smaller chunks won (128000
// columns: 8 chunks 653 against 4 at 673 us at three a CU and 679 at four;
// 65536: 4 at 357-363 against 2 at 385-387 and 397).  FP32's 512 x 8
// instance runs 8 waves per SIMD by itself and gains nothing from the smaller
// shape (128000 FP32: 8 chunks 1,279 against 16 at 1,328).  Past 8 chunks
// the exchange, where every chunk reads all of its partners' words, costs
// more than the slots gain (256000 BF16: 8 chunks 1,318 against 16 at
// 1,338-1,342).
int32_t fused_auto_chunks(int32_t dtype, int64_t V) {
  const int64_t nv = max_body_vecs(dtype, V);
  if (nv <= 4096) return 1;
  int64_t best_k = (nv + 4095) / 4096;
  double best_fill = 0.0;
  for (int64_t k = (nv + 4095) / 4096; k <= (nv + 2047) / 2048; ++k) {
    const int64_t c = (nv + k - 1) / k;
    const double fill = (double)c / (c <= 2048 ? 2048.0 : 4096.0);
    const bool tie_to_more = dtype == CE_BF16 && k <= 8 && c <= 2048 && fill >= best_fill - 0.01;
    if (fill > best_fill + 0.01 || tie_to_more) {
      best_fill = fill > best_fill ? fill : best_fill;
      best_k = k;
    }
  }
  return (int32_t)best_k;
}

hipError_t launch_zero_count(int32_t* n_out, hipStream_t stream) {
  hipLaunchKernelGGL(k_zero_count, dim3(1), dim3(64), 0, stream, n_out);
  return hipGetLastError();
}

hipError_t launch_fused(const FusedArgs& a, FusedShape shape, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  const int64_t grid = a.L.N * a.K;
  if (grid == 0) return hipSuccess;
  hipError_t e = hipSuccess;
  if (ev0 && (e = hipEventRecord(ev0, stream)) != hipSuccess) return e;
  e = (a.L.dtype == CE_BF16) ? launch_fused_dt<CE_BF16>(a, shape, grid, stream)
                             : launch_fused_dt<CE_F32>(a, shape, grid, stream);
  if (e != hipSuccess) return e;
  if (ev1) e = hipEventRecord(ev1, stream);
  return e;
}

hipError_t launch_fused_shards(const FusedArgs& a, const ShardSet& ss, FusedShape shape, hipStream_t stream,
                               hipEvent_t ev0, hipEvent_t ev1) {
  const int64_t grid = a.L.N * a.K;
  if (grid == 0) return hipSuccess;
  hipError_t e = hipSuccess;
  if (ev0 && (e = hipEventRecord(ev0, stream)) != hipSuccess) return e;
  e = (a.L.dtype == CE_BF16) ? launch_fused_shards_dt<CE_BF16>(a, ss, shape, grid, stream)
                             : launch_fused_shards_dt<CE_F32>(a, ss, shape, grid, stream);
  if (e != hipSuccess) return e;
  if (ev1) e = hipEventRecord(ev1, stream);
  return e;
}

hipError_t launch_stats(const StatsArgs& a, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  if (a.L.N == 0) return hipSuccess;
  hipError_t e = hipSuccess;
  if (ev0 && (e = hipEventRecord(ev0, stream)) != hipSuccess) return e;
  const dim3 grid((uint32_t)stream_grid(a.L.N));
  const int nv = row_vectors(a.L);
  if (a.L.dtype == CE_BF16) {
    if (nv <= 1024)
      hipLaunchKernelGGL((k_stats<CE_BF16, kShortT, kShortPB>), grid, dim3(kShortT), 0, stream, a);
    else if (nv <= 2048)
      hipLaunchKernelGGL((k_stats<CE_BF16, 256, 8>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((k_stats<CE_BF16, 512, 8>), grid, dim3(512), 0, stream, a);
  } else {
    if (nv <= 1024)
      hipLaunchKernelGGL((k_stats<CE_F32, kShortT, kShortPB>), grid, dim3(kShortT), 0, stream, a);
    else if (nv <= 2048)
      hipLaunchKernelGGL((k_stats<CE_F32, 256, 8>), grid, dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((k_stats<CE_F32, 512, 8>), grid, dim3(512), 0, stream, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev1) e = hipEventRecord(ev1, stream);
  return e;
}

hipError_t launch_backward(const BackwardArgs& args, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  if (args.L.N == 0) return hipSuccess;
  hipError_t e = hipSuccess;
  if (ev0 && (e = hipEventRecord(ev0, stream)) != hipSuccess) return e;
  BackwardArgs a = args;
  const int nv = row_vectors(a.L);
  // rows of more than 2048 vectors: items of 1024 x 4 vectors; shorter rows fit one batch
  a.K = nv <= 2048 ? 1 : (int32_t)((nv + 4095) / 4096);
  const dim3 grid((uint32_t)stream_grid(a.L.N * a.K));
  if (a.L.dtype == CE_BF16) {
    if (nv <= 1024)
      hipLaunchKernelGGL((k_backward<CE_BF16, kShortT, kShortPB>), grid, dim3(kShortT), 0, stream, a);
    else if (nv <= 2048)
      hipLaunchKernelGGL((k_backward<CE_BF16, 512, 4>), grid, dim3(512), 0, stream, a);
    else
      hipLaunchKernelGGL((k_backward<CE_BF16, 1024, 4>), grid, dim3(1024), 0, stream, a);
  } else {
    if (nv <= 1024)
      hipLaunchKernelGGL((k_backward<CE_F32, kShortT, kShortPB>), grid, dim3(kShortT), 0, stream, a);
    else if (nv <= 2048)
      hipLaunchKernelGGL((k_backward<CE_F32, 512, 4>), grid, dim3(512), 0, stream, a);
    else
      hipLaunchKernelGGL((k_backward<CE_F32, 1024, 4>), grid, dim3(1024), 0, stream, a);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev1) e = hipEventRecord(ev1, stream);
  return e;
}

hipError_t launch_combine(const CombineArgs& a, hipStream_t stream) {
  if (a.N == 0) return hipSuccess;
  hipLaunchKernelGGL(k_combine, dim3((uint32_t)((a.N + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// A staged gradient (written for an upstream gradient of 1) scaled in place
// by the upstream gradient once it is known: row r by g[r] (per_row) or all
// rows by g[0].  A row whose factor is exactly 1 is neither read nor written;
// zeros stay +0.0 (ignored rows keep their bit pattern for any factor).
template <int DT, int T, int PB>
__global__ __launch_bounds__(T) void k_scale(ScaleArgs a) {
  constexpr int E = ElemT<DT>::E, EB = ElemT<DT>::EB;
  const int tid = threadIdx.x;
  const RowLayout& L = a.L;
  for (int64_t r = blockIdx.x; r < L.N; r += gridDim.x) {
    const float s = a.per_row ? a.g[r] : a.g[0];
    if (s == 1.f) continue;
    const Row<DT> g = row_span<DT>(L, r);
    const Rsrc rb = make_rsrc(g.body, g.nv * 16);
    const Rsrc rh = make_rsrc(g.base, g.h * EB);
    const Rsrc rt = make_rsrc(g.tail, (int64_t)g.tn * EB);
    {
      const float hx = bload_elem<DT>(rh, tid), tx = bload_elem<DT>(rt, tid);
      bstore_elem<DT>(hx == 0.f ? 0.f : hx * s, rh, tid);  // lanes past the head or tail: dropped
      bstore_elem<DT>(tx == 0.f ? 0.f : tx * s, rt, tid);
    }
    for (int64_t base = 0; base < g.nv; base += (int64_t)T * PB) {
      uint4 v[PB];
#pragma unroll
      for (int j = 0; j < PB; ++j) v[j] = bload16(rb, (uint32_t)(base + j * T + tid) * 16u);
#pragma unroll
      for (int j = 0; j < PB; ++j) {
        float f[E];
        unpack<DT>(v[j], f);
#pragma unroll
        for (int e = 0; e < E; ++e) f[e] = f[e] == 0.f ? 0.f : f[e] * s;
        bstore16(pack<DT>(f), rb, (uint32_t)(base + j * T + tid) * 16u);  // dropped past the row
      }
    }
  }
}

// Workspace initialisation: every word zero except the header's magic,
// initialised size and epoch (1) (each word written once with its final value, so no two
// threads race on one word).  A fill kernel, not hipMemsetAsync, so that it
// can sit in a captured graph.
__global__ __launch_bounds__(1024) void k_ws_init(unsigned long long* p, int64_t nwords, unsigned long long bytes) {
  const int64_t stride = (int64_t)gridDim.x * 1024;
  for (int64_t i = (int64_t)blockIdx.x * 1024 + threadIdx.x; i < nwords; i += stride)
    p[i] = i == 1 ? kWsMagic : (i == 2 ? bytes : (i == 3 ? 1ull : 0ull));
}

hipError_t launch_ws_init(void* ws, size_t bytes, hipStream_t stream) {
  const int64_t nwords = (int64_t)(bytes / 8u);
  int64_t blocks = (nwords + 1023) / 1024;
  if (blocks > 2048) blocks = 2048;
  hipLaunchKernelGGL(k_ws_init, dim3((uint32_t)blocks), dim3(1024), 0, stream, static_cast<unsigned long long*>(ws),
                     nwords, (unsigned long long)bytes);
  return hipGetLastError();
}

// --------------------------------------------------------------------------
// The allocation-free fused call's workspace.  In host code `scratch` is only
// a stand-in for the symbol: its device address comes from
// hipGetSymbolAddress, per device, and host code passes that address, never
// the name.  Calls that use it on one device share it (and race if they
// overlap); each keeps the tagged-word protocol of a prepared workspace, so
// nothing needs clearing between calls.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t static_scratch(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    // the preparation must run once, not on every replay of a captured graph
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if ((e = hipStreamIsCapturing(stream, &cs)) != hipSuccess) return e;
    if (cs != hipStreamCaptureStatusNone) return hipErrorStreamCaptureUnsupported;
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    if ((e = launch_ws_init(p, kStaticScratchBytes, stream)) != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_scale(const ScaleArgs& a, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1) {
  if (a.L.N == 0) return hipSuccess;
  hipError_t e = hipSuccess;
  if (ev0 && (e = hipEventRecord(ev0, stream)) != hipSuccess) return e;
  const dim3 grid((uint32_t)stream_grid(a.L.N));
  if (a.L.dtype == CE_BF16)
    hipLaunchKernelGGL((k_scale<CE_BF16, kStreamT, kStreamPB>), grid, dim3(kStreamT), 0, stream, a);
  else
    hipLaunchKernelGGL((k_scale<CE_F32, kStreamT, kStreamPB>), grid, dim3(kStreamT), 0, stream, a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (ev1) e = hipEventRecord(ev1, stream);
  return e;
}

// --------------------------------------------------------------------------
// Chunked linear + cross-entropy: the count over all rows (and the mean's
// scale g / n, the upstream gradient every chunk's fused call then takes),
// and the loss from the chunks' sums.
__global__ __launch_bounds__(1024) void k_linear_prep(const int64_t* tgt, int64_t ts, int64_t N, int64_t ignore_idx,
                                                      int32_t reduce, const float* g, int32_t* n_out, float* scale) {
  const int32_t n = block_count_targets<1024>(tgt, 0, ts, N > 0 ? N : 1, N, ignore_idx);
  if (threadIdx.x == 0) {
    n_out[0] = n;
    if (reduce == CE_REDUCE_MEAN) scale[0] = (g ? g[0] : 1.f) / (float)n;
  }
}

__global__ __launch_bounds__(64) void k_linear_finish(const float* parts, int64_t nparts, int32_t reduce,
                                                      const int32_t* n, float* out) {
  if (threadIdx.x != 0) return;
  double tot = 0.0;
  for (int64_t i = 0; i < nparts; ++i) tot += (double)parts[i];
  out[0] = reduce == CE_REDUCE_MEAN ? (float)(tot / (double)n[0]) : (float)tot;  // n = 0: 0/0 = NaN
}

__global__ __launch_bounds__(256) void k_fill_f32(float* p, int64_t rows, int64_t cols, int64_t ld) {
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x)
    for (int64_t j = threadIdx.x; j < cols; j += 256) p[r * ld + j] = 0.f;
}

hipError_t launch_linear_prep(const int64_t* tgt, int64_t ts, int64_t N, int64_t ignore_idx, int32_t reduce,
                              const float* g, int32_t* n_out, float* scale, hipStream_t stream) {
  hipLaunchKernelGGL(k_linear_prep, dim3(1), dim3(1024), 0, stream, tgt, ts, N, ignore_idx, reduce, g, n_out, scale);
  return hipGetLastError();
}

hipError_t launch_linear_finish(const float* parts, int64_t nparts, int32_t reduce, const int32_t* n, float* out,
                                hipStream_t stream) {
  hipLaunchKernelGGL(k_linear_finish, dim3(1), dim3(64), 0, stream, parts, nparts, reduce, n, out);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, int64_t rows, int64_t cols, int64_t ld, hipStream_t stream) {
  if (rows == 0) return hipSuccess;
  const int64_t grid = rows < 65536 ? rows : 65536;
  hipLaunchKernelGGL(k_fill_f32, dim3((uint32_t)grid), dim3(256), 0, stream, p, rows, cols, ld);
  return hipGetLastError();
}

hipError_t launch_mean(const float* row_loss, int64_t N, const int32_t* n_valid, float* out, hipStream_t stream) {
  hipLaunchKernelGGL(k_mean, dim3(1), dim3(1024), 0, stream, row_loss, N, n_valid, out);
  return hipGetLastError();
}

}  // namespace vce
