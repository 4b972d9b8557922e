// BF16 matrix products of the chunked linear head on the gfx950 matrix cores
// (v_mfma_f32_32x32x16_bf16), FP32 accumulation:
//
//   C[M][N] (+)= sum_k A(m, k) B(n, k)
//
// with each operand either K-contiguous (A as [M][K], B as [N][K]) or
// M/N-contiguous (A as [K][M], B as [K][N]).  The head's three products map
// onto it as
//   logits_c [n][V] = h_c W^T    A = h_c (K-contig.)  B = W (K-contig.)  BF16 out
//   dh_c     [n][D] = G_c W      A = G_c (K-contig.)  B = W ([V][D], N-contig.)  BF16 out
//   dW       [V][D] (+)= G_c^T h_c   A = G_c ([n][V], M-contig.)  B = h_c ([n][D], N-contig.)  FP32 out
//
// Design (one 256 x 256 output tile per workgroup of 4 waves, 128 x 128 per
// wave, the FP32 accumulators in AGPRs):
//  * k-tiles of 64: every thread stages 8 chunks of 16 bytes of each operand
//    per k-tile through registers, in two register sets, so the loads of tile
//    kt+2 are in flight while tile kt+1 goes into LDS and tile kt feeds the
//    MFMAs.  Two loads deep is what keeps the operand stream near the rate
//    the matrix cores consume it (one deep, or loads straight into LDS, leave
//    them waiting).
//  * LDS holds two stages of both tiles (128 KiB).  K-contiguous tiles are
//    [256][64] with 128-byte rows and fragments read by ds_read_b128;
//    M/N-contiguous tiles are [64][256] with 512-byte rows and fragments read
//    by ds_read_b64_tr_b16, which hands every lane 4 consecutive k of its own
//    column.  Both layouts XOR-swizzle 16-byte chunks so that the reads and
//    writes are free of bank conflicts.
//  * Each k-tile runs 4 groups of 16 MFMAs; the next group's fragments, the
//    loads (group 0) and the LDS writes (spread over groups 0-2: the writes
//    compete with the fragment reads for the LDS data path, and bunched
//    together they stall it) are interleaved between them, and the one
//    barrier per k-tile sits before the last group, so the next tile's first
//    fragments are read while that group runs.
//  * Bounds: buffer loads with byte ranges read rows past M, N or K as zero;
//    K-contiguous elements past K (the rest of a row) are zeroed on their way
//    into LDS; stores are guarded.  Leading dimensions are multiples of 8 and
//    the operands 16-byte aligned, so no 16-byte chunk straddles a range end.
#include <stdint.h>

#include <type_traits>

#include <hip/hip_runtime.h>

#include "ce_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t Rsrc;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kBM = 256, kBN = 256, kBK = 64, kThreads = 256;
constexpr int kTile = 256 * kBK * 2;  // one operand's tile: 32 KiB
constexpr int kStage = 2 * kTile;

// s_waitcnt with one counter set and the others at their maxima
#define GEMM_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))
#define GEMM_WAIT_LGKM(n) __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | ((n) << 8))

__device__ __forceinline__ Rsrc rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}
// K-contiguous tile: chunk c (of 8) of row r at c ^ ((r >> 1) & 7)
__device__ __forceinline__ uint32_t swz_k(int r) { return (uint32_t)((r >> 1) & 7); }
__device__ __forceinline__ uint32_t off_k(int r, int c) { return (uint32_t)(r * 128 + ((c ^ swz_k(r)) << 4)); }
// M/N-contiguous tile: chunk c (of 32) of k-row k at c ^ (4 (k & 3))
__device__ __forceinline__ uint32_t swz_mn(int k) { return (uint32_t)((k & 3) << 2); }
__device__ __forceinline__ uint32_t off_mn(int k, int c) { return (uint32_t)(k * 512 + ((c ^ swz_mn(k)) << 4)); }

// One operand of a workgroup: where its k-tiles come from and how its
// fragments are read.  Thread t stages, per k-tile, rows t/8 + 32 j at chunk
// t%8 (K-contiguous) or k-rows t/32 + 8 j at chunk t%32 (M/N-contiguous),
// j < 8; its LDS slots for the 8 chunks are 4 KiB apart in both layouts.
template <bool KC>
struct Operand {
  const __bf16* p;
  int64_t ld;
  int R, r0, K;   // extent of M (or N), this block's first row (column), K
  uint32_t vo;    // this thread's byte offset in the block's rows (K-contig.) or in a k-tile's rows
  uint32_t jstr;  // bytes between its rows j and j+1
  uint32_t lw;    // its LDS byte offset for j = 0
  Rsrc rk;        // K-contiguous: the block's rows, for the whole K loop

  __device__ __forceinline__ void init(const __bf16* p_, int64_t ld_, int R_, int r0_, int K_, int tid) {
    p = p_, ld = ld_, R = R_, r0 = r0_, K = K_;
    if constexpr (KC) {
      const int r = tid >> 3, c = tid & 7;
      vo = (uint32_t)(r * ld * 2) + c * 16;
      jstr = (uint32_t)(32 * ld * 2);
      lw = off_k(r, c);
      const int rows = R - r0 < 256 ? R - r0 : 256;
      rk = rsrc(p + (int64_t)r0 * ld, (uint32_t)(rows * ld * 2));
    } else {
      const int k = tid >> 5, c = tid & 31;
      vo = (uint32_t)(k * ld * 2) + c * 16;
      jstr = (uint32_t)(8 * ld * 2);
      lw = off_mn(k, c);
    }
  }
  __device__ __forceinline__ void gload(int kt, u32x4 (&v)[8]) const {
    Rsrc r;
    uint32_t s0;
    if constexpr (KC) {
      r = rk;
      s0 = (uint32_t)(kt * kBK * 2);
    } else {
      // k-rows k0 .. k0+63 from column r0 on (rows past K out of range, so zero; a k-tile past K reads
      // nothing); the last row's range ends on a whole 16-byte chunk, inside the row's stride
      const int k0 = kt * kBK;
      const int krows = K - k0 < kBK ? K - k0 : kBK;
      const int64_t cols = ((int64_t)(R - r0) + 7) & ~(int64_t)7;
      r = rsrc(p + (int64_t)(k0 < K ? k0 : 0) * ld + r0,
               krows > 0 ? (uint32_t)(((int64_t)(krows - 1) * ld + cols) * 2) : 0u);
      s0 = 0;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = __builtin_amdgcn_raw_buffer_load_b128(r, (int)vo, (int)(s0 + j * jstr), 0);
  }
  // staged chunk j into LDS; with MASK (K-contiguous), elements at k >= K, which hold whatever follows in
  // memory, are zeroed on the way
  template <bool MASK>
  __device__ __forceinline__ void lwrite(unsigned char* tile, const u32x4 (&v)[8], int j, int kt, int tid) const {
    u32x4 keep = {~0u, ~0u, ~0u, ~0u};
    if constexpr (MASK && KC) {
      const int nv = K - (kt * kBK + (tid & 7) * 8);  // valid elements of this thread's 8
#pragma unroll
      for (int w = 0; w < 4; ++w) keep[w] = (nv >= 2 * w + 2) ? 0xffffffffu : (nv == 2 * w + 1 ? 0x0000ffffu : 0u);
    }
    *reinterpret_cast<u32x4*>(tile + lw + j * 4096) = (MASK && KC) ? (v[j] & keep) : v[j];
  }
  // fragment of rows (columns) rb .. rb+31 at k = kk*16 .. +15: lane l gets row rb + l%32 and
  // k = kk*16 + 8 (l/32) + e in element e (the MFMA's operand layout)
  __device__ __forceinline__ bf16x8 frag(const unsigned char* tile, int rb, int kk, int lane) const {
    if constexpr (KC) {
      return *reinterpret_cast<const bf16x8*>(tile + off_k(rb + (lane & 31), kk * 2 + (lane >> 5)));
    } else {
      // within each 16 lanes, lane s names k-row kb + s/4 at columns cb + 4 (s%4) .. +3 and receives
      // column cb + s at k-rows kb .. kb+3
      const int col = rb + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
      const int k = kk * 16 + 8 * (lane >> 5) + ((lane & 15) >> 2);
      const uint32_t a0 = off_mn(k, col >> 3) + (col & 7) * 2;
      const uint32_t a1 = off_mn(k + 4, col >> 3) + (col & 7) * 2;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + a0));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(tile + a1));
      return __builtin_bit_cast(bf16x8, (i16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
  }
};

// OUT 0: BF16 store, 1: FP32 store, 2: FP32 accumulate.  TAIL: the k-tiles (64 wide, an even number of them)
// reach past K, and a K-contiguous operand must have those elements zeroed.
template <bool AK, bool BKC, int OUT, bool TAIL>
__global__ __launch_bounds__(kThreads) void k_gemm(const __bf16* __restrict__ A, int64_t lda,
                                                   const __bf16* __restrict__ B, int64_t ldb, void* __restrict__ C,
                                                   int64_t ldc, int M, int N, int K, int mblocks) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * kStage];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // The 8 XCDs take blocks round-robin (block id mod 8); each gets a contiguous run of tiles, which it walks
  // in groups of 4 n-blocks, n fastest, so that the tiles resident on one XCD share operand slabs in its L2.
  constexpr int kGroup = 4;
  const int T = gridDim.x, per = (T + 7) / 8;
  const int L = (T & 7) ? (int)blockIdx.x : (int)((blockIdx.x & 7) * per + (blockIdx.x >> 3));
  const int nblocks = T / mblocks;
  const int grp = L / (kGroup * mblocks), first = grp * kGroup;
  const int gsz = nblocks - first < kGroup ? nblocks - first : kGroup;
  const int bn = first + (L - grp * kGroup * mblocks) % gsz, bm = (L - grp * kGroup * mblocks) / gsz;
  const int m0 = bm * kBM, n0 = bn * kBN;
  const int wm = wave & 1, wn = wave >> 1;
  Operand<AK> oa;
  Operand<BKC> ob;
  oa.init(A, lda, M, m0, K, tid);
  ob.init(B, ldb, N, n0, K, tid);
  u32x4 ra0[8], rb0[8], ra1[8], rb1[8];  // register set p: the k-tiles of parity p on their way to LDS
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x16){};
  bf16x8 fa[2][4], fb[2][4];
  auto fread = [&](int st, int kk, int s) {
    const unsigned char* as = smem + st * kStage;
    const unsigned char* bs = as + kTile;
    fa[s][0] = oa.frag(as, wm * 128, kk, lane);  // in the order the MFMAs use them: a0, b0..b3, a1..a3
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[s][j] = ob.frag(bs, wn * 128 + j * 32, kk, lane);
#pragma unroll
    for (int i = 1; i < 4; ++i) fa[s][i] = oa.frag(as, wm * 128 + i * 32, kk, lane);
  };
  auto mfmas = [&](int s) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s][i], fb[s][j], acc[i][j], 0, 0, 0);
  };
  constexpr int kReads = (AK ? 4 : 8) + (BKC ? 4 : 8);  // LDS read instructions per fragment set
  const int nk = (K + kBK - 1) / kBK;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  // k-tile kt of parity P: MODE 2 loads tile kt+2 into register set P (which held tile kt, already in LDS)
  // and writes tile kt+1 (set P^1, loaded one tile earlier) into the other LDS stage; MODE 0 (the last
  // tile) neither.  The tile count
  // is rounded up to even: a tile past K holds zeros (out of range, or masked), as do loads past the end.
  auto tile = [&](int kt, auto mode, auto parity) {
    constexpr int MODE = decltype(mode)::value;
    constexpr int P = decltype(parity)::value;
    auto& la = P ? ra1 : ra0;
    auto& lb = P ? rb1 : rb0;
    auto& wa = P ? ra0 : ra1;
    auto& wb = P ? rb0 : rb1;
    unsigned char* nxt = smem + (P ^ 1) * kStage;
    // tile kt+1's loads were issued a tile ago; its 16 chunks per operand go into LDS spread over groups 0-2
    if constexpr (MODE == 2) GEMM_WAIT_VM(0);
#pragma unroll
    for (int kk = 0; kk < 3; ++kk) {
      const int s = kk & 1;
      fread(P, kk + 1, s ^ 1);
      if constexpr (MODE == 2) {
        if (kk == 0) {
          oa.gload(kt + 2, la);
          ob.gload(kt + 2, lb);
        }
        // chunks j of each operand: group 0 takes j 0..1, group 1 j 2..4, group 2 j 5..7
        const int j0 = kk == 0 ? 0 : (kk == 1 ? 2 : 5), j1 = kk == 0 ? 2 : (kk == 1 ? 5 : 8);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          if (j >= j0 && j < j1) {
            oa.template lwrite<TAIL>(nxt, wa, j, kt + 1, tid);
            ob.template lwrite<TAIL>(nxt + kTile, wb, j, kt + 1, tid);
          }
      }
      mfmas(s);
      for (int q = 0; q < 8; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                          // an MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, kReads / 8, 0);                 // fragment reads
        if (MODE == 2 && kk == 0) __builtin_amdgcn_sched_group_barrier(0x020, 2, 0);  // global loads
      }
      for (int q = 0; q < 8; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (MODE == 2) __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);            // LDS writes
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (MODE == 2) {
      // tile kt+1 is in LDS for this wave and its reads of this stage are done; after the barrier, for all
      GEMM_WAIT_LGKM(0);
      __syncthreads();
      fread(P ^ 1, 0, 0);
    }
    mfmas(1);
    if constexpr (MODE == 2) {
      for (int q = 0; q < 8; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, kReads / 8, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  const int nk2 = (nk + 1) & ~1;
  oa.gload(0, ra0);
  ob.gload(0, rb0);
  oa.gload(1, ra1);
  ob.gload(1, rb1);
  GEMM_WAIT_VM(16);  // tile 0 has landed
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    oa.template lwrite<TAIL>(smem, ra0, j, 0, tid);
    ob.template lwrite<TAIL>(smem + kTile, rb0, j, 0, tid);
  }
  GEMM_WAIT_LGKM(0);
  __syncthreads();
  fread(0, 0, 0);
  for (int kt = 0; kt + 2 < nk2; kt += 2) {
    tile(kt, I2{}, I0{});
    tile(kt + 1, I2{}, I1{});
  }
  tile(nk2 - 2, I2{}, I0{});
  tile(nk2 - 1, I0{}, I1{});

  // lane l holds rows (e/4)*8 + (l/32)*4 + e%4 and column l%32 of each 32 x 32 tile; slice i is the wave's
  // rows i*32 .. +31 (64 values per lane)
  auto at = [&](int i, int j, int e, int& row, int& col) {
    row = m0 + wm * 128 + i * 32 + (lane >> 5) * 4 + (e >> 2) * 8 + (e & 3);
    col = n0 + wn * 128 + j * 32 + (lane & 31);
  };
  // C += acc (FP32) through 16-byte row vectors, which need C 16-byte aligned and its rows a multiple of 16
  // bytes; the written-only outputs keep the direct element stores, which the next tile's loads overlap
  const bool vec = OUT == 2 && ((uintptr_t)C & 15u) == 0 && (ldc % 4) == 0;
  if (vec) {
    // Each wave's slice goes through its own LDS region (32 rows of 136 floats: the pad puts rows r and r+4,
    // written by one instruction, on disjoint banks) and comes back as row vectors of 4 columns a lane.  The
    // main loop's last fragment reads must be done in every wave first.
    constexpr int kPad = 136;
    __syncthreads();
    float* reg = reinterpret_cast<float*>(smem) + wave * (32 * kPad);
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const int rbase = m0 + wm * 128, cbase = n0 + wn * 128;
    auto to_lds = [&](int i) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          reg[((lane >> 5) * 4 + (e >> 2) * 8 + (e & 3)) * kPad + j * 32 + (lane & 31)] = acc[i][j][e];
    };
    {
      float* __restrict__ Cf = static_cast<float*>(C);
      // lane l takes columns (l%32)*4 .. +3 of rows q*2 + l/32; the next slice's old values are loaded before
      // this slice is summed and stored
      f32x4 old[2][16];
      auto ld_old = [&](int i, f32x4 (&o)[16]) {
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int row = rbase + i * 32 + q * 2 + (lane >> 5), col = cbase + (lane & 31) * 4;
          const float* src = Cf + (int64_t)row * ldc + col;
          if (row < M && col + 4 <= N) {
            o[q] = *reinterpret_cast<const f32x4*>(src);
          } else {
            o[q] = (f32x4){};
#pragma unroll
            for (int k = 0; k < 4; ++k)
              if (row < M && col + k < N) o[q][k] = src[k];
          }
        }
      };
      ld_old(0, old[0]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (i + 1 < 4) ld_old(i + 1, old[(i + 1) & 1]);
        to_lds(i);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          const int r = q * 2 + (lane >> 5), c = (lane & 31) * 4;
          f32x4 v = *reinterpret_cast<const f32x4*>(reg + r * kPad + c);
          v += old[i & 1][q];
          const int row = rbase + i * 32 + r, col = cbase + c;
          if (row >= M) continue;
          float* dst = Cf + (int64_t)row * ldc + col;
          if (col + 4 <= N) {
            *reinterpret_cast<f32x4*>(dst) = v;
          } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
              if (col + k < N) dst[k] = v[k];
          }
        }
      }
    }
    return;
  }
  // element stores from the accumulator layout (and C += acc where C is not 16-byte aligned)
  if constexpr (OUT == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          int row, col;
          at(i, j, e, row, col);
          if (row < M && col < N) static_cast<__bf16*>(C)[(int64_t)row * ldc + col] = (__bf16)acc[i][j][e];
        }
  } else {
    float* __restrict__ Cf = static_cast<float*>(C);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          int row, col;
          at(i, j, e, row, col);
          if (row < M && col < N) {
            float* p = Cf + (int64_t)row * ldc + col;
            *p = OUT == 2 ? *p + acc[i][j][e] : acc[i][j][e];
          }
        }
  }
}

}  // namespace

namespace vce {

bool gemm_bf16_supported(const GemmBf16& g) {
  auto al16 = [](const void* p) { return ((uintptr_t)p & 15u) == 0; };
  if (g.M < 1 || g.N < 1 || g.K < 1 || g.lda % 8 || g.ldb % 8 || !al16(g.A) || !al16(g.B) || !g.C) return false;
  if ((g.a_kc ? g.K : g.M) > g.lda || (g.b_kc ? g.K : g.N) > g.ldb) return false;
  // the layouts and outputs of the head's three products
  const bool logits = g.a_kc && g.b_kc && g.out == 0, dh = g.a_kc && !g.b_kc && g.out == 0;
  const bool dw = !g.a_kc && !g.b_kc && (g.out == 1 || g.out == 2);
  if (!logits && !dh && !dw) return false;
  // byte offsets within one buffer range stay below 2^31 (a K-contiguous block's 256 rows, an M/N-contiguous
  // k-tile's 64 rows)
  const int64_t lim = (int64_t)1 << 31;
  if ((g.a_kc ? 256 : 64) * g.lda * 2 >= lim || (g.b_kc ? 256 : 64) * g.ldb * 2 >= lim) return false;
  const int64_t tiles = (int64_t)((g.M + kBM - 1) / kBM) * ((g.N + kBN - 1) / kBN);
  return tiles < lim;
}

hipError_t launch_gemm_bf16(const GemmBf16& g, hipStream_t stream) {
  if (!gemm_bf16_supported(g)) return hipErrorInvalidValue;
  const int mblocks = (g.M + kBM - 1) / kBM, nblocks = (g.N + kBN - 1) / kBN;
  const dim3 grid((unsigned)(mblocks * nblocks)), block(kThreads);
  const bool tail = g.K % (2 * kBK) != 0;  // the tile count is rounded up to even
  const __bf16* A = static_cast<const __bf16*>(g.A);
  const __bf16* B = static_cast<const __bf16*>(g.B);
#define CE_GEMM(AKv, BKv, O, T)                                                                                   \
  hipLaunchKernelGGL((k_gemm<AKv, BKv, O, T>), grid, block, 0, stream, A, g.lda, B, g.ldb, g.C, g.ldc, g.M, g.N, \
                     g.K, mblocks)
  if (g.a_kc && g.b_kc && g.out == 0) {
    if (tail) CE_GEMM(true, true, 0, true); else CE_GEMM(true, true, 0, false);
  } else if (g.a_kc && !g.b_kc && g.out == 0) {
    if (tail) CE_GEMM(true, false, 0, true); else CE_GEMM(true, false, 0, false);
  } else if (!g.a_kc && !g.b_kc && g.out == 1) {
    CE_GEMM(false, false, 1, false);
  } else if (!g.a_kc && !g.b_kc && g.out == 2) {
    CE_GEMM(false, false, 2, false);
  } else {
    return hipErrorInvalidValue;
  }
#undef CE_GEMM
  return hipGetLastError();
}

}  // namespace vce
