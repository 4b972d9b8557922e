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
// One 256 x 256 output tile per workgroup of 4 waves, 128 x 128 per wave, the FP32 accumulators in AGPRs,
// k-tiles of 64, two LDS stages (128 KiB).  Two kernels:
//  * k_gemm_dma (the default): both operands go from memory straight into LDS (buffer_load ... lds, 1 KiB
//    per wave instruction, whole 128-byte lines).  The one barrier per k-tile sits before its last group of
//    MFMAs: by then every wave holds the tile's last fragments and the next tile has landed, so the stage
//    just read takes the loads of the tile after next (spread over that last group and the next tile's
//    first two groups) while the next tile's first fragments are read.  The loads are issued in asm: the compiler cannot tell the two stages
//    of the LDS array apart and would otherwise wait for every load in flight before each LDS read.  BF16
//    results leave through a per-wave LDS slice as 16-byte row chunks (the MFMA operands are swapped so
//    that each lane holds 4 consecutive columns of one row).  The BF16 products (an even k-tile count) run
//    it in persistent form, k_gemm_dmap: one workgroup per CU walking its tiles, the load stream running
//    on across tile boundaries.  A dh product whose output tiles fill at most half the CUs splits its K
//    range instead (FP32 partial planes in a caller's scratch, summed in plane order by k_sum_planes).
//  * k_gemm (shapes the first does not take: a K-contiguous operand whose K is not a multiple of 64, which
//    must be masked on its way into LDS, or an M/N-contiguous operand whose k-extent exceeds a 31-bit byte
//    range): every thread stages 8 chunks of 16 bytes of each operand per k-tile through registers, in two
//    register sets, so the loads of tile kt+2 are in flight while tile kt+1 goes into LDS (ds_write) and
//    tile kt feeds the MFMAs; the barrier also sits before the last group.
// Common to both:
//  * LDS layouts: K-contiguous tiles are [256][64] with 128-byte rows, fragments read by ds_read_b128;
//    M/N-contiguous tiles are [64][256] with 512-byte rows, fragments read by ds_read_b64_tr_b16, which
//    hands every lane 4 consecutive k of its own column.  Both XOR-swizzle 16-byte chunks so that reads
//    and writes are free of bank conflicts.
//  * Each k-tile runs 4 groups of 16 MFMAs with the next group's fragments read between them.
//  * Bounds: buffer loads with byte ranges read rows past M, N or K as zero (an M/N-contiguous operand's
//    columns past M or N may read what follows them, which reaches only output rows or columns that are
//    never stored); stores are guarded.  Leading dimensions are multiples of 8 and the operands 16-byte
//    aligned, so no 16-byte chunk straddles a range end.
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
typedef __attribute__((address_space(3))) void lds_t;

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

// One wave's 1 KiB load from a buffer straight into LDS at `lds` (lane l's 16 bytes at lds + 16 l), from
// byte offset vo + soff of the buffer `desc`.  No registers receive data, so the compiler tracks nothing;
// the caller waits for it (vmcnt) and makes it visible to the other waves (barrier) before reading.
__device__ __forceinline__ void lds_dma16(u32x4 desc, uint32_t lds, uint32_t vo, uint32_t soff) {
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" : : "v"(vo), "s"(desc), "s"(soff), "{m0}"(lds) : "memory");
}
// raw buffer descriptor: base, no stride, `bytes` in range (reads past it return zero)
__device__ __forceinline__ u32x4 desc16(const void* p, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  return (u32x4){(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}

// One operand's loads straight into LDS: wave w fills 1 KiB blocks 8w .. 8w+7 of the operand's stage tile.
// K-contiguous: block q holds rows 8q .. 8q+7 (lane l: row 8q + l/8, physical chunk l%8, which holds the
// logical chunk (l%8) ^ swz_k(row)); the buffer is the block's rows, k-tile kt at byte offset 128 kt.
// M/N-contiguous: block q holds k-rows 2q, 2q+1 (lane l: k-row 2q + l/32, physical chunk l%32, holding the
// logical chunk (l%32) ^ swz_mn(k)); the buffer is rows 0 .. K-1 from column r0, k-tile kt at 64 kt rows.
template <bool KC>
struct DmaOperand {
  u32x4 d;
  uint32_t vo[8];
  uint32_t kstep;  // bytes between k-tiles
  __device__ __forceinline__ void init(const __bf16* p, int64_t ld, int R, int r0, int K, int wave, int lane) {
    if constexpr (KC) {
      const int rows = R - r0 < 256 ? R - r0 : 256;
      d = desc16(p + (int64_t)r0 * ld, (uint32_t)(rows * ld * 2));
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = (wave * 8 + j) * 8 + (lane >> 3);
        vo[j] = (uint32_t)(r * ld * 2) + ((((uint32_t)lane & 7u) ^ swz_k(r)) << 4);
      }
      kstep = kBK * 2;
    } else {
      // the range ends with row K-1's last column of this block (rounded up to a 16-byte chunk)
      const int64_t cols = ((int64_t)(R - r0) + 7) & ~(int64_t)7;
      d = desc16(p + r0, (uint32_t)(((int64_t)(K - 1) * ld + (cols < 256 ? cols : 256)) * 2));
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int k = (wave * 8 + j) * 2 + (lane >> 5);
        vo[j] = (uint32_t)(k * ld * 2) + ((((uint32_t)lane & 31u) ^ swz_mn(k)) << 4);
      }
      kstep = (uint32_t)(kBK * ld * 2);
    }
  }
};

// Tile L of the tile order: groups of 4 n-blocks, n fastest within a group, so that consecutive tiles
// share operand slabs.
__device__ __forceinline__ void tile_at(int L, int mblocks, int nblocks, int& m0, int& n0) {
  constexpr int kGroup = 4;
  const int grp = L / (kGroup * mblocks), first = grp * kGroup;
  const int gsz = nblocks - first < kGroup ? nblocks - first : kGroup;
  n0 = (first + (L - grp * kGroup * mblocks) % gsz) * kBN;
  m0 = ((L - grp * kGroup * mblocks) / gsz) * kBM;
}
// The workgroup's output tile.  The 8 XCDs take blocks round-robin (block id mod 8); each gets a contiguous
// run of the tile order, so that the tiles resident on one XCD share operand slabs in its L2.
__device__ __forceinline__ void tile_origin(int mblocks, int& m0, int& n0) {
  const int T = gridDim.x, per = (T + 7) / 8;
  const int L = (T & 7) ? (int)blockIdx.x : (int)((blockIdx.x & 7) * per + (blockIdx.x >> 3));
  tile_at(L, mblocks, T / mblocks, m0, n0);
}

// FP32 results (OUT 1: written, 2: added) from the accumulator layout: lane l holds rows
// (e/4)*8 + (l/32)*4 + e%4 and column l%32 of each 32 x 32 block.  C += acc goes through LDS (`smem`, free
// by now) as 16-byte row vectors where C allows them; the written-only output keeps element stores.
template <int OUT>
__device__ __forceinline__ void store_acc_f32(const f32x16 (&acc)[4][4], unsigned char* smem, void* C, int64_t ldc,
                                              int M, int N, int m0, int n0, int wm, int wn, int wave, int lane) {
  float* __restrict__ Cf = static_cast<float*>(C);
  const bool vec = OUT == 2 && ((uintptr_t)C & 15u) == 0 && (ldc % 4) == 0;
  if (vec) {
    // Each wave's slice goes through its own LDS region (32 rows of 136 floats: the pad puts rows r and r+4,
    // written by one instruction, on disjoint banks) and comes back as row vectors of 4 columns a lane.
    constexpr int kPad = 136;
    float* reg = reinterpret_cast<float*>(smem) + wave * (32 * kPad);
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const int rbase = m0 + wm * 128, cbase = n0 + wn * 128;
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
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          reg[((lane >> 5) * 4 + (e >> 2) * 8 + (e & 3)) * kPad + j * 32 + (lane & 31)] = acc[i][j][e];
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
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int row = m0 + wm * 128 + i * 32 + (lane >> 5) * 4 + (e >> 2) * 8 + (e & 3);
        const int col = n0 + wn * 128 + j * 32 + (lane & 31);
        if (row < M && col < N) {
          float* p = Cf + (int64_t)row * ldc + col;
          *p = OUT == 2 ? *p + acc[i][j][e] : acc[i][j][e];
        }
      }
}

// OUT 0: BF16 store, 1: FP32 store, 2: FP32 accumulate.  TAIL: the k-tiles (64 wide, an even number of them)
// reach past K, and a K-contiguous operand must have those elements zeroed.
template <bool AK, bool BKC, int OUT, bool TAIL>
__global__ __launch_bounds__(kThreads) void k_gemm(const __bf16* __restrict__ A, int64_t lda,
                                                   const __bf16* __restrict__ B, int64_t ldb, void* __restrict__ C,
                                                   int64_t ldc, int M, int N, int K, int mblocks) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * kStage];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int m0, n0;
  tile_origin(mblocks, m0, n0);
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

  if constexpr (OUT == 0) {
    // BF16 element stores from the accumulator layout (rows (e/4)*8 + (l/32)*4 + e%4, column l%32 of each
    // 32 x 32 block): 32 consecutive columns of two rows per instruction
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int row = m0 + wm * 128 + i * 32 + (lane >> 5) * 4 + (e >> 2) * 8 + (e & 3);
          const int col = n0 + wn * 128 + j * 32 + (lane & 31);
          if (row < M && col < N) static_cast<__bf16*>(C)[(int64_t)row * ldc + col] = (__bf16)acc[i][j][e];
        }
  } else {
    // C += acc reuses LDS: the main loop's last fragment reads must be done in every wave
    if constexpr (OUT == 2) __syncthreads();
    store_acc_f32<OUT>(acc, smem, C, ldc, M, N, m0, n0, wm, wn, wave, lane);
  }
}

// Both operands straight into LDS (shapes: gemm_dma_ok).  Same tile, LDS layouts and fragment reads as
// k_gemm; k-tile kt's loads start with the last MFMA group of tile kt-2, right after the barrier that frees
// that tile's stage, and finish in the first two groups of tile kt-1.
// ksplit > 0: split K (gridDim.y splits): split y takes k-tiles [y ksplit, (y+1) ksplit) of K and writes its
// FP32 partial product to plane y of C (cplane elements apart).
template <bool AK, bool BKC, int OUT>
__global__ __launch_bounds__(kThreads) void k_gemm_dma(const __bf16* __restrict__ A, int64_t lda,
                                                       const __bf16* __restrict__ B, int64_t ldb, void* __restrict__ C,
                                                       int64_t ldc, int M, int N, int K, int mblocks, int ksplit,
                                                       int64_t cplane) {
  constexpr bool BF16_OUT = OUT == 0;  // through LDS slices, from transposed accumulator blocks
  if (ksplit > 0) {
    const int k0 = (int)blockIdx.y * ksplit;
    A += AK ? (int64_t)k0 : (int64_t)k0 * lda;
    B += BKC ? (int64_t)k0 : (int64_t)k0 * ldb;
    K = K - k0 < ksplit ? K - k0 : ksplit;
    C = static_cast<float*>(C) + (int64_t)blockIdx.y * cplane;
  }
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * kStage];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  int m0, n0;
  tile_origin(mblocks, m0, n0);
  const int wm = wave & 1, wn = wave >> 1;
  DmaOperand<AK> da;
  DmaOperand<BKC> db;
  da.init(A, lda, M, m0, K, wave, lane);
  db.init(B, ldb, N, n0, K, wave, lane);
  const Operand<AK> oa{};  // fragment reads
  const Operand<BKC> ob{};
  const u32x4 none = desc16(A, 0);  // loads past the last k-tile: out of range, no memory traffic
  const uint32_t lwave = (uint32_t)(uintptr_t)(lds_t*)smem + (uint32_t)wave * 8192u;
  const int nk = (K + kBK - 1) / kBK;
  // load q of k-tile kt (0-7: A's blocks, 8-15: B's) into stage kt % 2.  Tile kt+2's loads go out spread
  // over three MFMA groups: A's 8 with tile kt's last group (right after the barrier that frees the stage),
  // B's 8 with the first two groups of tile kt+1, 4 in each; bunched into one group they back up the
  // memory pipeline and hold up the MFMAs queued behind them.
  constexpr int kLast = 8, kG0 = 4, kG1 = 4;
  static_assert(kLast <= 8 && kG0 <= 8 && kG1 <= 8 && kLast + kG0 + kG1 == 16, "one load per MFMA pair, 16 per tile");
  auto issue = [&](int kt, int q) {
    const uint32_t st = lwave + (uint32_t)(kt & 1) * kStage + (q >= 8 ? kTile : 0) + (q & 7) * 1024;
    const bool live = kt < nk;
    if (q < 8) lds_dma16(live ? da.d : none, st, da.vo[q], (uint32_t)kt * da.kstep);
    else lds_dma16(live ? db.d : none, st, db.vo[q - 8], (uint32_t)kt * db.kstep);
  };
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x16){};
  bf16x8 fa[2][4], fb[2][4];
  // fragment read q of tile kt at k-step kk into set s, in the order the MFMAs use them: q 0 A block 0,
  // 1-4 B blocks 0-3, 5-7 A blocks 1-3
  auto read = [&](int kt, int kk, int s, int q) {
    const unsigned char* as = smem + (kt & 1) * kStage;
    if (q == 0) fa[s][0] = oa.frag(as, wm * 128, kk, lane);
    else if (q <= 4) fb[s][q - 1] = ob.frag(as + kTile, wn * 128 + (q - 1) * 32, kk, lane);
    else fa[s][q - 4] = oa.frag(as, wm * 128 + (q - 4) * 32, kk, lane);
  };
  auto mfma = [&](int s, int n) {
    const int i = n >> 2, j = n & 3;
    if (BF16_OUT)  // the transposed block: lane l gets row l%32 and columns 8q + 4(l/32) .. +3 in 4q .. 4q+3
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[s][j], fa[s][i], acc[i][j], 0, 0, 0);
    else
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[s][i], fb[s][j], acc[i][j], 0, 0, 0);
  };
#pragma unroll
  for (int q = 0; q < 16; ++q) issue(0, q);
#pragma unroll
  for (int q = 0; q < 16; ++q) issue(1, q);
  GEMM_WAIT_VM(16);  // tile 0 has landed (this wave's part)
  __syncthreads();
#pragma unroll
  for (int q = 0; q < 8; ++q) read(0, 0, 0, q);
  for (int kt = 0; kt < nk; ++kt) {
    // groups 0-2: k-steps 0-2, the next step's fragments read between the MFMAs; groups 0 and 1 also issue
    // the rest of tile kt+1's loads (tile 1 went out whole before the loop)
#pragma unroll
    for (int kk = 0; kk < 3; ++kk) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (kk == 0 && q < kG0 && kt > 0) issue(kt + 1, kLast + q);
        if (kk == 1 && q < kG1 && kt > 0) issue(kt + 1, kLast + kG0 + q);
        mfma(kk & 1, 2 * q);
        mfma(kk & 1, 2 * q + 1);
        read(kt, kk + 1, (kk + 1) & 1, q);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // every wave holds tile kt's last fragments and has tile kt+1's loads done; after the barrier tile kt's
    // stage takes tile kt+2 and tile kt+1 is readable
    GEMM_WAIT_VM(0);
    GEMM_WAIT_LGKM(0);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (q < kLast) issue(kt + 2, q);
      mfma(1, 2 * q);
      mfma(1, 2 * q + 1);
      read(kt + 1, 0, 0, q);  // after the last tile: a stage's stale contents, never used
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  GEMM_WAIT_VM(0);
  GEMM_WAIT_LGKM(0);
  __syncthreads();
  if constexpr (BF16_OUT) {
    // per wave, 32 rows x 128 columns at a time through 8 KiB of LDS (8-byte unit u of row r at u ^ r),
    // out as 16-byte row chunks (16 lanes a row, 4 rows an instruction)
    unsigned char* slice = smem + wave * 8192;
    __bf16* Cb = static_cast<__bf16*>(C);
    const bool vec = ((uintptr_t)C & 15u) == 0 && (ldc & 7) == 0;
    const int row0 = m0 + wm * 128, col0 = n0 + wn * 128;
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = lane & 31, h = lane >> 5;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bf16x4 v = {(__bf16)acc[i][j][4 * q], (__bf16)acc[i][j][4 * q + 1], (__bf16)acc[i][j][4 * q + 2],
                            (__bf16)acc[i][j][4 * q + 3]};
          const int u = 8 * j + 2 * q + h;
          *reinterpret_cast<bf16x4*>(slice + r * 256 + ((u ^ r) << 3)) = v;
        }
      // 16-byte chunk t of row rr holds units 2t and 2t+1, at chunk t ^ (rr/2), in swapped order for odd rr
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const int rr = g * 4 + (lane >> 4), t = lane & 15;
        u32x4 v = *reinterpret_cast<const u32x4*>(slice + rr * 256 + ((t ^ (rr >> 1)) << 4));
        if (rr & 1) v = (u32x4){v[2], v[3], v[0], v[1]};
        const int row = row0 + i * 32 + rr, col = col0 + t * 8;
        if (row < M) {
          __bf16* dst = Cb + (int64_t)row * ldc + col;
          if (vec && col + 8 <= N) {
            *reinterpret_cast<u32x4*>(dst) = v;
          } else {
            const bf16x8 b = __builtin_bit_cast(bf16x8, v);
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (col + e < N) dst[e] = b[e];
          }
        }
      }
    }
  } else {
    store_acc_f32<OUT>(acc, smem, C, ldc, M, N, m0, n0, wm, wn, wave, lane);
  }
}

// The S FP32 partial planes of a split product ([M][N] each, N a multiple of 4), summed in plane order and
// rounded once to BF16 (out row stride ldo).
__global__ __launch_bounds__(256) void k_sum_planes(const float* __restrict__ part, int S, int64_t plane, int M,
                                                     int N, __bf16* __restrict__ out, int64_t ldo) {
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x, nq = (int64_t)M * (N / 4);
  if (q >= nq) return;
  const int64_t r = q / (N / 4), c = (q - r * (N / 4)) * 4;
  f32x4 acc = *reinterpret_cast<const f32x4*>(part + r * N + c);
  for (int s = 1; s < S; ++s) acc += *reinterpret_cast<const f32x4*>(part + (int64_t)s * plane + r * N + c);
  const bf16x4 v = {(__bf16)acc[0], (__bf16)acc[1], (__bf16)acc[2], (__bf16)acc[3]};
  __bf16* dst = out + r * ldo + c;
  if (((uintptr_t)dst & 7u) == 0) {
    *reinterpret_cast<bf16x4*>(dst) = v;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) dst[e] = v[e];
  }
}

// Persistent form of k_gemm_dma for BF16 outputs (an even k-tile count of at least 2): one workgroup per CU
// walks its tiles in the order of tile_origin, the load stream runs on across tile boundaries (the next
// tile's first k-tiles load during this tile's last two), and results leave through an LDS slice of their
// own (160 KiB in all), so the next tile's loads are not held up by the epilogue.
template <bool AK, bool BKC>
__global__ __launch_bounds__(kThreads) void k_gemm_dmap(const __bf16* __restrict__ A, int64_t lda,
                                                        const __bf16* __restrict__ B, int64_t ldb, __bf16* __restrict__ C,
                                                        int64_t ldc, int M, int N, int K, int mblocks, int ntiles) {
  __shared__ __attribute__((aligned(1024))) unsigned char smem[2 * kStage + 4 * 8192];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int wm = wave & 1, wn = wave >> 1;
  // tiles: with a multiple of 8 workgroups, XCD x = block % 8 owns the contiguous run [x per, (x+1) per) of
  // the tile order and its G/8 workgroups take those tiles in turn; otherwise workgroup b takes b, b+G, ...
  const int G = gridDim.x;
  const bool xcd = (G & 7) == 0;
  const int per = (ntiles + 7) / 8;
  const int t_lo = xcd ? (int)(blockIdx.x & 7) * per : 0;
  const int t_hi = xcd ? (t_lo + per < ntiles ? t_lo + per : ntiles) : ntiles;
  const int first = xcd ? (int)(blockIdx.x >> 3) : (int)blockIdx.x, gstep = xcd ? G / 8 : G;
  const int mine = t_hi - t_lo > first ? (t_hi - t_lo - first + gstep - 1) / gstep : 0;
  if (mine == 0) return;
  const int nblocks = ntiles / mblocks;
  auto origin = [&](int i, int& m0, int& n0) { tile_at(t_lo + first + i * gstep, mblocks, nblocks, m0, n0); };
  DmaOperand<AK> da;  // vo and kstep do not depend on the tile; d is set per tile below
  DmaOperand<BKC> db;
  da.init(A, lda, M, 0, K, wave, lane);
  db.init(B, ldb, N, 0, K, wave, lane);
  const u32x4 none = desc16(A, 0);
  auto descs = [&](int i, u32x4& a, u32x4& b) {
    if (i >= mine) {
      a = none, b = none;
      return;
    }
    int m0, n0;
    origin(i, m0, n0);
    DmaOperand<AK> ta;
    DmaOperand<BKC> tb;
    ta.init(A, lda, M, m0, K, wave, lane);
    tb.init(B, ldb, N, n0, K, wave, lane);
    a = ta.d, b = tb.d;
  };
  const Operand<AK> oa{};
  const Operand<BKC> ob{};
  const uint32_t lwave = (uint32_t)(uintptr_t)(lds_t*)smem + (uint32_t)wave * 8192u;
  const int nk = (K + kBK - 1) / kBK;
  u32x4 ca, cb, na, nb;  // this tile's and the next tile's buffers
  descs(0, ca, cb);
  descs(1, na, nb);
  // load q of k-tile k (stage k % 2; nk is even, so every tile starts in stage 0) from buffers (a, b)
  auto issue = [&](const u32x4& a, const u32x4& b, int k, int q) {
    const uint32_t st = lwave + (uint32_t)(k & 1) * kStage + (q >= 8 ? kTile : 0) + (q & 7) * 1024;
    if (q < 8) lds_dma16(a, st, da.vo[q], (uint32_t)k * da.kstep);
    else lds_dma16(b, st, db.vo[q - 8], (uint32_t)k * db.kstep);
  };
  constexpr int kLast = 8, kG0 = 4, kG1 = 4;
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x16){};
  bf16x8 fa[2][4], fb[2][4];
  auto read = [&](int k, int kk, int s, int q) {
    const unsigned char* as = smem + (k & 1) * kStage;
    if (q == 0) fa[s][0] = oa.frag(as, wm * 128, kk, lane);
    else if (q <= 4) fb[s][q - 1] = ob.frag(as + kTile, wn * 128 + (q - 1) * 32, kk, lane);
    else fa[s][q - 4] = oa.frag(as, wm * 128 + (q - 4) * 32, kk, lane);
  };
  auto mfma = [&](int s, int n) {
    const int i = n >> 2, j = n & 3;
    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[s][j], fa[s][i], acc[i][j], 0, 0, 0);
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  // k-tile kt of this tile; WHERE: 0 kt+1 and kt+2 in this tile, 1 kt+2 is the next tile's k-tile 0,
  // 2 (the last) kt+1 and kt+2 are the next tile's 0 and 1, and the next fragments are read after the
  // epilogue
  auto step = [&](int kt, auto where) {
    constexpr int W = decltype(where)::value;
    const u32x4& a1 = W == 2 ? na : ca;
    const u32x4& b1 = W == 2 ? nb : cb;
    const int k1 = W == 2 ? 0 : kt + 1;
    const u32x4& a2 = W >= 1 ? na : ca;
    const u32x4& b2 = W >= 1 ? nb : cb;
    const int k2 = W == 2 ? 1 : (W == 1 ? 0 : kt + 2);
#pragma unroll
    for (int kk = 0; kk < 3; ++kk) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (kk == 0 && q < kG0) issue(a1, b1, k1, kLast + q);
        if (kk == 1 && q < kG1) issue(a1, b1, k1, kLast + kG0 + q);
        mfma(kk & 1, 2 * q);
        mfma(kk & 1, 2 * q + 1);
        read(kt, kk + 1, (kk + 1) & 1, q);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    GEMM_WAIT_VM(0);
    GEMM_WAIT_LGKM(0);
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      if (q < kLast) issue(a2, b2, k2, q);
      mfma(1, 2 * q);
      mfma(1, 2 * q + 1);
      if (W != 2) read(kt + 1, 0, 0, q);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // k-tile 0 whole and k-tile 1's A loads; its B loads go out in k-tile 0's first groups like any other
#pragma unroll
  for (int q = 0; q < 16; ++q) issue(ca, cb, 0, q);
#pragma unroll
  for (int q = 0; q < 8; ++q) issue(ca, cb, 1, q);
  GEMM_WAIT_VM(8);
  __syncthreads();
  unsigned char* slice = smem + 2 * kStage + wave * 8192;
  const bool vec = ((uintptr_t)C & 15u) == 0 && (ldc & 7) == 0;
  for (int ti = 0; ti < mine; ++ti) {
#pragma unroll
    for (int q = 0; q < 8; ++q) read(0, 0, 0, q);
    for (int kt = 0; kt + 2 < nk; ++kt) step(kt, I0{});
    step(nk - 2, I1{});
    step(nk - 1, I2{});
    // the tile out through this wave's slice (32 rows x 128 columns at a time), as 16-byte row chunks
    int m0, n0;
    origin(ti, m0, n0);
    const int row0 = m0 + wm * 128, col0 = n0 + wn * 128;
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = lane & 31, h = lane >> 5;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const bf16x4 v = {(__bf16)acc[i][j][4 * q], (__bf16)acc[i][j][4 * q + 1], (__bf16)acc[i][j][4 * q + 2],
                            (__bf16)acc[i][j][4 * q + 3]};
          const int u = 8 * j + 2 * q + h;
          *reinterpret_cast<bf16x4*>(slice + r * 256 + ((u ^ r) << 3)) = v;
        }
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const int rr = g * 4 + (lane >> 4), t = lane & 15;
        u32x4 v = *reinterpret_cast<const u32x4*>(slice + rr * 256 + ((t ^ (rr >> 1)) << 4));
        if (rr & 1) v = (u32x4){v[2], v[3], v[0], v[1]};
        const int row = row0 + i * 32 + rr, col = col0 + t * 8;
        if (row < M) {
          __bf16* dst = C + (int64_t)row * ldc + col;
          if (vec && col + 8 <= N) {
            *reinterpret_cast<u32x4*>(dst) = v;
          } else {
            const bf16x8 bv = __builtin_bit_cast(bf16x8, v);
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (col + e < N) dst[e] = bv[e];
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = (f32x16){};
    ca = na, cb = nb;
    descs(ti + 2, na, nb);
  }
  GEMM_WAIT_VM(0);
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

// Shapes k_gemm_dma takes: K-contiguous operands need K % 64 == 0 (their rows are not masked on the way
// in), and an M/N-contiguous operand's k-extent must fit a 31-bit byte range from its first column.
// Compute units of the current device (cached per device; 256 on an MI355X).
static int cu_count() {
  static int cached[64];
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if ((n = __atomic_load_n(&cached[dev], __ATOMIC_RELAXED)) > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  __atomic_store_n(&cached[dev], n, __ATOMIC_RELAXED);
  return n;
}

static bool gemm_dma_ok(const GemmBf16& g) {
  const int64_t lim = (int64_t)1 << 31;
  auto mn_ok = [&](int64_t ld) { return ((int64_t)(g.K - 1) * ld + 256) * 2 < lim; };
  return (g.a_kc ? g.K % kBK == 0 : mn_ok(g.lda)) && (g.b_kc ? g.K % kBK == 0 : mn_ok(g.ldb));
}

hipError_t launch_gemm_bf16(const GemmBf16& g, hipStream_t stream) {
  if (!gemm_bf16_supported(g)) return hipErrorInvalidValue;
  const int mblocks = (g.M + kBM - 1) / kBM, nblocks = (g.N + kBN - 1) / kBN;
  const dim3 grid((unsigned)(mblocks * nblocks)), block(kThreads);
  const __bf16* A = static_cast<const __bf16*>(g.A);
  const __bf16* B = static_cast<const __bf16*>(g.B);
  const int nk = (g.K + kBK - 1) / kBK;
  // dh with few output tiles (a short chunk): the K range split so that the tiles times the splits fill the
  // compute units, each split's FP32 partial in a plane of the scratch, then the planes summed
  if (g.out == 0 && g.a_kc && !g.b_kc && g.scratch && ((uintptr_t)g.scratch & 15u) == 0 && g.N % 4 == 0 &&
      gemm_dma_ok(g)) {
    const int tiles = mblocks * nblocks, cus = cu_count();
    const int64_t plane = (int64_t)g.M * g.N;
    int64_t S = (cus + tiles - 1) / tiles;
    if (S > nk) S = nk;
    if (S > (int64_t)(g.scratch_bytes / ((size_t)plane * 4))) S = (int64_t)(g.scratch_bytes / ((size_t)plane * 4));
    if (tiles * 2 <= cus && S >= 2) {
      const int per_split = (int)((nk + S - 1) / S);  // k-tiles a split
      const int splits = (nk + per_split - 1) / per_split;
      float* part = static_cast<float*>(g.scratch);
      hipLaunchKernelGGL((k_gemm_dma<true, false, 1>), dim3((unsigned)tiles, (unsigned)splits), block, 0, stream, A,
                         g.lda, B, g.ldb, (void*)part, (int64_t)g.N, g.M, g.N, g.K, mblocks, per_split * kBK, plane);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      const int64_t nq = plane / 4;
      hipLaunchKernelGGL(k_sum_planes, dim3((unsigned)((nq + 255) / 256)), dim3(256), 0, stream, part, splits, plane,
                         g.M, g.N, static_cast<__bf16*>(g.C), g.ldc);
      return hipGetLastError();
    }
  }
  if (gemm_dma_ok(g) && g.out == 0 && nk % 2 == 0) {
    // persistent: one workgroup per CU (at most one per tile)
    const int tiles = mblocks * nblocks, cus = cu_count();
    const dim3 pgrid((unsigned)(tiles < cus ? tiles : cus));
    __bf16* Cb = static_cast<__bf16*>(g.C);
    if (g.a_kc && g.b_kc)
      hipLaunchKernelGGL((k_gemm_dmap<true, true>), pgrid, block, 0, stream, A, g.lda, B, g.ldb, Cb, g.ldc, g.M, g.N,
                         g.K, mblocks, tiles);
    else if (g.a_kc && !g.b_kc)
      hipLaunchKernelGGL((k_gemm_dmap<true, false>), pgrid, block, 0, stream, A, g.lda, B, g.ldb, Cb, g.ldc, g.M, g.N,
                         g.K, mblocks, tiles);
    else
      return hipErrorInvalidValue;
    return hipGetLastError();
  }
  if (gemm_dma_ok(g)) {
#define CE_GEMM_DMA(AKv, BKv, O)                                                                                 \
  hipLaunchKernelGGL((k_gemm_dma<AKv, BKv, O>), grid, block, 0, stream, A, g.lda, B, g.ldb, g.C, g.ldc, g.M, g.N, \
                     g.K, mblocks, 0, (int64_t)0)
    if (g.a_kc && g.b_kc && g.out == 0) CE_GEMM_DMA(true, true, 0);
    else if (g.a_kc && !g.b_kc && g.out == 0) CE_GEMM_DMA(true, false, 0);
    else if (!g.a_kc && !g.b_kc && g.out == 1) CE_GEMM_DMA(false, false, 1);
    else if (!g.a_kc && !g.b_kc && g.out == 2) CE_GEMM_DMA(false, false, 2);
    else return hipErrorInvalidValue;
#undef CE_GEMM_DMA
    return hipGetLastError();
  }
  const bool tail = g.K % (2 * kBK) != 0;  // the tile count is rounded up to even
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
