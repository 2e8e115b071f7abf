// Prompt-chunk projections on the bf16 matrix cores: C[m][n] = sum_k A[m][k]
// W[n][k] for chunks of up to 2,048 rows, fp32 accumulation rounded once to
// bf16 (pull request "llama: Nanbeige4.3-33B on Metal, the bf16 release
// served as published", section "How": prompt chunks of up to 2,048 rows on
// the matrix units).
//
// Both operands are K-contiguous: activations [M][K] and published weights
// [N][K].  Every output is a chain of v_mfma_f32_16x16x32_bf16 over 32-deep k
// steps in increasing k: lane l of an MFMA reads row l%16 and 8 consecutive k
// at 8*(l/16) of each operand, and holds output rows 4*(l/16) + j of column
// l%16 in its four accumulators.  (The 16x16x32 form sustains a higher
// product rate on gfx950 than 32x32x16 at the same fragment traffic per
// product when each wave keeps the same sub-tile.)  Two kernels share that
// order, so every output's bits are the same whichever runs and whatever M
// is: gemm_alt_kernel (256 x 256 or 256 x 224 tiles, an alternating
// two-group schedule with LDS-direct operand copies) and gemm_kernel
// (smaller tiles, register-staged copies, one pinned interleaved schedule).
//
// Exact form: the matrix unit's own accumulation loses more than one fp32
// addition per product (a chain of 224 products at K = 7,168 carries a
// signed error of ~7.5 fp32 steps at the row's RMS, binary64 as reference,
// where the decode projections' lane sums carry ~1.3), so on request the
// running sums restart every 128 terms into fp32 totals: ~2.1 steps, at about
// twice the time (256 x 128 tiles of the register-staged kernel).
//
// Epilogues: STORE (bf16 and optionally the fp32 sum), RESIDUAL
// (h = bf16(h + bf16(acc))) and SWIGLU: the tile's columns alternate 32 gate
// rows and the same 32 up rows of the weights, so one wave holds g and u of
// the same outputs (16-column MFMA tiles j and j + 2 of each 64-column group)
// and writes bf16(bf16(silu(bf16(g))) * bf16(u)).
#include "common.h"
#include "launch.h"

#include <algorithm>

namespace {


struct GemmArgs {
  const bf16_t* A;
  int lda;
  int M, K;
  GemvSeg seg[3];  // STORE / RESIDUAL: weight segments by output column
  int nseg;
  const bf16_t* gate;  // SWIGLU
  const bf16_t* up;
  bf16_t* out;
  int ldo;
  float* out32;
  int ld32;
};

__device__ __forceinline__ float silu_r(float g) { return rbf(g / (1.0f + expf(-g))); }

// Epilogue of a wave's TM x TN 16x16 tiles at rows r0.., tile columns c0..
// (c0 a multiple of 64): lane l holds column l%16 and rows 4*(l/16) + r of
// each.  GUARD: some rows lie past M (only then are stores predicated, so a
// whole tile's stores issue back to back).
template <int EPI, int TM, int TN, bool GUARD>
__device__ __forceinline__ void store_rows(const GemmArgs& a, const f32x4_t (&acc)[TM][TN], int r0,
                                           int c0, int lane) {
  const int lc = lane & 15, hrow = (lane >> 4) * 4;
  if (EPI == GEMV_RESIDUAL) {
    // the residual values of a batch of 16-row groups are loaded first (rows
    // past M re-read the last row), so the wave waits for memory once per
    // batch rather than once per row; batches of at most 112 values
    constexpr int IB = TM * 4 * TN > 112 ? TM / 2 : TM;
    static_assert(TM % IB == 0, "whole batches");
#pragma unroll
    for (int i0 = 0; i0 < TM; i0 += IB) {
      bf16_t hv[IB][4][TN];
#pragma unroll
      for (int i = 0; i < IB; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int mr = r0 + (i0 + i) * 16 + hrow + r;
          const int m = GUARD ? min(mr, a.M - 1) : mr;
#pragma unroll
          for (int j = 0; j < TN; ++j) hv[i][r][j] = a.out[(size_t)m * a.ldo + c0 + j * 16 + lc];
        }
#pragma unroll
      for (int i = 0; i < IB; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = r0 + (i0 + i) * 16 + hrow + r;
          if (GUARD && m >= a.M) continue;
#pragma unroll
          for (int j = 0; j < TN; ++j)
            a.out[(size_t)m * a.ldo + c0 + j * 16 + lc] = f2bf(bf2f(hv[i][r][j]) + rbf(acc[i0 + i][j][r]));
        }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = r0 + i * 16 + hrow + r;
      if (GUARD && m >= a.M) continue;
      if (EPI == GEMV_SWIGLU) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          if ((j & 3) >= 2) continue;  // up tiles, read with their gate tile
          const int col = c0 + j * 16;  // gate tile column; up follows at +32
          const int n = (col >> 6) * 32 + (col & 31) + lc;
          float g = rbf(acc[i][j][r]), u = rbf(acc[i][j + 2][r]);
          a.out[(size_t)m * a.ldo + n] = f2bf(silu_r(g) * u);
        }
      } else {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = c0 + j * 16 + lc;
          a.out[(size_t)m * a.ldo + n] = f2bf(acc[i][j][r]);
          if (a.out32) a.out32[(size_t)m * a.ld32 + n] = acc[i][j][r];
        }
      }
    }
  }
}

template <int EPI, int TM, int TN>
__device__ __forceinline__ void store_tile(const GemmArgs& a, const f32x4_t (&acc)[TM][TN], int r0,
                                           int c0, int lane) {
  if (r0 + TM * 16 <= a.M) store_rows<EPI, TM, TN, false>(a, acc, r0, c0, lane);
  else store_rows<EPI, TM, TN, true>(a, acc, r0, c0, lane);
}

// Workgroup b runs on XCD b % 8; tiles are handed out so that each XCD
// takes a contiguous run of tile indices, and within a run the row tiles of
// one column tile are adjacent: the weight slice of a column tile is then
// fetched into one XCD's L2 and shared by the row tiles running beside it.
__device__ __forceinline__ int xcd_tile(int b, int nt) {
  const int full = nt / 8 * 8;
  return b < full ? (b % 8) * (nt / 8) + b / 8 : b;
}

// A BM x BN block tile staged through LDS in BK-deep slices, double-buffered
// (rows padded to BK + 8 elements); each wave owns a WM x WN sub-tile of
// 16x16 MFMA tiles.  Register budget: two waves per SIMD (two workgroups per
// CU when a workgroup has four waves).
template <int BM, int BN, int WM, int WN, int EPI, int BK, int FLUSH = 0>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64, (BM / WM) * (BN / WN) <= 4 ? 2 : 1)
void gemm_kernel(GemmArgs a, int mtiles) {
  constexpr int LDK = BK + 8;   // LDS row stride (bf16): 16-byte fragment reads stay conflict-free
  constexpr int CPR = BK / 8;   // 16-byte chunks per tile row
  constexpr int NWN = BN / WN;
  constexpr int NT = (BM / WM) * NWN * 64;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int A_LD = BM * CPR / NT, B_LD = BN * CPR / NT;  // 16-byte chunks per thread
  static_assert(A_LD * NT == BM * CPR && B_LD * NT == BN * CPR, "tile / thread mismatch");
  static_assert(EPI != GEMV_SWIGLU || WN % 64 == 0, "SWIGLU pairs 32-column halves");

  extern __shared__ __attribute__((aligned(16))) bf16_t smem[];
  bf16_t* sA0 = smem;
  bf16_t* sB0 = smem + 2 * BM * LDK;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (k/v tiles 3% faster)
  const int wm = wave / NWN, wn = wave % NWN;
  const int t = xcd_tile(blockIdx.x, gridDim.x);
  const int m0 = (t % mtiles) * BM, n0 = (t / mtiles) * BN;

  // global sources of this thread's chunks
  const bf16_t* srcA[A_LD];
  const bf16_t* srcB[B_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    int c = tid + i * NT, row = c / CPR, kc = c % CPR;
    int m = min(m0 + row, a.M - 1);
    srcA[i] = a.A + (size_t)m * a.lda + kc * 8;
  }
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    int c = tid + i * NT, row = c / CPR, kc = c % CPR;
    int col = n0 + row;  // tile column
    const bf16_t* w;
    if (EPI == GEMV_SWIGLU) {
      int pair = col >> 6, half = (col >> 5) & 1, r = col & 31;
      w = (half ? a.up : a.gate) + (size_t)(pair * 32 + r) * a.K;
    } else {
      const bf16_t* W = a.seg[0].W;
      int base = a.seg[0].n_begin;
      for (int s = 1; s < a.nseg; ++s)
        if (col >= a.seg[s].n_begin) { W = a.seg[s].W; base = a.seg[s].n_begin; }
      w = W + (size_t)(col - base) * a.K;
    }
    srcB[i] = w + kc * 8;
  }
  const int st_off = (tid / CPR) * LDK + (tid % CPR) * 8;  // chunk i: + i*(NT/CPR)*LDK

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;

  // Two register sets of staged global loads: the loads of k-tile kt + 2 are
  // issued while tile kt is consumed and tile kt + 1 waits in the other set,
  // so a load has two tiles' worth of products to arrive.  Loads past the
  // last tile are clamped to it (branch-free steps; never consumed).
  u32x4_t ra[2][A_LD], rb[2][B_LD];
  auto gload = [&](int set, int kt) {
    kt = min(kt, a.K / BK - 1);
#pragma unroll
    for (int i = 0; i < A_LD; ++i) ra[set][i] = *(const u32x4_t*)(srcA[i] + kt * BK);
#pragma unroll
    for (int i = 0; i < B_LD; ++i)
      rb[set][i] = __builtin_nontemporal_load((const u32x4_t*)(srcB[i] + kt * BK));
  };
  auto lstore = [&](int set, int buf) {
    bf16_t* sA = sA0 + buf * BM * LDK;
    bf16_t* sB = sB0 + buf * BN * LDK;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) *(u32x4_t*)&sA[st_off + i * (NT / CPR) * LDK] = ra[set][i];
#pragma unroll
    for (int i = 0; i < B_LD; ++i) *(u32x4_t*)&sB[st_off + i * (NT / CPR) * LDK] = rb[set][i];
  };

  const int nk = a.K / BK;
  const int lr = lane & 15, lk = (lane >> 4) * 8;
  const int fa_off = (wm * WM + lr) * LDK + lk, fb_off = (wn * WN + lr) * LDK + lk;
  constexpr int KS = BK / 32;       // MFMA steps per k-tile
  constexpr int NMF = TM * TN;      // MFMAs per step
  constexpr int NFR = TM + TN;      // fragment reads per step
  static_assert(NFR <= NMF, "one fragment read per product");

  // one k-tile: prefetch kt + 2 into `set`, consume kt, stage kt + 1 (other set)
  auto step = [&](int kt, int set) {
    const int buf = kt & 1;
    gload(set, kt + 2);
    const bf16_t* sA = sA0 + buf * BM * LDK + fa_off;
    const bf16_t* sB = sB0 + buf * BN * LDK + fb_off;
    // Fragments of step ks + 1 are read while step ks's products run.
    bf16x8_t fa[2][TM], fb[2][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[0][i] = *(const bf16x8_t*)&sA[i * 16 * LDK];
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[0][j] = *(const bf16x8_t*)&sB[j * 16 * LDK];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < KS) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
          fa[cur ^ 1][i] = *(const bf16x8_t*)&sA[i * 16 * LDK + (ks + 1) * 32];
#pragma unroll
        for (int j = 0; j < TN; ++j)
          fb[cur ^ 1][j] = *(const bf16x8_t*)&sB[j * 16 * LDK + (ks + 1) * 32];
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
    }
    lstore(set ^ 1, buf ^ 1);
    // pinned order: the global loads first, the first step's fragment reads,
    // then each step's products interleaved with the next step's reads, the
    // staged writes riding on the last step
    __builtin_amdgcn_sched_group_barrier(0x020, A_LD + B_LD, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, NFR, 0);
#pragma unroll
    for (int ks = 0; ks < KS - 1; ++ks) {
#pragma unroll
      for (int f = 0; f < NFR; ++f) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, NMF - NFR, 0);
    }
    constexpr int NW = A_LD + B_LD;
    constexpr int NP = NW < NMF ? NW : NMF;
#pragma unroll
    for (int f = 0; f < NP; ++f) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
    }
    if (NMF > NP) __builtin_amdgcn_sched_group_barrier(0x008, NMF - NP, 0);
    if (NW > NP) __builtin_amdgcn_sched_group_barrier(0x200, NW - NP, 0);
    __syncthreads();
  };

  // FLUSH > 0: every FLUSH k-tiles the matrix unit's running sums are added
  // to fp32 totals and restarted from zero, so each chain of products
  // accumulates only FLUSH * BK terms (the matrix unit's internal additions
  // lose more than an fp32 addition per product; short chains keep their
  // error at the scale of a partial sum).
  f32x4_t mst[FLUSH ? TM : 1][FLUSH ? TN : 1];
  auto flush = [&](int kt) {
    if constexpr (FLUSH > 0) {
      if ((kt + 1) % FLUSH == 0 || kt + 1 == nk) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              mst[i][j][r] = kt + 1 == FLUSH || (kt + 1 < FLUSH && kt + 1 == nk)
                                 ? acc[i][j][r] : mst[i][j][r] + acc[i][j][r];
              acc[i][j][r] = 0.f;
            }
          }
      }
    }
  };
  gload(0, 0);
  gload(1, 1);
  lstore(0, 0);
  __syncthreads();
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    step(kt, 0);
    flush(kt);
    step(kt + 1, 1);
    flush(kt + 1);
  }
  if (kt < nk) {
    step(kt, 0);
    flush(kt);
  }

  if constexpr (FLUSH > 0) store_tile<EPI, TM, TN>(a, mst, m0 + wm * WM, n0 + wn * WN, lane);
  else store_tile<EPI, TM, TN>(a, acc, m0 + wm * WM, n0 + wn * WN, lane);
}

// ---------------------------------------------------------------------------
// 256 x BN tiles (BN = 256 or 224) on an alternating schedule.  Eight waves,
// two per SIMD, in two groups: group g (waves 4g .. 4g + 3, one per SIMD)
// owns tile columns g*BN/2 .. (g+1)*BN/2 - 1, wave q of a group rows
// 64q .. 64q + 63: a 64 x BN/2 sub-tile of 16x16 MFMA tiles.  Phases
// alternate: in one a group's waves issue nothing but products of a whole
// 64-deep k-tile from registers, while the other group's waves read their
// next k-tile's fragments from LDS and issue the copies of a later k-tile;
// then the groups swap.  The SIMD's matrix pipe is fed by one wave while its
// partner waits on memory, so the LDS reads and copies stay off the products'
// path.  BN = 224 puts 7,168-wide projections on exactly 256 tiles at
// M = 2,048 (224 tiles of 256 would leave an eighth of the CUs idle).
//
// Operand tiles go from global memory straight to LDS (16-byte LDS-direct
// loads, one KiB = 8 rows of 128 bytes per copy), double-buffered: rows of
// 64 k, chunk c of row r stored at chunk c ^ ((r >> 1) & 7), so a fragment
// read (rows l%16, one chunk per 16 lanes) touches every bank once per 16
// lanes.  A region of tile kt's buffer is refilled with tile kt + 2 as soon
// as its readers are done, by the group that is loading, so the two groups
// issue equal shares of the copies: the weight rows of group 0's columns
// (read by group 0 only) by group 1 while it reads tile kt, the activation
// rows (read by both) by group 0 in the next phase, and the weight rows of
// group 1's columns (read by group 1 only) by group 1 in its next load phase.
// The products run in the same order as gemm_kernel's, so the two give the
// same bits.

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Phase boundary: nothing is scheduled across it, this wave's LDS reads
// have completed, then all waves meet.  (__syncthreads would also wait for
// the copies in flight.)
__device__ __forceinline__ void phase_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

template <int N>
__device__ __forceinline__ void wait_copies() {  // at most N of this wave's copies in flight
  static_assert(N == 0, "wait counts in use");
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// NTW: weight copies carry the non-temporal hint (for projections whose
// activation operand is too large to stay cached beside the weight stream).
template <int EPI, int BN, bool NTW>
__global__ __launch_bounds__(512, 1) void gemm_alt_kernel(GemmArgs a, int mtiles) {
  constexpr int BM = 256, BK = 64, WM = 64, WN = BN / 2, TM = WM / 16, TN = WN / 16, KS = 2;
  constexpr int TILE = BM * BK * 2;  // bytes of an activation k-tile; LDS: A0 A1 B0 B1, TILE each
  constexpr int NCB = BN / 8, NCB0 = NCB / 2;  // weight copies per k-tile; those of group 0's columns
  static_assert(BN % 32 == 0 && BN <= BM && (EPI != GEMV_SWIGLU || WN % 64 == 0), "tile width");
  static_assert(NCB0 <= 16 && NCB0 > 12, "group 1 issues three or four copies per wave");
  extern __shared__ __attribute__((aligned(16))) bf16_t smem[];
  uint8_t* lds = (uint8_t*)smem;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int grp = wave >> 2, q = wave & 3;
  const int t = xcd_tile(blockIdx.x, gridDim.x);
  const int m0 = (t % mtiles) * BM, n0 = (t / mtiles) * BN;

  // Copy c of an operand tile covers rows 8c .. 8c + 7; lane l writes slot l:
  // row 8c + l/8, stored chunk l%8, holding logical chunk
  // (l%8) ^ ((row >> 1) & 7) = (l%8) ^ ((4(c%2) + l/16) & 7).
  const int lrow = lane >> 3;
  const uint32_t xs0 = (uint32_t)(((lane & 7) ^ ((lane >> 4) & 7)) * 16);
  const uint32_t xs1 = (uint32_t)(((lane & 7) ^ ((4 + (lane >> 4)) & 7)) * 16);
  const uint8_t* gA = (const uint8_t*)(a.A + (size_t)m0 * a.lda);
  const uint32_t rsA = (uint32_t)a.lda * 2, rsB = (uint32_t)a.K * 2;
  const uint8_t* gB[2];
  if (EPI == GEMV_SWIGLU) {  // tile columns alternate 32 gate and 32 up rows
    gB[0] = (const uint8_t*)(a.gate + (size_t)(n0 / 2) * a.K);
    gB[1] = (const uint8_t*)(a.up + (size_t)(n0 / 2) * a.K);
  } else {  // the tile lies inside one segment (boundaries are multiples of BN)
    const bf16_t* W = a.seg[0].W;
    int sb = a.seg[0].n_begin;
    for (int sg = 1; sg < a.nseg; ++sg)
      if (n0 >= a.seg[sg].n_begin) { W = a.seg[sg].W; sb = a.seg[sg].n_begin; }
    gB[0] = gB[1] = (const uint8_t*)(W + (size_t)(n0 - sb) * a.K);
  }
  const int mlast = a.M - 1 - m0;  // activation rows past M re-read the last row
  // weight copies: a lane part (two registers) plus a uniform part taken
  // through readfirstlane, so no per-copy offsets stay live in registers
  const uint32_t lb0 = (uint32_t)lrow * rsB + xs0, lb1 = (uint32_t)lrow * rsB + xs1;
  auto copy = [&](int kt, bool opA, int c) {
    const uint8_t* b;
    uint32_t go;
    if (opA) {
      b = gA;
      go = (uint32_t)min(8 * c + lrow, mlast) * rsA + ((c & 1) ? xs1 : xs0) + (uint32_t)kt * (BK * 2);
    } else {
      // tile row 8c + lrow; SWIGLU rows alternate 32 gate and 32 up rows
      const uint32_t wrow = EPI == GEMV_SWIGLU ? (uint32_t)((c >> 3) * 32 + 8 * (c & 3)) : (uint32_t)(8 * c);
      b = EPI == GEMV_SWIGLU ? gB[(c >> 2) & 1] : gB[0];
      go = ((c & 1) ? lb1 : lb0) +
           (uint32_t)__builtin_amdgcn_readfirstlane((int)(wrow * rsB + (uint32_t)kt * (BK * 2)));
    }
    const int loff = (opA ? 0 : 2 * TILE) + (kt & 1) * TILE + c * 1024;
    if (NTW && !opA) __builtin_amdgcn_global_load_lds((const void*)(b + go), (lds_ptr_t)(lds + loff), 16, 0, 2);
    else __builtin_amdgcn_global_load_lds((const void*)(b + go), (lds_ptr_t)(lds + loff), 16, 0, 0);
  };

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.f;

  // fragment of a 16-row tile: lane l reads row l%16, logical chunk
  // 4ks + l/16, stored at that ^ ((l%16 >> 1) & 7)
  const int lr = lane & 15, swz = (lr >> 1) & 7;
  uint32_t fa_off[KS], fb_off[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint32_t ch = (uint32_t)(((4 * ks + (lane >> 4)) ^ swz) * 16);
    fa_off[ks] = (uint32_t)(q * WM + lr) * 128 + ch;
    fb_off[ks] = 2 * TILE + (uint32_t)(grp * WN + lr) * 128 + ch;
  }
  bf16x8_t fa[KS][TM], fb[KS][TN];
  auto load_frags = [&](int kt) {
    const uint32_t bo = (uint32_t)(kt & 1) * TILE;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int i = 0; i < TM; ++i) fa[ks][i] = *(const bf16x8_t*)(lds + fa_off[ks] + bo + i * 16 * 128);
#pragma unroll
      for (int j = 0; j < TN; ++j) fb[ks][j] = *(const bf16x8_t*)(lds + fb_off[ks] + bo + j * 16 * 128);
    }
  };
  auto multiply = [&]() {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[ks][i], fb[ks][j], acc[i][j], 0, 0, 0);
  };

  const int nk = a.K / BK;
  // k-tiles 0 and 1: waves 0-3 copy the activation tiles, 4-7 the weights
  for (int k = 0; k < 2 && k < nk; ++k) {
    if (grp == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) copy(k, true, q * 8 + i);
    } else {
#pragma unroll
      for (int i = 0; i < (NCB + 3) / 4; ++i)
        if (q + 4 * i < NCB) copy(k, false, q + 4 * i);
    }
  }
  wait_copies<0>();
  phase_barrier();
  // Phase 2kt: group 0 multiplies tile kt; group 1 copies the weight rows of
  // group 0's columns of tile kt + 2 and of its own columns of tile kt + 1,
  // then reads tile kt's fragments.  Phase 2kt + 1: group 1 multiplies tile
  // kt; group 0 copies tile kt + 2's activation rows and reads tile kt + 1's
  // fragments.  A wave waits for its copies at the end of its next
  // multiplying phase, before the barrier that precedes the copied region's
  // first reader.
  if (grp == 0) {
    load_frags(0);
    for (int kt = 0; kt < nk; ++kt) {
      multiply();
      wait_copies<0>();
      phase_barrier();
      if (kt + 2 < nk) {
        if (kt == 0) {  // in phase 0 group 0 was still reading those rows of tile 0
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (q + 4 * i < NCB0) copy(kt + 2, false, q + 4 * i);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) copy(kt + 2, true, q * 8 + i);
      }
      if (kt + 1 < nk) load_frags(kt + 1);
      phase_barrier();
    }
  } else {
    for (int kt = 0; kt < nk; ++kt) {
      if (kt >= 1 && kt + 2 < nk) {  // group 0's weight rows of tile kt + 2
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (q + 4 * i < NCB0) copy(kt + 2, false, q + 4 * i);
      }
      if (kt >= 1 && kt + 1 < nk) {  // own weight rows of tile kt + 1
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (NCB0 + q + 4 * i < NCB) copy(kt + 1, false, NCB0 + q + 4 * i);
      }
      load_frags(kt);
      phase_barrier();
      multiply();
      wait_copies<0>();
      phase_barrier();
    }
  }

  store_tile<EPI, TM, TN>(a, acc, m0 + q * WM, n0 + grp * WN, lane);
}

template <int EPI, int BN, bool NTW>
void launch_alt_nt(const GemmArgs& a, int ncols, hipStream_t s) {
  const int mtiles = (a.M + 255) / 256;
  const int nt = (ncols / BN) * mtiles;
  const size_t lds = (size_t)4 * 256 * 64 * 2;
  static bool attr = false;  // one-time opt-in above the default dynamic LDS limit
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)gemm_alt_kernel<EPI, BN, NTW>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    attr = true;
  }
  launch_k((gemm_alt_kernel<EPI, BN, NTW>), dim3(nt), dim3(512), lds, s, a, mtiles);
}

// Weight copies are non-temporal when the activation operand exceeds 64 MB:
// measured on the 2,048 x 22,016 down-projection input (90 MB), the hint
// keeps the activations cached and saves ~6%; with the 29 MB inputs of the
// other projections it gains nothing (gate/up) or costs 2-3% (o).
template <int EPI, int BN>
void launch_alt(const GemmArgs& a, int ncols, hipStream_t s) {
  if ((size_t)a.M * a.K * 2 > ((size_t)64 << 20)) launch_alt_nt<EPI, BN, true>(a, ncols, s);
  else launch_alt_nt<EPI, BN, false>(a, ncols, s);
}

template <int BM, int BN, int WM, int WN, int EPI, int BK = 64, int FLUSH = 0>
void launch_tile(const GemmArgs& a, int ncols, hipStream_t s) {
  const int mtiles = (a.M + BM - 1) / BM;
  const int nt = (ncols / BN) * mtiles;
  const size_t lds = (size_t)2 * (BM + BN) * (BK + 8) * sizeof(bf16_t);
  static bool attr = false;  // one-time opt-in above the default dynamic LDS limit
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)gemm_kernel<BM, BN, WM, WN, EPI, BK, FLUSH>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    attr = true;
  }
  launch_k((gemm_kernel<BM, BN, WM, WN, EPI, BK, FLUSH>), dim3(nt),
                     dim3((BM / WM) * (BN / WN) * 64), lds, s, a, mtiles);
}

}  // namespace

// Compute units of the current device (tiles are handed out in rounds of
// one workgroup per CU).
static int cu_count() {
  static int n = 0;
  if (!n) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
      n = 256;
  }
  return n;
}

// Tile shapes for a launch.  Relative time of a round (one workgroup per
// CU), in full rounds of 256 x 256 tiles at the same K, measured at
// M = 2,048: 256 x 224 0.875, 256 x 128 (eight waves of 64 x 64) 0.70,
// 128 x 128 0.45; a partial round with a fraction f of the CUs busy costs
// (0.67 + 0.33 f) of a full one (fewer busy CUs run at a higher clock).
enum GemmShape { SH_ALT256, SH_ALT224, SH_256X128, SH_128X128 };

static double round_cost(long tiles, int cus, double per_round) {
  const long full = tiles / cus, rest = tiles % cus;
  return per_round * ((double)full + (rest ? 0.67 + 0.33 * (double)rest / cus : 0.0));
}

// Cheapest shape for ncols tile columns (a multiple of 128) whose weight
// segments start at the relative columns bnd[0..nb): the alternating
// kernels need every segment boundary on a tile boundary, 256 x 224 is not
// used for SWIGLU (its gate/up pairs span 64 columns).
static GemmShape best_shape(int M, int ncols, bool swiglu, const int* bnd, int nb, int cus,
                            double* cost) {
  auto on = [&](int w) {
    if (ncols % w) return false;
    for (int i = 0; i < nb; ++i)
      if (bnd[i] % w) return false;
    return true;
  };
  const long mt = (M + 255) / 256, mt2 = (M + 127) / 128;
  GemmShape sh = SH_128X128;
  double c = round_cost(mt2 * (ncols / 128), cus, 0.45), x;
  if ((x = round_cost(mt * (ncols / 128), cus, 0.70)) < c) { c = x; sh = SH_256X128; }
  if (on(256) && (x = round_cost(mt * (ncols / 256), cus, 1.0)) < c) { c = x; sh = SH_ALT256; }
  if (!swiglu && on(224) && (x = round_cost(mt * (ncols / 224), cus, 0.875)) < c) { c = x; sh = SH_ALT224; }
  *cost = c;
  return sh;
}

template <int EPI>
static void launch_shape(GemmShape sh, const GemmArgs& a, int ncols, hipStream_t s) {
  if (sh == SH_ALT256) launch_alt<EPI, 256>(a, ncols, s);
  else if (sh == SH_256X128) launch_tile<256, 128, 64, 64, EPI>(a, ncols, s);
  else if (sh == SH_128X128) launch_tile<128, 128, 64, 64, EPI>(a, ncols, s);
  else if constexpr (EPI != GEMV_SWIGLU) launch_alt<EPI, 224>(a, ncols, s);
}

// The output columns [c0, c1) of a as a launch of its own: output pointers
// moved by c0, the segments overlapping the range clipped and rebased.
static GemmArgs column_range(const GemmArgs& a, int c0, int c1) {
  GemmArgs r = a;
  r.nseg = 0;
  for (int i = 0; i < a.nseg; ++i) {
    const GemvSeg& g = a.seg[i];
    const int b = std::max(g.n_begin, c0), e = std::min(g.n_end, c1);
    if (b >= e) continue;
    r.seg[r.nseg++] = GemvSeg{g.W + (size_t)(b - g.n_begin) * a.K, b - c0, e - c0};
  }
  r.out = a.out + c0;
  if (a.out32) r.out32 = a.out32 + c0;
  return r;
}

// ncols: tile columns (N, or 2F for SWIGLU); a multiple of 128.  The whole
// width runs as one launch of the cheapest shape, or (STORE and RESIDUAL)
// as two launches split at a weight segment boundary when that is cheaper:
// the q/k/v projection of the 33B shape (9,216 columns) runs q on 256 x 224
// tiles (256 of them at M = 2,048) and k, v on 128 x 128 tiles instead of
// 288 tiles of 256 x 256.  The split of K into 64-deep tiles and 32-deep
// MFMA steps, and so every output's bits, is the same for all shapes.
template <int EPI>
static void launch_epi(const GemmArgs& a, int ncols, hipStream_t s) {
  const int cus = cu_count();
  int bnd[3], nb = 0;
  if (EPI != GEMV_SWIGLU)
    for (int i = 0; i < a.nseg; ++i)
      if (a.seg[i].n_begin > 0) bnd[nb++] = a.seg[i].n_begin;
  double best;
  GemmShape sh = best_shape(a.M, ncols, EPI == GEMV_SWIGLU, bnd, nb, cus, &best);
  int split = 0;
  GemmShape sl = sh, sr = sh;
  for (int i = 0; i < nb; ++i) {
    const int b = bnd[i];
    if (b % 128 || b >= ncols) continue;
    int lb[3], ln = 0, rb[3], rn = 0;
    for (int j = 0; j < nb; ++j) {
      if (bnd[j] < b) lb[ln++] = bnd[j];
      else if (bnd[j] > b) rb[rn++] = bnd[j] - b;
    }
    double cl, cr;
    const GemmShape l = best_shape(a.M, b, false, lb, ln, cus, &cl);
    const GemmShape r = best_shape(a.M, ncols - b, false, rb, rn, cus, &cr);
    if (cl + cr + 0.02 < best) { best = cl + cr + 0.02; split = b; sl = l; sr = r; }
  }
  if (!split) {
    launch_shape<EPI>(sh, a, ncols, s);
    return;
  }
  launch_shape<EPI>(sl, column_range(a, 0, split), split, s);
  launch_shape<EPI>(sr, column_range(a, split, ncols), ncols - split, s);
}

// Exact form: 256 x 128 tiles of the register-staged kernel whose running
// sums restart every two k-tiles (128 terms) into fp32 totals; every output
// still sums its k-tiles in increasing order.
template <int EPI>
static void launch_exact(const GemmArgs& a, int ncols, hipStream_t s) {
  launch_tile<256, 128, 64, 64, EPI, 64, 2>(a, ncols, s);
}

void launch_gemm(int epi, const void* A, int lda, int M, int K, const GemvSeg* seg, int nseg,
                 const void* gate, const void* up, void* out, int ldo, float* out32, int ld32,
                 int ncols, bool exact, hipStream_t s) {
  GemmArgs a{};
  a.A = (const bf16_t*)A;
  a.lda = lda;
  a.M = M;
  a.K = K;
  for (int i = 0; i < 3; ++i) a.seg[i] = (seg && i < nseg) ? seg[i] : GemvSeg{nullptr, 0, 0};
  a.nseg = nseg;
  a.gate = (const bf16_t*)gate;
  a.up = (const bf16_t*)up;
  a.out = (bf16_t*)out;
  a.ldo = ldo;
  a.out32 = out32;
  a.ld32 = ld32;
  if (exact) {
    if (epi == GEMV_STORE) launch_exact<GEMV_STORE>(a, ncols, s);
    else if (epi == GEMV_RESIDUAL) launch_exact<GEMV_RESIDUAL>(a, ncols, s);
    else launch_exact<GEMV_SWIGLU>(a, ncols, s);
    return;
  }
  if (epi == GEMV_STORE) launch_epi<GEMV_STORE>(a, ncols, s);
  else if (epi == GEMV_RESIDUAL) launch_epi<GEMV_RESIDUAL>(a, ncols, s);
  else launch_epi<GEMV_SWIGLU>(a, ncols, s);
}
