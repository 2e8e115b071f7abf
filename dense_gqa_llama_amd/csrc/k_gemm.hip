// Prompt-chunk projections on the bf16 matrix cores: C[m][n] = sum_k A[m][k]
// W[n][k] for chunks of up to 2,048 rows, fp32 accumulation rounded once to
// bf16 (pull request "llama: Nanbeige4.3-33B on Metal, the bf16 release
// served as published", section "How": prompt chunks of up to 2,048 rows on
// the matrix units).
//
// Both operands are K-contiguous: activations [M][K] and published weights
// [N][K].  A BM x BN block tile is staged through LDS in BK = 64 slices,
// double-buffered; each wave owns a WM x WN sub-tile made of 32x32 output
// tiles of v_mfma_f32_32x32x16_bf16.  Lane l of an MFMA reads row l%32 and 8
// consecutive k at 8*(l/32) of each operand (one 16-byte LDS read), and holds
// output rows 8*(j/4) + 4*(l/32) + j%4 of column l%32 in its accumulators.
// Every output's K loop runs in the same order whatever M is.
//
// Epilogues: STORE (bf16 and optionally the fp32 sum), RESIDUAL
// (h = bf16(h + bf16(acc))) and SWIGLU: the tile's columns alternate 32 gate
// rows and the same 32 up rows of the weights, so one wave holds g and u of
// the same outputs and writes bf16(bf16(silu(bf16(g))) * bf16(u)).
#include "common.h"
#include "launch.h"

namespace {

constexpr int BK = 64;
constexpr int LDK = BK + 8;  // LDS row stride (bf16): rows land 4 banks apart

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

// Workgroup b runs on XCD b % 8; tiles are handed out so that each XCD
// takes a contiguous run of tile indices, and within a run the row tiles of
// one column tile are adjacent: the weight slice of a column tile is then
// fetched into one XCD's L2 and shared by the row tiles running beside it.
__device__ __forceinline__ int xcd_tile(int b, int nt) {
  const int full = nt / 8 * 8;
  return b < full ? (b % 8) * (nt / 8) + b / 8 : b;
}

template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64) void gemm_kernel(GemmArgs a, int mtiles) {
  constexpr int NWN = BN / WN;
  constexpr int NT = (BM / WM) * NWN * 64;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int A_LD = BM * 8 / NT, B_LD = BN * 8 / NT;  // 16-byte chunks per thread
  static_assert(A_LD * NT == BM * 8 && B_LD * NT == BN * 8, "tile / thread mismatch");
  static_assert(EPI != GEMV_SWIGLU || WN % 64 == 0, "SWIGLU pairs 32-column tiles");

  extern __shared__ __attribute__((aligned(16))) bf16_t smem[];
  bf16_t* sA0 = smem;
  bf16_t* sB0 = smem + 2 * BM * LDK;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / NWN, wn = wave % NWN;
  const int t = xcd_tile(blockIdx.x, gridDim.x);
  const int m0 = (t % mtiles) * BM, n0 = (t / mtiles) * BN;

  // global sources of this thread's chunks
  const bf16_t* srcA[A_LD];
  const bf16_t* srcB[B_LD];
#pragma unroll
  for (int i = 0; i < A_LD; ++i) {
    int c = tid + i * NT, row = c >> 3, kc = c & 7;
    int m = min(m0 + row, a.M - 1);
    srcA[i] = a.A + (size_t)m * a.lda + kc * 8;
  }
#pragma unroll
  for (int i = 0; i < B_LD; ++i) {
    int c = tid + i * NT, row = c >> 3, kc = c & 7;
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
  const int st_off = (tid >> 3) * LDK + (tid & 7) * 8;  // LDS offset of chunk i: + i*(NT/8)*LDK

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  u32x4_t ra[A_LD], rb[B_LD];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < A_LD; ++i) ra[i] = *(const u32x4_t*)(srcA[i] + kt * BK);
#pragma unroll
    for (int i = 0; i < B_LD; ++i) rb[i] = __builtin_nontemporal_load((const u32x4_t*)(srcB[i] + kt * BK));
  };
  auto lstore = [&](int buf) {
    bf16_t* sA = sA0 + buf * BM * LDK;
    bf16_t* sB = sB0 + buf * BN * LDK;
#pragma unroll
    for (int i = 0; i < A_LD; ++i) *(u32x4_t*)&sA[st_off + i * (NT / 8) * LDK] = ra[i];
#pragma unroll
    for (int i = 0; i < B_LD; ++i) *(u32x4_t*)&sB[st_off + i * (NT / 8) * LDK] = rb[i];
  };

  const int nk = a.K / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  const int lr = lane & 31, lk = (lane >> 5) * 8;
  const int fa_off = (wm * WM + lr) * LDK + lk, fb_off = (wn * WN + lr) * LDK + lk;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const bf16_t* sA = sA0 + buf * BM * LDK + fa_off;
    const bf16_t* sB = sB0 + buf * BN * LDK + fb_off;
    // fragments of step kk + 16 are read while step kk's products run
    bf16x8_t fa[2][TM], fb[2][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) fa[0][i] = *(const bf16x8_t*)&sA[i * 32 * LDK];
#pragma unroll
    for (int j = 0; j < TN; ++j) fb[0][j] = *(const bf16x8_t*)&sB[j * 32 * LDK];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < BK / 16) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
          fa[cur ^ 1][i] = *(const bf16x8_t*)&sA[i * 32 * LDK + (ks + 1) * 16];
#pragma unroll
        for (int j = 0; j < TN; ++j)
          fb[cur ^ 1][j] = *(const bf16x8_t*)&sB[j * 32 * LDK + (ks + 1) * 16];
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[cur][i], fb[cur][j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue
  const int hrow = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm * WM + i * 32 + 8 * (r >> 2) + hrow + (r & 3);
      if (m >= a.M) continue;
      if (EPI == GEMV_SWIGLU) {
#pragma unroll
        for (int j = 0; j < TN; j += 2) {
          const int col = n0 + wn * WN + j * 32;  // gate tile column; up follows at +32
          const int n = (col >> 6) * 32 + lr;
          float g = rbf(acc[i][j][r]), u = rbf(acc[i][j + 1][r]);
          a.out[(size_t)m * a.ldo + n] = f2bf(silu_r(g) * u);
        }
      } else {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = n0 + wn * WN + j * 32 + lr;
          const float v = acc[i][j][r];
          bf16_t* o = a.out + (size_t)m * a.ldo + n;
          if (EPI == GEMV_STORE) {
            *o = f2bf(v);
            if (a.out32) a.out32[(size_t)m * a.ld32 + n] = v;
          } else {
            *o = f2bf(bf2f(*o) + rbf(v));
          }
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN, int EPI>
void launch_tile(const GemmArgs& a, int ncols, hipStream_t s) {
  const int mtiles = (a.M + BM - 1) / BM;
  const int nt = (ncols / BN) * mtiles;
  const size_t lds = (size_t)2 * (BM + BN) * LDK * sizeof(bf16_t);
  static bool attr = false;  // one-time opt-in above the default dynamic LDS limit
  if (!attr) {
    (void)hipFuncSetAttribute((const void*)gemm_kernel<BM, BN, WM, WN, EPI>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    attr = true;
  }
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, EPI>), dim3(nt),
                     dim3((BM / WM) * (BN / WN) * 64), lds, s, a, mtiles);
}

}  // namespace

// ncols: tile columns (N, or 2F for SWIGLU); a multiple of 128.  Widths that
// are multiples of 256 take 256 x 256 tiles (eight waves of 128 x 64), which
// halve the LDS and L2 traffic per product of the 128 x 128 tiles; the split
// of K into 16-deep MFMA steps, and so every output's bits, is the same for
// both.
void launch_gemm(int epi, const void* A, int lda, int M, int K, const GemvSeg* seg, int nseg,
                 const void* gate, const void* up, void* out, int ldo, float* out32, int ld32,
                 int ncols, hipStream_t s) {
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
  const bool big = ncols % 256 == 0;
  if (epi == GEMV_STORE) {
    if (big) launch_tile<256, 256, 128, 64, GEMV_STORE>(a, ncols, s);
    else launch_tile<128, 128, 64, 64, GEMV_STORE>(a, ncols, s);
  } else if (epi == GEMV_RESIDUAL) {
    if (big) launch_tile<256, 256, 128, 64, GEMV_RESIDUAL>(a, ncols, s);
    else launch_tile<128, 128, 64, 64, GEMV_RESIDUAL>(a, ncols, s);
  } else {
    if (big) launch_tile<256, 256, 128, 64, GEMV_SWIGLU>(a, ncols, s);
    else launch_tile<128, 128, 64, 64, GEMV_SWIGLU>(a, ncols, s);
  }
}
