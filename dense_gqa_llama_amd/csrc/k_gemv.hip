// Decode row projections: y[r][n] = sum_k W[n][k] x[r][k] for windows of
// 1..16 rows, fp32 sums rounded once to bf16 (pull request "llama:
// Nanbeige4.3-33B on Metal, the bf16 release served as published", section
// "How": decode windows with fp32 sums rounded once).
//
// HBM-bound: every weight byte is read once per step.  Each wave owns a few
// output rows n; lane l reads W[n][8l + 512j .. +8] as one 16-byte load (a
// wave reads 1 KiB of a row per step, fully coalesced) and accumulates with
// v_dot2c_f32_bf16 into per-(n, r) fp32 partials, then a fixed xor butterfly
// sums the 64 lanes.  The order of every partial sum depends only on K, never
// on the window size R or on the batch, so a row computed inside a 16-row
// window equals the same row computed alone, bit for bit.
#include "common.h"
#include "launch.h"

// Weight rows are streamed once per step: nontemporal loads.
#ifndef GEMV_WLOAD
#define GEMV_WLOAD(p) __builtin_nontemporal_load(p)
#endif

struct GemvArgs {
  GemvSeg seg[3];
  int nseg;
  int K;
  const bf16_t* x;
  int ldx;
  bf16_t* out;
  int ldo;
  float* out32;
  int ld32;
  // QKV_ROPE: rows of this launch are rows row0.. of the pass described by tab
  RowTable tab;
  const float2* rope;  // [pass rows][d/2] (cos, sin) as bf16 values
  int nq, nkv, d, row0;
  // NORM: the input rows are raw residuals, normalised here with this weight
  const bf16_t* normw;
  float eps;
  // 16-byte vectors per row of each chunk of the input rows staged in LDS (a
  // multiple of the loop step, or at least K/8: one chunk)
  int xcv;
};

__device__ __forceinline__ float silu_bf16(float g) { return rbf(g / (1.0f + expf(-g))); }

constexpr int ilog2(int n) { return n <= 1 ? 0 : 1 + ilog2(n / 2); }

// Sums over the 64 lanes of NG groups of KG partials (v[g][k]), scattered:
// afterwards v[0][0..KG-1] holds the sums of group lane >> (6 - log2 NG).
// Each exchange halves the groups a lane carries (it keeps one half and adds
// its partner's copy of it), lane bits 32, 16, 8, ... in turn, then the rest
// of the butterfly runs on the kept group: every sum is associated exactly as
// wave_sum's (xor 32, 16, 8, 4, 2, 1), own partial first, with NG - 1 + 6 -
// log2 NG exchanges per partial instead of 6 NG.
template <int NG, int KG>
__device__ __forceinline__ void reduce_scatter(float (&v)[NG][KG], int lane) {
  constexpr int K = ilog2(NG);
  static_assert((1 << K) == NG && K <= 6, "power-of-two group count up to 64");
#pragma unroll
  for (int t = 0; t < K; ++t) {
    const int m = 32 >> t;
    const int half = (NG >> t) / 2;
    const bool up = lane & m;
#pragma unroll
    for (int j = 0; j < NG / 2; ++j) {
      if (j >= half) break;
#pragma unroll
      for (int k = 0; k < KG; ++k) {
        const float lo = v[j][k], hi = v[j + half][k];
        const float keep = up ? hi : lo, send = up ? lo : hi;
        v[j][k] = keep + __shfl_xor(send, m, WAVE);
      }
    }
  }
#pragma unroll
  for (int m = 32 >> K; m >= 1; m >>= 1)
#pragma unroll
    for (int k = 0; k < KG; ++k) v[0][k] += __shfl_xor(v[0][k], m, WAVE);
}

// NR weight rows per wave; for SWIGLU the first NR/2 come from the gate
// matrix and the last NR/2 from the up matrix, for the same output columns.
// WPB waves per workgroup (NT threads) share the staged input rows.
template <int R, int NR, int EPI, bool NORM, int P, int WPB>
__global__ __launch_bounds__(64 * WPB) void gemv_kernel(GemvArgs a) {
  constexpr int NT = 64 * WPB;
  extern __shared__ u32x4_t sx[];  // a chunk of the (normalised) input rows, [R][xcv]
  constexpr int COLS = EPI == GEMV_SWIGLU ? NR / 2 : NR;
  static_assert(EPI != GEMV_QKV_ROPE || NR == 4, "rotation pairs come four rows per wave");
  // the wave index as a scalar: row pointers and chunk bounds in scalar
  // registers (the looped model's gate/up 22.6 -> 21.4 us, same bits).  For
  // windows of 15-16 rows it stays a vector value: the kernel then holds
  // enough registers for three waves per SIMD instead of four, which those
  // windows run faster (16 rows: 407 against 419 us per 33B layer).
  const int wave = R >= 15 ? (int)(threadIdx.x >> 6) : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int n0 = (blockIdx.x * WPB + wave) * COLS;  // first output column of this wave

  const u32x4_t* wp[NR];
  int nloc = n0;
  int head = 0, i0 = 0;
  if (EPI == GEMV_QKV_ROPE) {
    // wave -> head and the rotation pairs (i0, i0 + d/2), (i0 + 1, i0 + 1 + d/2)
    const int half = a.d >> 1, per_head = half >> 1;
    const int wv = blockIdx.x * WPB + wave;
    head = wv / per_head;
    i0 = 2 * (wv % per_head);
    const bf16_t* W;
    int hl;
    if (head < a.nq) { W = a.seg[0].W; hl = head; }
    else if (head < a.nq + a.nkv) { W = a.seg[1].W; hl = head - a.nq; }
    else { W = a.seg[2].W; hl = head - a.nq - a.nkv; }
    const int base = hl * a.d + i0;
    const int rows4[4] = {base, base + 1, base + half, base + half + 1};
#pragma unroll
    for (int i = 0; i < NR; ++i) wp[i] = (const u32x4_t*)(W + (size_t)rows4[i] * a.K);
  } else if (EPI == GEMV_SWIGLU) {
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      const bf16_t* W = i < COLS ? a.seg[0].W : a.seg[1].W;
      wp[i] = (const u32x4_t*)(W + (size_t)(n0 + (i % COLS)) * a.K);
    }
  } else {
    const bf16_t* W = a.seg[0].W;
    int base = a.seg[0].n_begin;
    for (int s = 1; s < a.nseg; ++s)
      if (n0 >= a.seg[s].n_begin) { W = a.seg[s].W; base = a.seg[s].n_begin; }
    nloc = n0 - base;
#pragma unroll
    for (int i = 0; i < NR; ++i) wp[i] = (const u32x4_t*)(W + (size_t)(nloc + i) * a.K);
  }

  float acc[NR][R];
#pragma unroll
  for (int i = 0; i < NR; ++i)
#pragma unroll
    for (int r = 0; r < R; ++r) acc[i][r] = 0.f;

  const int nv = a.K >> 3;
  const u32x4_t* xb = (const u32x4_t*)a.x;
  const int xs = a.ldx >> 3;
  const u32x4_t* nw = (const u32x4_t*)a.normw;
  const int cv = a.xcv;
  const bool whole = cv >= nv;
  constexpr int RP = R <= 1 ? 1 : R <= 2 ? 2 : R <= 4 ? 4 : R <= 8 ? 8 : 16;
  // q/k: the lane that stores row r's rotated outputs reads their (cos, sin)
  // now, so the epilogue waits on no memory.
  float2 rc0 = {0.f, 0.f}, rc1 = {0.f, 0.f};
  if (EPI == GEMV_QKV_ROPE && head < a.nq + a.nkv) {
    const int r = lane >> (6 - ilog2(RP));
    if (r < R) {
      const size_t t = (size_t)(a.row0 + r) * (a.d >> 1) + i0;
      rc0 = a.rope[t];
      rc1 = a.rope[t + 1];
    }
  }
  // With the norm fused and whole input rows of at most XPRE vectors per
  // thread, the rows and the norm weight are read before the weight
  // prefetch: they arrive first, so the rows are staged and normalised while
  // the first weight vectors are still in flight.
  constexpr int XPRE = 4;
  const int tot0 = R * nv;
  const bool pre = NORM && whole && tot0 <= XPRE * NT;
  u32x4_t xpre[NORM ? XPRE : 1] = {}, gpre[NORM ? XPRE : 1] = {};
  if (NORM && pre) {
#pragma unroll
    for (int j = 0; j < XPRE; ++j) {
      const int i = threadIdx.x + NT * j;
      if (i < tot0) {
        const int r = i / nv, vv = i - r * nv;
        xpre[j] = xb[r * xs + vv];
        gpre[j] = nw[vv];
      }
    }
  }
  // Software pipeline, P steps deep: the weight vectors of the next P steps
  // are in flight while this step's are consumed; the first loads are issued
  // before the input rows are staged, so the staging overlaps them.  Every
  // load is issued unconditionally (past the end a lane re-reads the row's
  // last vector), so the loads in flight never depend on the lane and the
  // waits stay exact.  The partial sums still take the vectors v = lane,
  // lane + 64, ... in order.
  u32x4_t wq[P][NR];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int v = min(lane + p * WAVE, nv - 1);
#pragma unroll
    for (int i = 0; i < NR; ++i) wq[p][i] = GEMV_WLOAD(wp[i] + v);
  }
  // The input rows are staged in LDS a chunk of xcv vectors at a time, the
  // whole rows when they fit: every wave walks the same steps, so the chunk
  // boundaries and their barriers are uniform.  With NORM and whole rows the
  // norm factors are summed from LDS and the rows normalised in place; with
  // chunks, wave r first sums row r from memory and each chunk is normalised
  // as it is staged.  Both take the same binary64 norm arithmetic.
  __shared__ double srs[NORM ? R : 1];
  if (NORM && pre) {
#pragma unroll
    for (int j = 0; j < XPRE; ++j) {
      const int i = threadIdx.x + NT * j;
      if (i < tot0) sx[i] = xpre[j];
    }
    __syncthreads();
    if (wave < R) {
      const double rs = row_inv_rms_lds(sx + wave * cv, a.K, a.eps);
      if (lane == 0) srs[wave] = rs;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < XPRE; ++j) {
      const int i = threadIdx.x + NT * j;
      if (i < tot0) sx[i] = norm8(xpre[j], gpre[j], srs[i / nv]);
    }
    __syncthreads();
  }
  if (NORM && !whole) {
    if (wave < R) {
      const double rs = row_inv_rms(a.x + (size_t)wave * a.ldx, a.K, a.eps);
      if (lane == 0) srs[wave] = rs;
    }
    __syncthreads();
  }
  int c0 = 0;
  for (int base = 0; base < nv; base += P * WAVE) {
    if (base % cv == 0 && !(NORM && pre)) {
      if (base) __syncthreads();  // the previous chunk's readers are done
      const int cn = min(cv, nv - base), tot = R * cn;
      // XU vectors per thread and pass; past the end a thread repeats the
      // last vector (the same value to the same slot)
      constexpr int XU = NORM ? 2 : 4;
      for (int i0 = threadIdx.x; i0 < tot; i0 += XU * NT) {
        u32x4_t t[XU], g[XU];
        int o[XU], rr[XU];
#pragma unroll
        for (int j = 0; j < XU; ++j) {
          const int i = min(i0 + NT * j, tot - 1);
          const int r = i / cn, vv = i - r * cn;
          t[j] = xb[r * xs + base + vv];
          if (NORM && !whole) g[j] = nw[base + vv];
          o[j] = r * cv + vv;
          rr[j] = r;
        }
#pragma unroll
        for (int j = 0; j < XU; ++j) sx[o[j]] = NORM && !whole ? norm8(t[j], g[j], srs[rr[j]]) : t[j];
      }
      __syncthreads();
      if (NORM && whole) {
        if (wave < R) {
          const double rs = row_inv_rms_lds(sx + wave * cv, a.K, a.eps);
          if (lane == 0) srs[wave] = rs;
        }
        __syncthreads();
        for (int i0 = threadIdx.x; i0 < tot; i0 += 4 * NT) {
          u32x4_t g[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) g[j] = nw[min(i0 + NT * j, tot - 1) % cn];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int i = i0 + NT * j;
            if (i < tot) sx[i] = norm8(sx[i], g[j], srs[i / cn]);
          }
        }
        __syncthreads();
      }
      c0 = base;
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int v = base + p * WAVE + lane;
      u32x4_t w[NR];
#pragma unroll
      for (int i = 0; i < NR; ++i) w[i] = wq[p][i];
      const int vn = min(v + P * WAVE, nv - 1);
#pragma unroll
      for (int i = 0; i < NR; ++i) wq[p][i] = GEMV_WLOAD(wp[i] + vn);
      if (v < nv) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const u32x4_t xv = sx[r * cv + (v - c0)];
#pragma unroll
          for (int i = 0; i < NR; ++i) {
            float t = acc[i][r];
            t = dot2(w[i].x, xv.x, t);
            t = dot2(w[i].y, xv.y, t);
            t = dot2(w[i].z, xv.z, t);
            t = dot2(w[i].w, xv.w, t);
            acc[i][r] = t;
          }
        }
      }
    }
  }
  // Lane sums, scattered so that one lane holds each output's sums (rows
  // padded to a power of two with zeros), then one store per lane.
  if (EPI == GEMV_QKV_ROPE) {
    // one group per row: its four outputs (two rotation pairs) in one lane
    float v[RP][4];
#pragma unroll
    for (int r = 0; r < RP; ++r)
#pragma unroll
      for (int k = 0; k < 4; ++k) v[r][k] = r < R ? acc[k][r] : 0.f;
    reduce_scatter<RP, 4>(v, lane);
    constexpr int SH = 6 - ilog2(RP);
    const int r = lane >> SH;
    if (r < R && (lane & ((1 << SH) - 1)) == 0) {
      const int rt = a.row0 + r;
      const int seq = rt / a.tab.rows_per_seq;
      const int p = a.tab.pos0[seq] + rt % a.tab.rows_per_seq;
      const int half = a.d >> 1, kvd = a.nkv * a.d;
      const float x0 = rbf(v[0][0]), x1 = rbf(v[0][1]);
      const float y0 = rbf(v[0][2]), y1 = rbf(v[0][3]);
      bf16_t* dst;
      if (head >= a.nq + a.nkv) {  // values: no rotation
        dst = a.tab.v[seq] + (size_t)p * kvd + (head - a.nq - a.nkv) * a.d + i0;
        dst[0] = f2bf(x0);
        dst[1] = f2bf(x1);
        dst[half] = f2bf(y0);
        dst[half + 1] = f2bf(y1);
      } else {
        dst = head < a.nq ? a.out + (size_t)rt * a.ldo + head * a.d + i0
                          : a.tab.k[seq] + (size_t)p * kvd + (head - a.nq) * a.d + i0;
        const float2 c0 = rc0, c1 = rc1;
        dst[0] = f2bf(rbf(x0 * c0.x) + rbf(-y0 * c0.y));
        dst[half] = f2bf(rbf(y0 * c0.x) + rbf(x0 * c0.y));
        dst[1] = f2bf(rbf(x1 * c1.x) + rbf(-y1 * c1.y));
        dst[half + 1] = f2bf(rbf(y1 * c1.x) + rbf(x1 * c1.y));
      }
    }
    return;
  }

  // one group per (column c, row r): for SWIGLU the gate and up sums
  constexpr int KG = EPI == GEMV_SWIGLU ? 2 : 1;
  constexpr int NG = COLS * RP;
  float v[NG][KG];
#pragma unroll
  for (int c = 0; c < COLS; ++c)
#pragma unroll
    for (int r = 0; r < RP; ++r) {
      v[c * RP + r][0] = r < R ? acc[c][r] : 0.f;
      if (KG == 2) v[c * RP + r][KG - 1] = r < R ? acc[c + COLS][r] : 0.f;
    }
  reduce_scatter<NG, KG>(v, lane);
  constexpr int SH = 6 - ilog2(NG);
  const int gi = lane >> SH, c = gi / RP, r = gi % RP;
  if (r < R && (lane & ((1 << SH) - 1)) == 0) {
    const int n = n0 + c;
    if (EPI == GEMV_STORE) {
      a.out[(size_t)r * a.ldo + n] = f2bf(v[0][0]);
      if (a.out32) a.out32[(size_t)r * a.ld32 + n] = v[0][0];
    } else if (EPI == GEMV_RESIDUAL) {
      bf16_t* h = a.out + (size_t)r * a.ldo + n;
      *h = f2bf(bf2f(*h) + rbf(v[0][0]));
    } else {
      float g = rbf(v[0][0]), u = rbf(v[0][KG - 1]);
      a.out[(size_t)r * a.ldo + n] = f2bf(silu_bf16(g) * u);
    }
  }
}

// Input rows staged in LDS: whole rows for one-row steps up to 64 KB, for
// normalised windows up to GEMV_NORM_WHOLE_BYTES; otherwise chunks of at most
// 32 KB (a multiple of the loop step).
constexpr int GEMV_XLDS_BYTES = 64 * 1024;
constexpr int GEMV_XCHUNK_BYTES = 32 * 1024;
constexpr int GEMV_NORM_WHOLE_BYTES = 32 * 1024;

template <int R, int EPI, bool NORM>
static void launch_r(GemvArgs a, int N, hipStream_t s) {
  // Four weight rows per wave; the prefetch depth is four steps for one-row
  // steps and two for windows (register budget of the R*4 partials).
  constexpr int NR = 4;
  constexpr int P = R == 1 ? 4 : 2;
  constexpr int COLS = EPI == GEMV_SWIGLU ? NR / 2 : NR;
  const int grid = N / (4 * COLS);
  const int nv = a.K / 8;
  int cv;
  const size_t rows_bytes = (size_t)R * a.K * 2;
  if ((R == 1 && rows_bytes <= GEMV_XLDS_BYTES) || (NORM && rows_bytes <= GEMV_NORM_WHOLE_BYTES)) {
    cv = nv;
  } else {
    cv = GEMV_XCHUNK_BYTES / (16 * R) / (P * WAVE) * (P * WAVE);
    if (cv >= nv) cv = nv;
  }
  a.xcv = cv;
  const size_t xbytes = (size_t)R * cv * 16;
  // A one-row projection with fewer than 256 workgroups of four waves (the
  // 3B-shaped model's o and down: 192) would leave CUs idle: it runs as
  // one-wave workgroups instead, every wave doing the same arithmetic (measured
  // on that model: down 17.3 -> 15.2 us, decode 308 -> 317 tok/s).
  if (R == 1 && grid < 256)
    launch_k((gemv_kernel<R, NR, EPI, NORM, P, 1>), dim3(grid * 4), dim3(64), xbytes, s, a);
  else
    launch_k((gemv_kernel<R, NR, EPI, NORM, P, 4>), dim3(grid), dim3(256), xbytes, s, a);
}

// Inputs are normalised inside the projection for windows of up to
// GEMV_NORM_ROWS rows; larger windows arrive normalised by rmsnorm_kernel
// (same bits: the norm is binary64, correctly rounded).
template <int EPI>
static void launch_epi(int rows, const GemvArgs& a, int N, hipStream_t s) {
  if (a.normw) {
    switch (rows) {
      case 1: launch_r<1, EPI, true>(a, N, s); break;
      case 2: launch_r<2, EPI, true>(a, N, s); break;
      case 3: launch_r<3, EPI, true>(a, N, s); break;
      case 4: launch_r<4, EPI, true>(a, N, s); break;
      default: break;
    }
    return;
  }
  switch (rows) {
#define CASE(R) \
  case R: launch_r<R, EPI, false>(a, N, s); break;
    CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8)
    CASE(9) CASE(10) CASE(11) CASE(12) CASE(13) CASE(14) CASE(15) CASE(16)
#undef CASE
    default: break;
  }
}

// Column counts must be multiples of 16 (every served width is a multiple of
// 128), so no wave straddles a segment or the end.
void launch_gemv(int epi, const GemvSeg* seg, int nseg, int N, int K, const void* x, int ldx,
                 int rows, void* out, int ldo, float* out32, int ld32, const void* normw,
                 float eps, hipStream_t s) {
  GemvArgs a;
  for (int i = 0; i < 3; ++i) a.seg[i] = i < nseg ? seg[i] : seg[0];
  a.nseg = nseg;
  a.K = K;
  a.x = (const bf16_t*)x;
  a.ldx = ldx;
  a.out = (bf16_t*)out;
  a.ldo = ldo;
  a.out32 = out32;
  a.ld32 = ld32;
  a.rope = nullptr;
  a.nq = a.nkv = a.d = a.row0 = 0;
  a.normw = rows <= GEMV_NORM_ROWS ? (const bf16_t*)normw : nullptr;
  a.eps = eps;
  if (epi == GEMV_STORE) launch_epi<GEMV_STORE>(rows, a, N, s);
  else if (epi == GEMV_RESIDUAL) launch_epi<GEMV_RESIDUAL>(rows, a, N, s);
  else launch_epi<GEMV_SWIGLU>(rows, a, N, s);
}

// q/k/v projection of decode rows with RoPE and the cache write fused: q goes
// to qout [pass rows][nq*d], k and v to their cache slots.
void launch_gemv_qkv_rope(const GemvSeg* seg, int K, const void* x, int ldx, int rows, int row0,
                          void* qout, const RowTable& tab, const void* rope, int nq, int nkv,
                          int d, const void* normw, float eps, hipStream_t s) {
  GemvArgs a;
  for (int i = 0; i < 3; ++i) a.seg[i] = seg[i];
  a.nseg = 3;
  a.K = K;
  a.x = (const bf16_t*)x;
  a.ldx = ldx;
  a.out = (bf16_t*)qout;
  a.ldo = nq * d;
  a.out32 = nullptr;
  a.ld32 = 0;
  a.tab = tab;
  a.rope = (const float2*)rope;
  a.nq = nq;
  a.nkv = nkv;
  a.d = d;
  a.row0 = row0;
  a.normw = rows <= GEMV_NORM_ROWS ? (const bf16_t*)normw : nullptr;
  a.eps = eps;
  const int N = (nq + 2 * nkv) * d;  // four columns per wave, 16 per workgroup
  launch_epi<GEMV_QKV_ROPE>(rows, a, N, s);
}
