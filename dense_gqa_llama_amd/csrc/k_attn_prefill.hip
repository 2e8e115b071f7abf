// Causal grouped-query attention for prompt chunks on the bf16 matrix cores
// (pull request "llama: Nanbeige4.3-33B on Metal, the bf16 release served as
// published", section "How": prompt chunks over a position-major cache).
//
// One workgroup = one query head and 128 chunk rows (4 waves x 32 rows).  Key
// tiles of 64 cache slots are staged in LDS (keys [slot][d], values
// transposed [d][slot]), double-buffered: the next tile's global loads are in
// flight while the current tile is consumed.  Per tile a wave computes
// S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys as rows, queries as
// columns, so each lane holds 32 scores of one query and the softmax
// reductions stay in registers plus one xor-32 exchange), updates the running
// max and sum in fp32 (online softmax, in base 2 with the 1/sqrt(d) scale
// folded into the exponent), and accumulates O^T += V^T P^T.  The
// probabilities enter that product as the sum of two bf16 parts (hi =
// bf16(p), lo = bf16(p - hi): two MFMAs), which keeps about 16 significant
// bits of each weight; the query rows' running state and the output
// accumulators are fp32, and the output is rounded once to bf16.  The P^T
// operand is the S^T accumulator registers themselves: an MFMA sums over its
// k slots in any order, so V^T is read in the key order those registers hold.
// The causal mask is applied only on tiles that reach past a wave's first
// query.
#include "common.h"
#include "launch.h"

namespace {

constexpr int QT = 128;  // chunk rows per workgroup
constexpr int KT = 64;   // cache slots per LDS tile
constexpr int VPAD = 8;  // V^T rows of 144 B: 16-byte fragment reads are conflict-free

// Column of tile slot s in the transposed value tile.  Within each 16-slot
// step the slots are stored in the order the PV product's k slots take them
// (lane half h reads k slots 8h .. 8h + 7 = keys 4h .. 4h + 3, 8 + 4h .. 11 +
// 4h): slots 0-3, 8-11, 4-7, 12-15, so a fragment is one 16-byte read.
__device__ __forceinline__ int vcol(int s) {
  return (s & ~15) | ((s >> 2) & 1) << 3 | ((s >> 3) & 1) << 2 | (s & 3);
}

__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf2;
  bf2 v = {(__bf16)a, (__bf16)b};  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// nonzero when either bf16 half of w has an all-ones exponent (Inf or NaN)
__device__ __forceinline__ uint32_t nonfinite2(uint32_t w) {
  return ((w & 0x7F807F80u) + 0x00800080u) & 0x80008000u;
}

template <int D>
__global__ __launch_bounds__(256, 2) void attn_prefill_kernel(const bf16_t* __restrict__ q,
                                                           const bf16_t* __restrict__ kc,
                                                           const bf16_t* __restrict__ vc,
                                                           int rows, int pos0, int nq, int nkv,
                                                           bf16_t* __restrict__ out) {
  constexpr int KLD = D + 8;
  constexpr int VLD = KT + VPAD;
  constexpr int KCH = KT * D / 8 / 256;   // 16-byte key chunks per thread per tile
  constexpr int DCH = D / 8;              // 16-byte chunks per slot
  constexpr int VS = KT * DCH / 256;      // value slots per thread per tile
  constexpr int NGRP = KT / VS;           // value slot groups per tile
  static_assert(VS == 2 || VS == 4, "value staging takes 2 or 4 slots per thread");
  static_assert(NGRP * DCH == 256 && NGRP <= 32, "value staging covers the tile");
  __shared__ __attribute__((aligned(16))) bf16_t sK[2][KT * KLD];
  __shared__ __attribute__((aligned(16))) bf16_t sV[2][D * VLD];
  __shared__ uint32_t sBadM[2][4][VS];  // per staging wave and slot j of a group: group bits
  __shared__ int sBadW[2][4];           // some slot of the tile is flagged (per staging wave)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Heaviest row blocks first over the whole grid (longest-first keeps the
  // last round short).  Workgroup b runs on XCD b % 8: with eight KV heads,
  // XCD x takes the query heads of KV head x, so each XCD's L2 holds one
  // head's keys and values.
  const int nblk = (rows + QT - 1) / QT, G = nq / nkv;
  int rb, h;
  if (nkv == 8) {
    const int j = blockIdx.x / 8;
    rb = nblk - 1 - j / G;
    h = (blockIdx.x % 8) * G + j % G;
  } else {
    rb = nblk - 1 - blockIdx.x / nq;
    h = blockIdx.x % nq;
  }
  const int g = h / G;
  const int r0 = rb * QT;
  const int lq = lane & 31, half = lane >> 5;
  const int qrow = r0 + wave * 32 + lq;               // this lane's query row in the chunk
  const int qpos = pos0 + min(qrow, rows - 1);         // its absolute position
  const int wave_first = pos0 + min(r0 + wave * 32, rows - 1);
  const int wave_last = pos0 + min(r0 + wave * 32 + 31, rows - 1);
  const int block_last = pos0 + min(r0 + QT - 1, rows - 1);
  const int kvd = nkv * D;
  const float c2 = 1.4426950408889634f / sqrtf((float)D);  // log2(e) / sqrt(d)

  // Q^T fragments: lane holds q[qrow][16t + 8*half .. +8] for t < D/16
  bf16x8_t qf[D / 16];
  {
    const bf16_t* src = q + ((size_t)min(qrow, rows - 1) * nq + h) * D + 8 * half;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) qf[t] = *(const bf16x8_t*)(src + 16 * t);
  }

  // staging: keys as KCH chunks (slot c/DCH, dims (c%DCH)*8); values as a
  // group of VS consecutive slots VS*(tid%NGRP) .. at dims 8*(tid/NGRP), so
  // the 16 lanes of an LDS write fill one transposed row
  const int vslot = VS * (tid % NGRP), vdc = 8 * (tid / NGRP);
  u32x4_t rk[KCH], rv[VS];
  // Slots past the block's last query are masked for every row of the block;
  // their loads are clamped to that last slot (a valid cache row).
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + i * 256, p = min(k0 + c / DCH, block_last);
      rk[i] = *(const u32x4_t*)(kc + (size_t)p * kvd + g * D + (c % DCH) * 8);
    }
#pragma unroll
    for (int j = 0; j < VS; ++j) {
      const int p = min(k0 + vslot + j, block_last);
      rv[j] = *(const u32x4_t*)(vc + (size_t)p * kvd + g * D + vdc);
    }
  };
  // Values are staged transposed.  On a tile where some row of the block has
  // masked slots, a masked slot still meets a zero weight in the value
  // product, and 0 * NaN would leak into earlier rows, so non-finite values
  // are staged as zero there and their slot flagged: a score against a
  // flagged slot that is not masked becomes NaN, which is what the rows
  // attending to it get.  On the other tiles every row attends to every slot
  // and a non-finite value reaches every row through the product itself.
  const int block_first = pos0 + r0;
  auto lstore = [&](int buf, int k0) {
    const bool masked = k0 + KT - 1 > block_first;  // uniform per workgroup
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + i * 256;
      *(u32x4_t*)&sK[buf][(c / DCH) * KLD + (c % DCH) * 8] = rk[i];
    }
    uint32_t badj[VS];
    uint32_t any = 0;
#pragma unroll
    for (int j = 0; j < VS; ++j) {
      badj[j] = masked ? nonfinite2(rv[j].x) | nonfinite2(rv[j].y) | nonfinite2(rv[j].z) |
                             nonfinite2(rv[j].w)
                       : 0u;
      any |= badj[j];
    }
    if (any) {  // rare: zero the non-finite halves
#pragma unroll
      for (int j = 0; j < VS; ++j) {
        uint32_t w[4] = {rv[j].x, rv[j].y, rv[j].z, rv[j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if ((w[e] & 0x7F80u) == 0x7F80u) w[e] &= 0xFFFF0000u;
          if ((w[e] & 0x7F800000u) == 0x7F800000u) w[e] &= 0x0000FFFFu;
        }
        rv[j] = u32x4_t{w[0], w[1], w[2], w[3]};
      }
    }
    // transpose VS slots x eight dims into eight rows of sV
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // dims vdc + 2e (low halves) and vdc + 2e + 1 (high halves)
      const uint32_t w0 = rv[0][e], w1 = rv[1][e];
      const uint32_t lo01 = (w0 & 0xFFFFu) | (w1 << 16), hi01 = (w0 >> 16) | (w1 & 0xFFFF0000u);
      if (VS == 4) {
        const uint32_t w2 = rv[VS > 2 ? 2 : 0][e], w3 = rv[VS > 2 ? 3 : 0][e];
        const uint32_t lo23 = (w2 & 0xFFFFu) | (w3 << 16), hi23 = (w2 >> 16) | (w3 & 0xFFFF0000u);
        *(uint2*)&sV[buf][(vdc + 2 * e) * VLD + vcol(vslot)] = make_uint2(lo01, lo23);
        *(uint2*)&sV[buf][(vdc + 2 * e + 1) * VLD + vcol(vslot)] = make_uint2(hi01, hi23);
      } else {
        *(uint32_t*)&sV[buf][(vdc + 2 * e) * VLD + vcol(vslot)] = lo01;
        *(uint32_t*)&sV[buf][(vdc + 2 * e + 1) * VLD + vcol(vslot)] = hi01;
      }
    }
    if (!masked) {  // nothing zeroed, nothing flagged
      if (lane == 0) sBadW[buf][wave] = 0;
      return;
    }
    // per wave and slot j of a group: the groups holding a flagged value
    // in this wave's dims (lanes l, l + NGRP, ... share a group)
#pragma unroll
    for (int j = 0; j < VS; ++j) {
      uint32_t f = badj[j];
#pragma unroll
      for (int m = NGRP; m < WAVE; m <<= 1) f |= __shfl_xor(f, m, WAVE);
      const uint64_t b = __ballot(f != 0);
      if (lane == 0) sBadM[buf][wave][j] = (uint32_t)b & (uint32_t)((1ull << NGRP) - 1);
    }
    const int wany = __any(any != 0);
    if (lane == 0) sBadW[buf][wave] = wany;
  };

  f32x16_t acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  float mrow = -INFINITY, lrow = 0.f;

  const int ntiles = block_last / KT + 1;
  gload(0);
  lstore(0, 0);
  __syncthreads();
  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * KT, buf = kt & 1;
    if (kt + 1 < ntiles) gload(k0 + KT);
    if (k0 <= wave_last) {
      // S^T = K Q^T for 64 keys (two 32-key halves) x 32 queries
      f32x16_t s[2];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[u][r] = 0.f;
      // the two halves' products interleave (independent accumulators)
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const bf16x8_t kf = *(const bf16x8_t*)&sK[buf][(32 * u + lq) * KLD + 16 * t + 8 * half];
          s[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t], s[u], 0, 0, 0);
        }
      }
      // keys of register r of half u: k0 + 32u + 8*(r/4) + 4*half + r%4
      // (raw scores here; the scale enters the exponent below)
      const bool diag = k0 + KT - 1 > wave_first;
      const bool any_bad = sBadW[buf][0] | sBadW[buf][1] | sBadW[buf][2] | sBadW[buf][3];
      if (any_bad) {  // rare: zeroed non-finite values (flag reads kept off the common path)
        const volatile uint32_t* bm = &sBadM[buf][0][0];
        uint32_t gm[VS];
#pragma unroll
        for (int j = 0; j < VS; ++j) gm[j] = bm[j] | bm[VS + j] | bm[2 * VS + j] | bm[3 * VS + j];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ko = 32 * u + 8 * (r >> 2) + 4 * half + (r & 3);
            if (gm[ko % VS] >> (ko / VS) & 1u) s[u][r] = NAN;
          }
      }
      if (diag) {  // tiles reaching past the wave's first query
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (k0 + 32 * u + 8 * (r >> 2) + 4 * half + (r & 3) > qpos) s[u][r] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[u][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
      const float mnew = fmaxf(mrow, mx);
      // weights exp2(c2 * (s - m)) with c2 = log2(e)/sqrt(d), as one
      // multiply-add per score; a row with no unmasked key yet keeps zero
      // weights.  The rescale factor is exactly 1 while the maximum holds (a
      // tile all of whose keys are masked for a row leaves its sums alone, so
      // a row's bits never depend on which other rows share its chunk).
      const float mref = mnew == -INFINITY ? 0.f : mnew;
      const float moff = -mref * c2;
      const float alpha = __builtin_amdgcn_exp2f((mrow - mref) * c2);
      mrow = mnew;
      if (!__all(alpha == 1.f)) {
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][r] *= alpha;
      }
      // O^T += V^T P^T in four k-steps of 16 keys; k slot 8*half + i of step
      // st holds key 16*st + 8*(i/4) + 4*half + i%4 (the S^T register order).
      // p = hi + lo with hi = bf16(p), lo = bf16(p - hi).
      float psum = 0.f;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        uint32_t pk[4], pl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[st >> 1][8 * (st & 1) + 2 * i], c2, moff));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[st >> 1][8 * (st & 1) + 2 * i + 1], c2, moff));
          psum += p0;
          psum += p1;
          const uint32_t hw = cvt_pk_bf16(p0, p1);
          pk[i] = hw;
          pl[i] = cvt_pk_bf16(p0 - __uint_as_float(hw << 16), p1 - __uint_as_float(hw & 0xFFFF0000u));
        }
        const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, u32x4_t{pk[0], pk[1], pk[2], pk[3]});
        const bf16x8_t pfl = __builtin_bit_cast(bf16x8_t, u32x4_t{pl[0], pl[1], pl[2], pl[3]});
        bf16x8_t vf[D / 32];
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
          vf[i] = *(const bf16x8_t*)&sV[buf][(i * 32 + lq) * VLD + 16 * st + 8 * half];
        // hi parts over all accumulators, then lo parts: no back-to-back
        // dependent products
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pf, acc[i], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pfl, acc[i], 0, 0, 0);
      }
      psum += __shfl_xor(psum, 32, WAVE);
      lrow = lrow * alpha + psum;
    }
    if (kt + 1 < ntiles) lstore(buf ^ 1, k0 + KT);
    __syncthreads();
  }

  // O = O^T / l: lane holds column qrow, rows d = 32i + 8(r/4) + 4*half + r%4
  if (qrow < rows) {
    const float inv = 1.0f / lrow;
    bf16_t* dst = out + ((size_t)qrow * nq + h) * D;
#pragma unroll
    for (int i = 0; i < D / 32; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) dst[32 * i + 8 * (r >> 2) + 4 * half + (r & 3)] = f2bf(acc[i][r] * inv);
  }
}

}  // namespace

// q: [rows][nq][d] after RoPE; kc/vc: the sequence's slabs for this execution,
// already holding positions [0, pos0 + rows); out: [rows][nq][d].
void launch_attn_prefill(const void* q, const void* kc, const void* vc, int rows, int pos0, int nq,
                         int nkv, int d, void* out, hipStream_t s) {
  dim3 grid((rows + QT - 1) / QT * nq);
  if (d == 64)
    hipLaunchKernelGGL(attn_prefill_kernel<64>, grid, dim3(256), 0, s, (const bf16_t*)q,
                       (const bf16_t*)kc, (const bf16_t*)vc, rows, pos0, nq, nkv, (bf16_t*)out);
  else
    hipLaunchKernelGGL(attn_prefill_kernel<128>, grid, dim3(256), 0, s, (const bf16_t*)q,
                       (const bf16_t*)kc, (const bf16_t*)vc, rows, pos0, nq, nkv, (bf16_t*)out);
}
