// Causal grouped-query attention for prompt chunks on the bf16 matrix cores
// (pull request "llama: Nanbeige4.3-33B on Metal, the bf16 release served as
// published", section "How": prompt chunks over a position-major cache).
//
// One workgroup = four waves of 32 chunk rows: two query heads of a KV head x
// 64 rows, or an odd last head x 128 rows (64-row units track the causal
// diagonal more closely: 4% less time at 2k context, 2% at 129k).  Key
// tiles of 64 cache slots go from the cache straight into LDS (16-byte
// LDS-direct loads, keys and values both [slot][d]), double-buffered: the
// next tile's copies are in flight while the current tile is consumed.  Per
// tile a wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys as
// rows, queries as columns, so each lane holds 32 scores of one query and
// the softmax reductions stay in registers plus one xor-32 exchange), updates
// the running max and sum in fp32 (online softmax, in base 2 with the
// 1/sqrt(d) scale folded into the exponent), and accumulates O^T += V^T P^T.
// The V^T operand is read with ds_read_b64_tr_b16, which transposes four
// slots x four dims per 16 lanes on the way out of LDS.  The probabilities
// enter that product as the sum of two bf16 parts (hi = bf16(p), lo =
// bf16(p - hi): two MFMAs), which keeps about 16 significant bits of each
// weight; the query rows' running state and the output accumulators are
// fp32, and the output is rounded once to bf16.  The P^T operand is the S^T
// accumulator registers themselves: an MFMA sums over its k slots in any
// order, so V^T is read in the key order those registers hold.  The causal
// mask is applied only on tiles that reach past a wave's first query.
//
// Two forms (EXACT).  The fast form keeps two bf16 parts of each weight and
// one running MFMA chain over all tiles.  The exact form keeps three parts
// (hi, mid = bf16(p - hi), lo = bf16(p - hi - mid): 24 significant bits, as
// fp32) and sums each tile's products in fresh registers, entering them into
// the running sums with one fp32 multiply-add per element: the matrix unit's
// accumulation, which loses more than an fp32 addition per product, then never
// runs longer than one tile.  Measured against binary64 on 2,048-row chunks,
// the exact form's outputs equal the correctly rounded ones on 99.96% of
// elements (99.92% at 129k context), the fast form's on 99.86% (99.70%); the
// exact form costs 1.3-1.4x the time.
#include "common.h"
#include "launch.h"

namespace {

constexpr int QT = 128;  // chunk rows per workgroup
constexpr int KT = 64;   // cache slots per LDS tile

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;

__device__ __forceinline__ uint32_t cvt_pk_bf16(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf2;
  bf2 v = {(__bf16)a, (__bf16)b};  // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

// The low bf16 half of w as an fp32 value (w << 16).  Written as one
// instruction: from the plain shift the compiler rebuilds the half by
// converting the weight alone again and shifting, one more instruction per
// pair (2-3% of the fast form's time at 2k context).
__device__ __forceinline__ float lo_half(uint32_t w) {
  uint32_t r;
  asm("v_lshlrev_b32 %0, 16, %1" : "=v"(r) : "v"(w));
  return __uint_as_float(r);
}

// nonzero when either bf16 half of w has an all-ones exponent (Inf or NaN)
__device__ __forceinline__ uint32_t nonfinite2(uint32_t w) {
  return ((w & 0x7F807F80u) + 0x00800080u) & 0x80008000u;
}

template <int D, bool EXACT>
__global__ __launch_bounds__(256, 2) void attn_prefill_kernel(const bf16_t* __restrict__ q,
                                                           const bf16_t* __restrict__ kc,
                                                           const bf16_t* __restrict__ vc,
                                                           int rows, int pos0, int nq, int nkv,
                                                           bf16_t* __restrict__ out,
                                                           float* __restrict__ out32) {
  constexpr int CH = D / 8;             // 16-byte chunks per slot row
  constexpr int RPI = 64 / CH;          // slot rows per LDS-direct copy (1 KiB)
  constexpr int NPW = KT / RPI / 4;     // copies per wave per operand tile
  static_assert(NPW * RPI * 4 == KT, "copies cover the tile");
  // Tiles [slot][d], rows of 2D bytes, no padding.  Keys: chunk c of row r
  // stored at c ^ (r % CH), so the 16 rows of a fragment read hit 16
  // different chunk positions.  Values: 32-byte granule g of row r stored at
  // g ^ (r % (CH / 2)), so the eight rows of a transposed read spread evenly.
  __shared__ __attribute__((aligned(16))) bf16_t sK[2][KT * D];
  __shared__ __attribute__((aligned(16))) bf16_t sV[2][KT * D];
  __shared__ uint32_t sBad[2][4];  // per tile: slots whose value was not finite, 16 per wave

  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index as a scalar: every LDS-direct copy's destination (M0) and
  // the work unit's head and rows are then scalar arithmetic, not a lane
  // read-back per copy (3-8% less time, same bits)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // Work units per KV head g, 128 chunk rows (a span) at a time: the heads of
  // the group in pairs, each pair a workgroup of 64 rows (two waves per head),
  // so every staged key/value tile serves two heads; an odd last head takes
  // 128 rows (four waves).  Spans from the last (longest first); workgroup b
  // runs on XCD b % 8, so with eight KV heads XCD x serves KV head x.
  const int G = nq / nkv;
  const int npair = G / 2, nsingle = G & 1, per_span = nsingle + 2 * npair;
  const int nspan = (rows + QT - 1) / QT;
  const int g = blockIdx.x % nkv, j = blockIdx.x / nkv;
  const int span = nspan - 1 - j / per_span, k = j % per_span;
  int h, r0, nrows_wg, wrow;  // this wave's head, the workgroup's rows, this wave's first row
  if (k < nsingle) {
    h = g * G + G - 1;
    r0 = span * QT;
    nrows_wg = QT;
    wrow = r0 + 32 * wave;
  } else {
    const int kk = k - nsingle, pr = kk % npair, upper = kk / npair == 0;
    h = g * G + 2 * pr + (wave >> 1);
    r0 = span * QT + (upper ? QT / 2 : 0);
    nrows_wg = QT / 2;
    wrow = r0 + 32 * (wave & 1);
  }
  if (r0 >= rows) return;  // uniform per workgroup: the empty half of a ragged last span
  const int lq = lane & 31, half = lane >> 5;
  const int qrow = wrow + lq;                          // this lane's query row in the chunk
  const int qpos = pos0 + min(qrow, rows - 1);         // its absolute position
  const int wave_first = pos0 + min(wrow, rows - 1);
  const int wave_last = pos0 + min(wrow + 31, rows - 1);
  const int block_last = pos0 + min(r0 + nrows_wg - 1, rows - 1);
  const int kvd = nkv * D;
  const float c2 = 1.4426950408889634f / sqrtf((float)D);  // log2(e) / sqrt(d)

  // Q^T fragments: lane holds q[qrow][16t + 8*half .. +8] for t < D/16
  bf16x8_t qf[D / 16];
  {
    const bf16_t* src = q + ((size_t)min(qrow, rows - 1) * nq + h) * D + 8 * half;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) qf[t] = *(const bf16x8_t*)(src + 16 * t);
  }

  // LDS-direct copies of tile k0 into buffer buf: copy n of an operand
  // covers tile rows n*RPI .. n*RPI + RPI - 1; lane l writes 16-byte slot l:
  // row n*RPI + l/CH, stored chunk l%CH, so it fetches the logical chunk the
  // swizzle puts there.  Slots past the block's last query are masked for
  // every row of the block; their copies read that last slot (a valid row).
  const int crow = lane / CH, cch = lane % CH;
  auto issue = [&](int buf, int k0) {
#pragma unroll
    for (int m = 0; m < NPW; ++m) {
      const int n = wave * NPW + m, r = n * RPI + crow;
      const size_t src = (size_t)min(k0 + r, block_last) * kvd + g * D;
      __builtin_amdgcn_global_load_lds((const void*)(kc + src + 8 * (cch ^ (r % CH))),
                                       (lds_ptr_t)(&sK[buf][n * 512]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((const void*)(vc + src + 8 * (cch ^ (2 * (r % (CH / 2))))),
                                       (lds_ptr_t)(&sV[buf][n * 512]), 16, 0, 0);
    }
  };
  // On a tile where some row of the block has masked slots, a masked slot
  // still meets a zero weight in the value product, and 0 * NaN would leak
  // into earlier rows, so there non-finite values are zeroed in LDS and their
  // slot flagged: a score against a flagged slot that is not masked becomes
  // NaN, which is what the rows attending to it get.  On the other tiles
  // every row attends to every slot and a non-finite value reaches every row
  // through the product itself.
  const int block_first = pos0 + r0;
  auto fix_values = [&](int buf) {  // four threads per slot row, CH/4 chunks each
    constexpr int CPT = CH / 4;
    u32x4_t* rowp = (u32x4_t*)&sV[buf][(tid >> 2) * D] + (tid & 3) * CPT;
    uint32_t bad = 0;
#pragma unroll
    for (int c = 0; c < CPT; ++c) {
      u32x4_t v = rowp[c];
      const uint32_t b = nonfinite2(v.x) | nonfinite2(v.y) | nonfinite2(v.z) | nonfinite2(v.w);
      if (b) {
        uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if ((w[e] & 0x7F80u) == 0x7F80u) w[e] &= 0xFFFF0000u;
          if ((w[e] & 0x7F800000u) == 0x7F800000u) w[e] &= 0x0000FFFFu;
        }
        rowp[c] = u32x4_t{w[0], w[1], w[2], w[3]};
      }
      bad |= b;
    }
    bad |= __shfl_xor(bad, 1, WAVE);
    bad |= __shfl_xor(bad, 2, WAVE);
    const uint64_t m = __ballot(bad != 0);  // bit 4k: slot 16*wave + k
    uint32_t slots = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) slots |= (uint32_t)((m >> (4 * k)) & 1u) << k;
    if (lane == 0) sBad[buf][wave] = slots;
  };

  // V^T fragment of output block i, step st of the tile in buffer buf: lane l
  // needs dims 32i + l%32 of keys 16st + 8w + 4*half + e (w, e < 2, 4); a
  // transposed read gives the 16 lanes of group gq = l/16 four slots x one
  // dim each, lane x of the group naming slot 16st + 8w + 4*(gq/2) + x/4,
  // dims 32i + 16*(gq%2) + 4*(x%4)..+3
  auto vfrag = [&](int buf, int i, int st) {
    s16x4_t p2[2];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const int gq = lane >> 4, x = lane & 15;
      const int row = 16 * st + 8 * w + 4 * (gq >> 1) + (x >> 2);
      const int d = 32 * i + 16 * (gq & 1) + 4 * (x & 3);
      const int off = row * D + 8 * ((d >> 3) ^ (2 * (row % (CH / 2)))) + (d & 7);
      p2[w] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4_t*)(&sV[buf][off]));
    }
    return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(p2[0], p2[1], 0, 1, 2, 3, 4, 5, 6, 7));
  };

  f32x16_t acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  float mrow = -INFINITY, lrow = 0.f;

  const int ntiles = block_last / KT + 1;
  issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's copies are in LDS
  __syncthreads();
  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * KT, buf = kt & 1;
    if (kt + 1 < ntiles) issue(buf ^ 1, k0 + KT);
    const bool masked = k0 + KT - 1 > block_first;  // uniform per workgroup
    if (masked) {
      fix_values(buf);
      __syncthreads();
    }
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
          const int r = 32 * u + lq;  // stored chunk of logical chunk 2t + half
          const bf16x8_t kf = *(const bf16x8_t*)&sK[buf][r * D + 8 * ((2 * t + half) ^ (r % CH))];
          s[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t], s[u], 0, 0, 0);
        }
      }
      // keys of register r of half u: k0 + 32u + 8*(r/4) + 4*half + r%4
      // (raw scores here; the scale enters the exponent below)
      const bool diag = k0 + KT - 1 > wave_first;
      if (masked && (sBad[buf][0] | sBad[buf][1] | sBad[buf][2] | sBad[buf][3])) {
        // rare: zeroed non-finite values
        uint32_t gm[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) gm[w] = sBad[buf][w];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ko = 32 * u + 8 * (r >> 2) + 4 * half + (r & 3);
            if (gm[ko >> 4] >> (ko & 15) & 1u) s[u][r] = NAN;
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
      float psum = 0.f;
      if constexpr (EXACT) {
        // p = hi + mid + lo.  The weights of the whole tile are formed first
        // (the scores are then dead), then each pair of 32-dim output blocks
        // takes the tile's twelve products in fresh registers.
        bf16x8_t pf[4], pfm[4], pfl[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          uint32_t pk[4], pm[4], pl[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(s[st >> 1][8 * (st & 1) + 2 * i], c2, moff));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(s[st >> 1][8 * (st & 1) + 2 * i + 1], c2, moff));
            psum += p0;
            psum += p1;
            const uint32_t hw = cvt_pk_bf16(p0, p1);
            const float r0 = p0 - lo_half(hw), r1 = p1 - __uint_as_float(hw & 0xFFFF0000u);
            const uint32_t mw = cvt_pk_bf16(r0, r1);
            pk[i] = hw;
            pm[i] = mw;
            pl[i] = cvt_pk_bf16(r0 - lo_half(mw), r1 - __uint_as_float(mw & 0xFFFF0000u));
          }
          pf[st] = __builtin_bit_cast(bf16x8_t, u32x4_t{pk[0], pk[1], pk[2], pk[3]});
          pfm[st] = __builtin_bit_cast(bf16x8_t, u32x4_t{pm[0], pm[1], pm[2], pm[3]});
          pfl[st] = __builtin_bit_cast(bf16x8_t, u32x4_t{pl[0], pl[1], pl[2], pl[3]});
        }
#pragma unroll
        for (int i = 0; i < D / 32; i += 2) {
          f32x16_t oa, ob;
#pragma unroll
          for (int st = 0; st < 4; ++st) {
            const bf16x8_t va = vfrag(buf, i, st), vb = vfrag(buf, i + 1, st);
            // the two blocks' products alternate: no back-to-back dependent products
            oa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[st], st ? oa : f32x16_t{}, 0, 0, 0);
            ob = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb, pf[st], st ? ob : f32x16_t{}, 0, 0, 0);
            oa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pfm[st], oa, 0, 0, 0);
            ob = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb, pfm[st], ob, 0, 0, 0);
            oa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pfl[st], oa, 0, 0, 0);
            ob = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vb, pfl[st], ob, 0, 0, 0);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            acc[i][r] = fmaf(acc[i][r], alpha, oa[r]);
            acc[i + 1][r] = fmaf(acc[i + 1][r], alpha, ob[r]);
          }
        }
      } else {
      if (!__all(alpha == 1.f)) {
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][r] *= alpha;
      }
      // O^T += V^T P^T in four k-steps of 16 keys; k slot 8*half + i of step
      // st holds key 16*st + 8*(i/4) + 4*half + i%4 (the S^T register order).
      // p = hi + lo with hi = bf16(p), lo = bf16(p - hi).
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
          pl[i] = cvt_pk_bf16(p0 - lo_half(hw), p1 - __uint_as_float(hw & 0xFFFF0000u));
        }
        const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, u32x4_t{pk[0], pk[1], pk[2], pk[3]});
        const bf16x8_t pfl = __builtin_bit_cast(bf16x8_t, u32x4_t{pl[0], pl[1], pl[2], pl[3]});
        bf16x8_t vf[D / 32];
#pragma unroll
        for (int i = 0; i < D / 32; ++i) vf[i] = vfrag(buf, i, st);
        // hi parts over all accumulators, then lo parts: no back-to-back
        // dependent products
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pf, acc[i], 0, 0, 0);
#pragma unroll
        for (int i = 0; i < D / 32; ++i)
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i], pfl, acc[i], 0, 0, 0);
      }
      }
      psum += __shfl_xor(psum, 32, WAVE);
      lrow = lrow * alpha + psum;
    }
    // this wave's copies of the next tile are in LDS; after the barrier all
    // are, and this tile's readers are done
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
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
    if (out32) {  // parity probe: the value before its rounding
      float* d32 = out32 + ((size_t)qrow * nq + h) * D;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) d32[32 * i + 8 * (r >> 2) + 4 * half + (r & 3)] = acc[i][r] * inv;
    }
  }
}

}  // namespace

// q: [rows][nq][d] after RoPE; kc/vc: the sequence's slabs for this execution,
// already holding positions [0, pos0 + rows); out: [rows][nq][d]; out32
// (nullable): the same before rounding.
template <int D, bool EXACT>
static void launch_dx(const void* q, const void* kc, const void* vc, int rows, int pos0, int nq,
                      int nkv, void* out, float* out32, hipStream_t s) {
  const int G = nq / nkv;
  dim3 grid((rows + QT - 1) / QT * nkv * (G % 2 + 2 * (G / 2)));
  launch_k((attn_prefill_kernel<D, EXACT>), grid, dim3(256), 0, s, (const bf16_t*)q,
                     (const bf16_t*)kc, (const bf16_t*)vc, rows, pos0, nq, nkv, (bf16_t*)out,
                     out32);
}

void launch_attn_prefill(const void* q, const void* kc, const void* vc, int rows, int pos0, int nq,
                         int nkv, int d, void* out, float* out32, bool exact, hipStream_t s) {
  if (d == 64) {
    if (exact) launch_dx<64, true>(q, kc, vc, rows, pos0, nq, nkv, out, out32, s);
    else launch_dx<64, false>(q, kc, vc, rows, pos0, nq, nkv, out, out32, s);
  } else {
    if (exact) launch_dx<128, true>(q, kc, vc, rows, pos0, nq, nkv, out, out32, s);
    else launch_dx<128, false>(q, kc, vc, rows, pos0, nq, nkv, out, out32, s);
  }
}
