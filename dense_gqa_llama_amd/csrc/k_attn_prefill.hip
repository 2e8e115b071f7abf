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
constexpr int VPAD = 4;

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
  static_assert(VS == 2 || VS == 4, "value staging takes 2 or 4 slots per thread");
  __shared__ __attribute__((aligned(16))) bf16_t sK[2][KT * KLD];
  __shared__ __attribute__((aligned(16))) bf16_t sV[2][D * VLD];
  __shared__ int sBad[2][KT];   // slot holds a non-finite value
  __shared__ int sBadW[2][4];   // some slot of the tile does (per staging wave)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // heaviest row blocks first: block x covers rows of block (nblk - 1 - x)
  const int rb = gridDim.x - 1 - blockIdx.x;
  const int h = blockIdx.y, g = h / (nq / nkv);
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

  // staging: keys as KCH chunks (slot c/DCH, dims (c%DCH)*8), values as VS
  // consecutive slots VS*(tid/DCH) .. at dims (tid%DCH)*8
  const int vslot = VS * (tid / DCH), vdc = (tid % DCH) * 8;
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
  // Values are staged transposed.  A masked slot still meets a zero weight in
  // the value product, and 0 * NaN would leak into earlier rows, so
  // non-finite values are staged as zero and their slot flagged: a score
  // against a flagged slot that is not masked becomes NaN, which is what the
  // rows attending to it would get.
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + i * 256;
      *(u32x4_t*)&sK[buf][(c / DCH) * KLD + (c % DCH) * 8] = rk[i];
    }
    uint32_t badj[VS];
    uint32_t any = 0;
#pragma unroll
    for (int j = 0; j < VS; ++j) {
      badj[j] = nonfinite2(rv[j].x) | nonfinite2(rv[j].y) | nonfinite2(rv[j].z) | nonfinite2(rv[j].w);
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
        *(uint2*)&sV[buf][(vdc + 2 * e) * VLD + vslot] = make_uint2(lo01, lo23);
        *(uint2*)&sV[buf][(vdc + 2 * e + 1) * VLD + vslot] = make_uint2(hi01, hi23);
      } else {
        *(uint32_t*)&sV[buf][(vdc + 2 * e) * VLD + vslot] = lo01;
        *(uint32_t*)&sV[buf][(vdc + 2 * e + 1) * VLD + vslot] = hi01;
      }
    }
    // a slot's flag is the OR over the DCH threads holding its dims
#pragma unroll
    for (int j = 0; j < VS; ++j) {
      uint32_t f = badj[j];
#pragma unroll
      for (int m = 1; m < DCH; m <<= 1) f |= __shfl_xor(f, m, WAVE);
      if (vdc == 0) sBad[buf][vslot + j] = f != 0;
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
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * KT, buf = kt & 1;
    if (kt + 1 < ntiles) gload(k0 + KT);
    if (k0 <= wave_last) {
      // S^T = K Q^T for 64 keys (two 32-key halves) x 32 queries
      f32x16_t s[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[u][r] = 0.f;
#pragma unroll
        for (int t = 0; t < D / 16; ++t) {
          bf16x8_t kf = *(const bf16x8_t*)&sK[buf][(32 * u + lq) * KLD + 16 * t + 8 * half];
          s[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t], s[u], 0, 0, 0);
        }
      }
      // keys of register r of half u: k0 + 32u + 8*(r/4) + 4*half + r%4
      const bool any_bad = sBadW[buf][0] | sBadW[buf][1] | sBadW[buf][2] | sBadW[buf][3];
      const bool diag = k0 + KT - 1 > wave_first;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[u][r] *= c2;
      if (any_bad | diag) {  // tiles on the diagonal, or holding a non-finite value
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int ko = 32 * u + 8 * (r >> 2) + 4 * half + (r & 3);
            float v = sBad[buf][ko] ? NAN : s[u][r];
            s[u][r] = k0 + ko > qpos ? -INFINITY : v;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[u][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
      const float mnew = fmaxf(mrow, mx);
      // a row with no unmasked key yet keeps zero weights
      const float mref = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = __builtin_amdgcn_exp2f(mrow - mref);
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
          const float p0 = __builtin_amdgcn_exp2f(s[st >> 1][8 * (st & 1) + 2 * i] - mref);
          const float p1 = __builtin_amdgcn_exp2f(s[st >> 1][8 * (st & 1) + 2 * i + 1] - mref);
          psum += p0;
          psum += p1;
          const uint32_t hw = cvt_pk_bf16(p0, p1);
          pk[i] = hw;
          pl[i] = cvt_pk_bf16(p0 - __uint_as_float(hw << 16), p1 - __uint_as_float(hw & 0xFFFF0000u));
        }
        const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, u32x4_t{pk[0], pk[1], pk[2], pk[3]});
        const bf16x8_t pfl = __builtin_bit_cast(bf16x8_t, u32x4_t{pl[0], pl[1], pl[2], pl[3]});
#pragma unroll
        for (int i = 0; i < D / 32; ++i) {
          const bf16_t* vrow = &sV[buf][(i * 32 + lq) * VLD + 16 * st + 4 * half];
          const uint2 lo = *(const uint2*)vrow, hi = *(const uint2*)(vrow + 8);
          const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, u32x4_t{lo.x, lo.y, hi.x, hi.y});
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, acc[i], 0, 0, 0);
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pfl, acc[i], 0, 0, 0);
        }
      }
      psum += __shfl_xor(psum, 32, WAVE);
      lrow = lrow * alpha + psum;
    }
    if (kt + 1 < ntiles) lstore(buf ^ 1);
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
  dim3 grid((rows + QT - 1) / QT, nq);
  if (d == 64)
    hipLaunchKernelGGL(attn_prefill_kernel<64>, grid, dim3(256), 0, s, (const bf16_t*)q,
                       (const bf16_t*)kc, (const bf16_t*)vc, rows, pos0, nq, nkv, (bf16_t*)out);
  else
    hipLaunchKernelGGL(attn_prefill_kernel<128>, grid, dim3(256), 0, s, (const bf16_t*)q,
                       (const bf16_t*)kc, (const bf16_t*)vc, rows, pos0, nq, nkv, (bf16_t*)out);
}
