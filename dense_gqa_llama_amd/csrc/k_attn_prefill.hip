// Causal grouped-query attention for prompt chunks on the bf16 matrix cores
// (pull request "llama: Nanbeige4.3-33B on Metal, the bf16 release served as
// published", section "How": prompt chunks over a position-major cache).
//
// One workgroup = one query head and 128 chunk rows (4 waves x 32 rows).  Key
// tiles of 64 cache slots are staged in LDS (keys [slot][d], values
// transposed [d][slot]) and shared by the four waves.  Per 32-key sub-tile a
// wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (keys as rows,
// queries as columns, so each lane holds 16 scores of one query and the
// softmax reductions stay in registers plus one xor-32 exchange), updates the
// running max and sum in fp32 (online softmax), and accumulates
// O^T += V^T P^T.  The probabilities enter that product as the sum of two
// bf16 parts (hi = bf16(p), lo = bf16(p - hi): two MFMAs), which keeps about
// 16 significant bits of each weight; the query rows' running state and the
// output accumulators are fp32, and the output is rounded once to bf16.
// The P^T operand is the S^T accumulator registers themselves: an MFMA sums
// over its k slots in any order, so V^T is read in the key order those
// registers hold.
#include "common.h"
#include "launch.h"

namespace {

constexpr int QT = 128;  // chunk rows per workgroup
constexpr int KT = 64;   // cache slots per LDS tile
constexpr int VPAD = 4;

template <int D>
__global__ __launch_bounds__(256) void attn_prefill_kernel(const bf16_t* __restrict__ q,
                                                           const bf16_t* __restrict__ kc,
                                                           const bf16_t* __restrict__ vc,
                                                           int rows, int pos0, int nq, int nkv,
                                                           bf16_t* __restrict__ out) {
  constexpr int KLD = D + 8;
  constexpr int VLD = KT + VPAD;
  __shared__ __attribute__((aligned(16))) bf16_t sK[KT * KLD];
  __shared__ __attribute__((aligned(16))) bf16_t sV[D * VLD];
  __shared__ int sBad[KT];  // slot holds a non-finite value

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = blockIdx.y, g = h / (nq / nkv);
  const int r0 = blockIdx.x * QT;
  const int lq = lane & 31, half = lane >> 5;
  const int qrow = r0 + wave * 32 + lq;               // this lane's query row in the chunk
  const int qpos = pos0 + min(qrow, rows - 1);         // its absolute position
  const int wave_last = pos0 + min(r0 + wave * 32 + 31, rows - 1);
  const int block_last = pos0 + min(r0 + QT - 1, rows - 1);
  const int kvd = nkv * D;
  const float scale = 1.0f / sqrtf((float)D);

  // Q^T fragments: lane holds q[qrow][16t + 8*half .. +8] for t < D/16
  bf16x8_t qf[D / 16];
  {
    const bf16_t* src = q + ((size_t)min(qrow, rows - 1) * nq + h) * D + 8 * half;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) qf[t] = *(const bf16x8_t*)(src + 16 * t);
  }

  f32x16_t acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  float mrow = -INFINITY, lrow = 0.f;

  const int ntiles = block_last / KT + 1;
  for (int kt = 0; kt < ntiles; ++kt) {
    const int k0 = kt * KT;
    __syncthreads();  // previous tile's readers are done
    if (tid < KT) sBad[tid] = 0;
    __syncthreads();
    // Stage keys [slot][d] and values transposed [d][slot].  Slots past the
    // block's last query are zero (their scores are masked).  A masked slot
    // still meets a zero weight in the value product, and 0 * NaN would leak
    // into earlier rows, so non-finite values are staged as zero and their
    // slot flagged: a score against a flagged slot that is not masked becomes
    // NaN, which is what the rows attending to it would get.
    for (int c = tid; c < KT * D / 8; c += 256) {
      int slot = c / (D / 8), dc = (c % (D / 8)) * 8;
      int p = k0 + slot;
      u32x4_t kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
      if (p <= block_last) {
        kv = *(const u32x4_t*)(kc + (size_t)p * kvd + g * D + dc);
        vv = *(const u32x4_t*)(vc + (size_t)p * kvd + g * D + dc);
      }
      *(u32x4_t*)&sK[slot * KLD + dc] = kv;
      uint32_t w[4] = {vv.x, vv.y, vv.z, vv.w};
      int bad = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        bf16_t lo = (bf16_t)(w[e] & 0xFFFF), hi = (bf16_t)(w[e] >> 16);
        if ((lo & 0x7F80) == 0x7F80) { bad = 1; lo = 0; }
        if ((hi & 0x7F80) == 0x7F80) { bad = 1; hi = 0; }
        sV[(dc + 2 * e) * VLD + slot] = lo;
        sV[(dc + 2 * e + 1) * VLD + slot] = hi;
      }
      if (bad) sBad[slot] = 1;
    }
    __syncthreads();
    if (k0 > wave_last) continue;  // every key of this tile is after this wave's queries

#pragma unroll
    for (int sub = 0; sub < KT; sub += 32) {
      const int ks = k0 + sub;
      if (ks > wave_last) break;
      // S^T = K Q^T for 32 keys x 32 queries
      f32x16_t s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        bf16x8_t kf = *(const bf16x8_t*)&sK[(sub + lq) * KLD + 16 * t + 8 * half];
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[t], s, 0, 0, 0);
      }
      // scale, causal mask, tile max (keys of reg r: ks + 8*(r/4) + 4*half + r%4)
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int kp = ks + 8 * (r >> 2) + 4 * half + (r & 3);
        float v = kp <= qpos ? (sBad[kp - k0] ? NAN : s[r] * scale) : -INFINITY;
        s[r] = v;
        mx = fmaxf(mx, v);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, WAVE));
      const float mnew = fmaxf(mrow, mx);
      // a row with no unmasked key yet keeps zero weights
      const float alpha = mnew == -INFINITY ? 1.f : expf(mrow - mnew);
      // p = hi + lo with hi = bf16(p), lo = bf16(p - hi): about 16 significant
      // bits of each weight reach the matrix product
      float psum = 0.f;
      uint32_t pk[8], pl[8];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float p0 = mnew == -INFINITY ? 0.f : expf(s[r] - mnew);
        float p1 = mnew == -INFINITY ? 0.f : expf(s[r + 1] - mnew);
        bf16_t h0 = f2bf(p0), h1 = f2bf(p1);
        psum += p0 + p1;
        pk[r / 2] = pack_bf2(h0, h1);
        pl[r / 2] = pack_bf2(f2bf(p0 - bf2f(h0)), f2bf(p1 - bf2f(h1)));
      }
      psum += __shfl_xor(psum, 32, WAVE);
      lrow = lrow * alpha + psum;
      mrow = mnew;
#pragma unroll
      for (int i = 0; i < D / 32; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][r] *= alpha;
      // O^T += V^T P^T, two k-steps of 16 keys; k slot 8*half + i holds key
      // 16*st + 8*(i/4) + 4*half + i%4 (the S^T register order)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        u32x4_t pw = {pk[4 * st], pk[4 * st + 1], pk[4 * st + 2], pk[4 * st + 3]};
        u32x4_t plw = {pl[4 * st], pl[4 * st + 1], pl[4 * st + 2], pl[4 * st + 3]};
        bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pw);
        bf16x8_t pfl = __builtin_bit_cast(bf16x8_t, plw);
#pragma unroll
        for (int i = 0; i < D / 32; ++i) {
          const bf16_t* vrow = &sV[(i * 32 + lq) * VLD + sub + 16 * st + 4 * half];
          uint2 lo = *(const uint2*)vrow, hi = *(const uint2*)(vrow + 8);
          u32x4_t vw = {lo.x, lo.y, hi.x, hi.y};
          bf16x8_t vf = __builtin_bit_cast(bf16x8_t, vw);
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, acc[i], 0, 0, 0);
          acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pfl, acc[i], 0, 0, 0);
        }
      }
    }
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
