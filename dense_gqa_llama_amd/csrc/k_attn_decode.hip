// Grouped-query attention for decode rows (pull request "llama:
// Nanbeige4.3-33B on Metal, the bf16 release served as published", section
// "How": decode rows over key blocks at absolute positions).
//
// A row at absolute position p attends to cache slots [0, p].  The slots are
// cut into blocks anchored at absolute positions, of KB(p) slots: 64 while
// p + 1 <= 64 * 64, doubling so that a row never has more than 64 blocks.  The
// partition, and so every sum, depends only on p: a row computed inside a
// window or beside other sequences equals the row computed alone.
//
// One workgroup per (block, KV head, row).  It walks its block in sub-blocks
// of 64 slots: four lanes per slot read the slot's key row (256 contiguous
// bytes for d = 128) and score it against the G query heads sharing the KV
// head (fp32, v_dot2c_f32_bf16), an online softmax keeps the running max and
// sum per head, and lanes per value dimension accumulate exp(s - m) v.  The
// block's (max, sum, unnormalised output) is written as a partial.  A second
// kernel, one workgroup per (query head, row), merges a row's blocks in block
// order, o = sum_b e^(m_b - M) o_b / sum_b e^(m_b - M) l_b, rounded once to
// bf16.  (The kernel boundary makes the partials visible across the chip's
// separate L2s; merging inside the first kernel would need a device-scope
// release in every workgroup.)
#include "common.h"
#include "launch.h"

namespace {

constexpr int SUB = 64;    // slots per sub-block
constexpr int MAXB = 64;   // blocks per row at most

__device__ __forceinline__ int block_slots(int p) {
  int kb = SUB;
  while (p + 1 > kb * MAXB) kb <<= 1;
  return kb;
}

template <int D, int G>
__global__ __launch_bounds__(256) void attn_decode_kernel(const bf16_t* __restrict__ q,
                                                          RowTable tab, int nq, int nkv,
                                                          float* __restrict__ part) {
  constexpr int DP = D / 2;        // value pairs per head
  constexpr int NG = 256 / DP;     // slot groups in the value pass
  constexpr int DQ = D / 4;        // key dims per lane in the score pass
  __shared__ __attribute__((aligned(16))) uint32_t qs[G][DP];
  __shared__ float S[G][SUB];
  __shared__ float Ms[G], Ls[G], As[G];
  __shared__ float O[NG][G][D];

  const int b = blockIdx.x, g = blockIdx.y, rt = blockIdx.z;
  const int seq = rt / tab.rows_per_seq;
  const int p = tab.pos0[seq] + rt % tab.rows_per_seq;
  const int kb = block_slots(p);
  const int nb = p / kb + 1;
  if (b >= nb) return;  // uniform per workgroup
  const int start = b * kb, end = min(start + kb, p + 1);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kvd = nkv * D;

  const int dp = tid % DP, grp = tid / DP;
  const float scale = 1.0f / sqrtf((float)D);
  const bf16_t* kbase = tab.k[seq] + (size_t)g * D;
  const uint32_t* vbase = (const uint32_t*)(tab.v[seq] + (size_t)g * D) + dp;
  const int kslot = tid >> 2, qq = tid & 3;  // score pass: lanes 4k..4k+3 share slot k
  constexpr int KPL = SUB / NG;              // value pass: slots per lane

  // The key and value loads of a sub-block are issued together, one
  // sub-block ahead of their use, so a block costs one memory round trip
  // rather than three (query, keys, then values).
  u32x4_t kreg[DQ / 8];
  uint32_t vv[KPL];
  auto issue = [&](int s0) {
    const int nk = min(SUB, end - s0);
    if (kslot < nk) {
      const u32x4_t* krow = (const u32x4_t*)(kbase + (size_t)(s0 + kslot) * kvd + qq * DQ);
#pragma unroll
      for (int j = 0; j < DQ / 8; ++j) kreg[j] = krow[j];
    }
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const int k = grp + i * NG;
      vv[i] = k < nk ? vbase[(size_t)(s0 + k) * (kvd / 2)] : 0u;
    }
  };
  issue(start);

  const uint32_t* qsrc = (const uint32_t*)(q + ((size_t)rt * nq + (size_t)g * G) * D);
  for (int i = tid; i < G * DP; i += 256) qs[i / DP][i % DP] = qsrc[i];
  if (tid < G) { Ms[tid] = -INFINITY; Ls[tid] = 0.f; }

  float o0[G], o1[G];
#pragma unroll
  for (int h = 0; h < G; ++h) { o0[h] = 0.f; o1[h] = 0.f; }
  __syncthreads();

  for (int s0 = start; s0 < end; s0 += SUB) {
    const int nk = min(SUB, end - s0);
    // scores: lanes 4k..4k+3 share slot k, each over D/4 dims
    {
      float s[G];
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] = 0.f;
      if (kslot < nk) {
#pragma unroll
        for (int j = 0; j < DQ / 8; ++j) {
          const u32x4_t kv = kreg[j];
#pragma unroll
          for (int h = 0; h < G; ++h) {
            const u32x4_t qv = *(const u32x4_t*)&qs[h][qq * (DQ / 2) + 4 * j];
            float t = s[h];
            t = dot2(qv.x, kv.x, t);
            t = dot2(qv.y, kv.y, t);
            t = dot2(qv.z, kv.z, t);
            t = dot2(qv.w, kv.w, t);
            s[h] = t;
          }
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float t = s[h];
        t += __shfl_xor(t, 1, WAVE);
        t += __shfl_xor(t, 2, WAVE);
        if (qq == 0) S[h][kslot] = kslot < nk ? t * scale : -INFINITY;
      }
    }
    __syncthreads();
    // online softmax per head: one wave per head, lane = slot
    for (int h = wave; h < G; h += 4) {
      float v = S[h][lane];
      float mt = wave_max(v);
      float mold = Ms[h];
      float mnew = fmaxf(mold, mt);
      float e = lane < nk ? expf(v - mnew) : 0.f;
      S[h][lane] = e;
      float lt = wave_sum(e);
      if (lane == 0) {
        float a = expf(mold - mnew);  // 0 on the first sub-block (mold = -inf)
        As[h] = a;
        Ls[h] = Ls[h] * a + lt;
        Ms[h] = mnew;
      }
    }
    __syncthreads();
    // o = o * alpha + sum_k e_k v_k over this sub-block's slots grp, grp+NG, ...
#pragma unroll
    for (int h = 0; h < G; ++h) {
      o0[h] *= As[h];
      o1[h] *= As[h];
    }
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const int k = grp + i * NG;
      if (k >= nk) break;
      const float v0 = bf_lo(vv[i]), v1 = bf_hi(vv[i]);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float e = S[h][k];
        o0[h] = fmaf(e, v0, o0[h]);
        o1[h] = fmaf(e, v1, o1[h]);
      }
    }
    if (s0 + SUB < end) issue(s0 + SUB);
    __syncthreads();  // S is rewritten by the next sub-block
  }

#pragma unroll
  for (int h = 0; h < G; ++h) {
    O[grp][h][2 * dp] = o0[h];
    O[grp][h][2 * dp + 1] = o1[h];
  }
  __syncthreads();
  for (int i = tid; i < G * (D + 2); i += 256) {
    const int h = i / (D + 2), j = i % (D + 2);
    float val;
    if (j == 0) val = Ms[h];
    else if (j == 1) val = Ls[h];
    else {
      val = 0.f;
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) val += O[gi][h][j - 2];
    }
    part[(((size_t)rt * nq + (size_t)g * G + h) * MAXB + b) * (D + 2) + j] = val;
  }

}

template <int D>
__global__ __launch_bounds__(D) void attn_merge_kernel(const float* __restrict__ part,
                                                       RowTable tab, int nq,
                                                       bf16_t* __restrict__ out) {
  __shared__ float wts[MAXB];
  __shared__ float lsum[MAXB];
  const int h = blockIdx.x, rt = blockIdx.y, j = threadIdx.x;
  const int seq = rt / tab.rows_per_seq;
  const int p = tab.pos0[seq] + rt % tab.rows_per_seq;
  const int nb = p / block_slots(p) + 1;
  const float* pp = part + ((size_t)rt * nq + h) * MAXB * (D + 2);
  // every load of the row is issued before the first is needed
  float ob[MAXB];
#pragma unroll
  for (int b = 0; b < MAXB; ++b) ob[b] = b < nb ? pp[(size_t)b * (D + 2) + 2 + j] : 0.f;
  if (j < nb) {
    wts[j] = pp[(size_t)j * (D + 2)];
    lsum[j] = pp[(size_t)j * (D + 2) + 1];
  }
  __syncthreads();
  float M = -INFINITY;
  for (int b = 0; b < nb; ++b) M = fmaxf(M, wts[b]);
  __syncthreads();
  if (j < nb) wts[j] = expf(wts[j] - M);
  __syncthreads();
  float L = 0.f, O = 0.f;
#pragma unroll
  for (int b = 0; b < MAXB; ++b) {
    if (b < nb) {
      const float w = wts[b];
      L = fmaf(lsum[b], w, L);
      O = fmaf(ob[b], w, O);
    }
  }
  out[((size_t)rt * nq + h) * D + j] = f2bf(O / L);
}

template <int D, int G>
void launch_dg(const void* q, const RowTable& tab, int rows, int nq, int nkv, float* part,
               int nb_launch, void* out, hipStream_t s) {
  hipLaunchKernelGGL((attn_decode_kernel<D, G>), dim3(nb_launch, nkv, rows), dim3(256), 0, s,
                     (const bf16_t*)q, tab, nq, nkv, part);
  hipLaunchKernelGGL((attn_merge_kernel<D>), dim3(nq, rows), dim3(D), 0, s, part, tab, nq,
                     (bf16_t*)out);
}

template <int D>
void launch_d(int G, const void* q, const RowTable& tab, int rows, int nq, int nkv, float* part,
              int nb_launch, void* out, hipStream_t s) {
  switch (G) {
#define CASE(g) \
  case g: launch_dg<D, g>(q, tab, rows, nq, nkv, part, nb_launch, out, s); break;
    CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8)
#undef CASE
    default: break;
  }
}

int host_block_slots(int p) {
  int kb = SUB;
  while (p + 1 > kb * MAXB) kb <<= 1;
  return kb;
}

}  // namespace

int attn_max_blocks() { return MAXB; }

// q: [rows][nq][d] after RoPE; out: [rows][nq][d].  part holds
// rows * nq * 64 * (d + 2) floats.
void launch_attn_decode(const void* q, const RowTable& tab, int rows, int nq, int nkv, int d,
                        float* part, void* out, hipStream_t s) {
  int nb_launch = 1;
  int nseq = (rows + tab.rows_per_seq - 1) / tab.rows_per_seq;
  for (int i = 0; i < nseq; ++i)
    for (int r = 0; r < tab.rows_per_seq; ++r) {
      int p = tab.pos0[i] + r;
      nb_launch = max(nb_launch, p / host_block_slots(p) + 1);
    }
  int G = nq / nkv;
  if (d == 64) launch_d<64>(G, q, tab, rows, nq, nkv, part, nb_launch, out, s);
  else launch_d<128>(G, q, tab, rows, nq, nkv, part, nb_launch, out, s);
}
