// Grouped-query attention for decode rows (pull request "llama:
// Nanbeige4.3-33B on Metal, the bf16 release served as published", section
// "How": decode rows over key blocks at absolute positions).
//
// A row at absolute position p attends to cache slots [0, p].  Keys are
// split into blocks of KB slots anchored at absolute positions (block b holds
// slots [b*KB, (b+1)*KB)), so the work a row does depends only on p, never on
// the window or batch it came in.  Pass 1, one workgroup per (block, KV
// head, row): the G query heads that share the KV head score the block's keys
// (fp32), take the block max m_b, the exponentials' sum l_b and the
// unnormalised sum o_b of exp(s - m_b) v.  Pass 2, one workgroup per
// (query head, row): merge the blocks in block order,
// o = sum_b e^(m_b - M) o_b / sum_b e^(m_b - M) l_b, rounded once to bf16.
#include "common.h"
#include "launch.h"

#define KB 256

int attn_key_block() { return KB; }

template <int D, int G>
__global__ __launch_bounds__(256) void attn_partial_kernel(const bf16_t* __restrict__ q,
                                                           RowTable tab, int nq, int nkv,
                                                           float* __restrict__ part,
                                                           int max_blocks) {
  constexpr int DP = D / 2;          // bf16 pairs per head
  constexpr int NG = 256 / DP;       // key groups in the value pass
  __shared__ __attribute__((aligned(16))) uint32_t qs[G][DP];
  __shared__ float S[G][KB];
  __shared__ float O[NG][G][D];
  const int b = blockIdx.x, g = blockIdx.y, rt = blockIdx.z;
  const int seq = rt / tab.rows_per_seq;
  const int p = tab.pos0[seq] + rt % tab.rows_per_seq;
  const int start = b * KB;
  if (start > p) return;  // this row has no keys in block b (uniform per workgroup)
  const int nk = min(KB, p + 1 - start);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  const uint32_t* qsrc = (const uint32_t*)(q + ((size_t)rt * nq + (size_t)g * G) * D);
  for (int i = tid; i < G * DP; i += 256) qs[i / DP][i % DP] = qsrc[i];
  __syncthreads();

  // scores: thread t scores key start + t for the G heads
  const float scale = 1.0f / sqrtf((float)D);
  {
    float s[G];
#pragma unroll
    for (int h = 0; h < G; ++h) s[h] = 0.f;
    if (tid < nk) {
      const uint4* krow =
          (const uint4*)(tab.k[seq] + ((size_t)(start + tid) * nkv + g) * D);
#pragma unroll 4
      for (int j = 0; j < D / 8; ++j) {
        uint4 kv = krow[j];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const uint4 qv = *(const uint4*)&qs[h][4 * j];
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
    for (int h = 0; h < G; ++h) S[h][tid] = tid < nk ? s[h] * scale : -INFINITY;
  }
  __syncthreads();

  // block max and exponentials per head (waves take heads round-robin)
  __shared__ float Mh[G], Lh[G];
  for (int h = wave; h < G; h += 4) {
    float m = -INFINITY;
    for (int k = lane; k < KB; k += WAVE) m = fmaxf(m, S[h][k]);
    m = wave_max(m);
    float l = 0.f;
    for (int k = lane; k < KB; k += WAVE) {
      float e = k < nk ? expf(S[h][k] - m) : 0.f;
      S[h][k] = e;
      l += e;
    }
    l = wave_sum(l);
    if (lane == 0) { Mh[h] = m; Lh[h] = l; }
  }
  __syncthreads();

  // o_b = sum_k e_k v_k: thread (grp, dp) covers dims 2dp, 2dp+1 for keys grp, grp+NG, ...
  {
    const int dp = tid % DP, grp = tid / DP;
    float o0[G], o1[G];
#pragma unroll
    for (int h = 0; h < G; ++h) { o0[h] = 0.f; o1[h] = 0.f; }
    const uint32_t* vbase = (const uint32_t*)(tab.v[seq] + ((size_t)start * nkv + g) * D) + dp;
    const int vstride = nkv * DP;  // uint32 per position
    for (int k = grp; k < nk; k += NG) {
      uint32_t vv = vbase[(size_t)k * vstride];
      float v0 = bf_lo(vv), v1 = bf_hi(vv);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float e = S[h][k];
        o0[h] = fmaf(e, v0, o0[h]);
        o1[h] = fmaf(e, v1, o1[h]);
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      O[grp][h][2 * dp] = o0[h];
      O[grp][h][2 * dp + 1] = o1[h];
    }
  }
  __syncthreads();

  for (int i = tid; i < G * (D + 2); i += 256) {
    int h = i / (D + 2), j = i % (D + 2);
    float val;
    if (j == 0) val = Mh[h];
    else if (j == 1) val = Lh[h];
    else {
      val = 0.f;
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) val += O[gi][h][j - 2];
    }
    part[(((size_t)rt * nq + (size_t)g * G + h) * max_blocks + b) * (D + 2) + j] = val;
  }
}

template <int D>
__global__ __launch_bounds__(128) void attn_merge_kernel(const float* __restrict__ part,
                                                         RowTable tab, int nq, int max_blocks,
                                                         bf16_t* __restrict__ out) {
  const int h = blockIdx.x, rt = blockIdx.y, j = threadIdx.x;
  if (j >= D) return;
  const int seq = rt / tab.rows_per_seq;
  const int p = tab.pos0[seq] + rt % tab.rows_per_seq;
  const int nb = p / KB + 1;
  const float* pp = part + ((size_t)rt * nq + h) * max_blocks * (D + 2);
  float M = -INFINITY;
  for (int b = 0; b < nb; ++b) M = fmaxf(M, pp[(size_t)b * (D + 2)]);
  float L = 0.f, O = 0.f;
  for (int b = 0; b < nb; ++b) {
    const float* q = pp + (size_t)b * (D + 2);
    float w = expf(q[0] - M);
    L = fmaf(q[1], w, L);
    O = fmaf(q[2 + j], w, O);
  }
  out[((size_t)rt * nq + h) * D + j] = f2bf(O / L);
}

template <int D, int G>
static void launch_dg(const void* q, const RowTable& tab, int rows, int nq, int nkv, float* part,
                      int max_blocks, int nb_launch, void* out, hipStream_t s) {
  hipLaunchKernelGGL((attn_partial_kernel<D, G>), dim3(nb_launch, nkv, rows), dim3(256), 0, s,
                     (const bf16_t*)q, tab, nq, nkv, part, max_blocks);
  hipLaunchKernelGGL((attn_merge_kernel<D>), dim3(nq, rows), dim3(D), 0, s, part, tab, nq,
                     max_blocks, (bf16_t*)out);
}

template <int D>
static void launch_d(int G, const void* q, const RowTable& tab, int rows, int nq, int nkv,
                     float* part, int max_blocks, int nb_launch, void* out, hipStream_t s) {
  switch (G) {
#define CASE(g) \
  case g: launch_dg<D, g>(q, tab, rows, nq, nkv, part, max_blocks, nb_launch, out, s); break;
    CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8)
#undef CASE
    default: break;
  }
}

// q: [rows][nq][d] after RoPE; out: [rows][nq][d].  part holds
// rows * nq * max_blocks * (d + 2) floats.
void launch_attn_decode(const void* q, const RowTable& tab, int rows, int nq, int nkv, int d,
                        float* part, int max_blocks, void* out, hipStream_t s) {
  int maxp = 0;
  int nseq = (rows + tab.rows_per_seq - 1) / tab.rows_per_seq;
  for (int i = 0; i < nseq; ++i) maxp = max(maxp, tab.pos0[i] + tab.rows_per_seq - 1);
  int nb_launch = maxp / KB + 1;
  int G = nq / nkv;
  if (d == 64) launch_d<64>(G, q, tab, rows, nq, nkv, part, max_blocks, nb_launch, out, s);
  else launch_d<128>(G, q, tab, rows, nq, nkv, part, max_blocks, nb_launch, out, s);
}
