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
// One workgroup per (block, KV head, row); its four waves each walk a fixed
// quarter of the block on their own, 16 slots at a time, with the next two
// tiles' keys and values in flight.  Scores come from one MFMA chain per tile,
// S^T = K Q^T (v_mfma_f32_16x16x32_bf16: the tile's 16 key rows against the G
// query heads sharing the KV head, padded to 16), so lane l holds head l%16 for
// slots 4(l/16)..+3; an online softmax keeps each head's running max and sum;
// lanes per value dimension pair accumulate exp(s - m) v in fp32 with the
// weights broadcast from the score lanes.  The quarters' (max, sum, output)
// are combined in quarter order into the block's partial.  A second kernel,
// one workgroup per (query head, row), merges a row's blocks in block order,
// o = sum_b e^(m_b - M) o_b / sum_b e^(m_b - M) l_b, rounded once to bf16.
// (The kernel boundary makes the partials visible across the chip's separate
// L2s; merging inside the first kernel would need a device-scope release in
// every workgroup.)
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

// WIDE: the wave index stays a vector value, which holds the kernel at ~216
// registers, two waves per SIMD; as a scalar it takes ~168 and runs three
// waves per SIMD.  Same arithmetic, same bits.  Measured per launch: one or
// two rows at 65k-131k positions (512-1,024 workgroups) take 4-10% less time
// with two waves per SIMD; 16-row windows at 4,096 positions (8,192
// workgroups) 14% less with three.
template <int D, int G, bool WIDE>
__global__ __launch_bounds__(256) void attn_decode_kernel(const bf16_t* __restrict__ q,
                                                          RowTable tab, int nq, int nkv,
                                                          float* __restrict__ part) {
  constexpr int TS = 16;        // slots per tile
  constexpr int KST = D / 32;   // MFMA steps over the head dimension
  constexpr int DP = D / 2;     // value pairs per head
  constexpr int NSG = 64 / DP;  // slot groups in the value pass (1 for d = 128, 2 for 64)
  constexpr int VPL = TS / NSG; // value slots per lane per tile
  static_assert(G <= 16 && NSG * DP == 64, "decode attention geometry");
  __shared__ float sm[4][G], sl[4][G];
  __shared__ float so[4][G][D];

  const int b = blockIdx.x, g = blockIdx.y, rt = blockIdx.z;
  const int seq = rt / tab.rows_per_seq;
  const int p = tab.pos0[seq] + rt % tab.rows_per_seq;
  const int kb = block_slots(p);
  const int nb = p / kb + 1;
  if (b >= nb) return;  // uniform per workgroup
  const int start = b * kb, end = min(start + kb, p + 1);
  const int lane = threadIdx.x & 63;
  const int wave = WIDE ? (int)(threadIdx.x >> 6) : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ql = kb / 4;  // a multiple of 16
  const int ws = start + wave * ql, we = min(ws + ql, end);  // this wave's slots
  const int ntile = we > ws ? (we - ws + TS - 1) / TS : 0;
  const int kvd = nkv * D;
  const float scale = 1.0f / sqrtf((float)D);

  // Q^T fragments (MFMA B operand): lane l holds head l%16, dims 8(l/16) + 32i
  const int hl = lane & 15, dq = (lane >> 4) * 8;
  bf16x8_t qf[KST];
#pragma unroll
  for (int i = 0; i < KST; ++i) {
    if (hl < G) {
      qf[i] = *(const bf16x8_t*)(q + ((size_t)rt * nq + (size_t)g * G + hl) * D + 32 * i + dq);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[i][e] = (__bf16)0.0f;
    }
  }
  // K fragments (A operand): lane l holds slot l%16 of the tile, dims
  // 8(l/16) + 32i; values: lane l holds pair l%DP of slots l/DP + NSG*j.
  // Slots past the wave's range re-read its last slot (never used).  The
  // loads are non-temporal: a step reads each layer's cache once, and 52
  // layers' caches and weights pass through the caches between two reads of
  // the same slot (in the 33B model: 2k context 0.7% more tok/s, 131k 3.9%).
  const bf16_t* kbase = tab.k[seq] + (size_t)g * D + dq;
  const uint32_t* vbase = (const uint32_t*)(tab.v[seq] + (size_t)g * D) + lane % DP;
  const int vg = lane / DP;
  bf16x8_t kq[2][KST];
  uint32_t vq[2][VPL];
  auto issue = [&](int t, int set) {
    const int s0 = ws + t * TS;
    const int sk = min(s0 + hl, we - 1);
#pragma unroll
    for (int i = 0; i < KST; ++i)
      kq[set][i] = __builtin_nontemporal_load((const bf16x8_t*)(kbase + (size_t)sk * kvd + 32 * i));
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const int sv = min(s0 + vg + NSG * j, we - 1);
      vq[set][j] = __builtin_nontemporal_load(vbase + (size_t)sv * (kvd / 2));
    }
  };

  float mrun = -INFINITY, lrun = 0.f;  // head hl's running max and sum
  float o0[G], o1[G];
#pragma unroll
  for (int h = 0; h < G; ++h) { o0[h] = 0.f; o1[h] = 0.f; }

  auto step = [&](int t, int set) {
    bf16x8_t kf[KST];
    uint32_t vv[VPL];
#pragma unroll
    for (int i = 0; i < KST; ++i) kf[i] = kq[set][i];
#pragma unroll
    for (int j = 0; j < VPL; ++j) vv[j] = vq[set][j];
    issue(t + 2, set);
    const int s0 = ws + t * TS;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < KST; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[i], qf[i], acc, 0, 0, 0);
    // lane l: head hl, slots s0 + 4(l/16) + j
    float sc[4], mt = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sc[j] = s0 + 4 * (lane >> 4) + j < we ? acc[j] * scale : -INFINITY;
      mt = fmaxf(mt, sc[j]);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 16, WAVE));
    mt = fmaxf(mt, __shfl_xor(mt, 32, WAVE));
    const float mnew = fmaxf(mrun, mt);
    const float alpha = expf(mrun - mnew);  // 0 on the first tile (mrun = -inf)
    float e[4], lt = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      e[j] = expf(sc[j] - mnew);
      lt += e[j];
    }
    lt += __shfl_xor(lt, 16, WAVE);
    lt += __shfl_xor(lt, 32, WAVE);
    lrun = lrun * alpha + lt;
    mrun = mnew;
    // o = o * alpha + (sum over the tile's slots of e v), the tile's sum
    // formed on its own first (weights from lane h + 16(u/4), register u%4,
    // for slot u): each running sum takes one rounding per tile, so its error
    // does not grow with the number of slots a wave walks.
    float t0[G], t1[G];
#pragma unroll
    for (int j = 0; j < VPL; ++j) {
      const float v0 = bf_lo(vv[j]), v1 = bf_hi(vv[j]);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float w;
        if (NSG == 1) {
          w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e[j % 4]), h + 16 * (j / 4)));
        } else {  // lanes of slot group vg take slot vg + 2j
          const int u0 = 2 * j, u1 = 2 * j + 1;
          const float w0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e[u0 % 4]), h + 16 * (u0 / 4)));
          const float w1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e[u1 % 4]), h + 16 * (u1 / 4)));
          w = vg ? w1 : w0;
        }
        t0[h] = j ? fmaf(w, v0, t0[h]) : w * v0;
        t1[h] = j ? fmaf(w, v1, t1[h]) : w * v1;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), h));
      o0[h] = fmaf(o0[h], a, t0[h]);
      o1[h] = fmaf(o1[h], a, t1[h]);
    }
  };
  if (ntile > 0) {
    issue(0, 0);
    issue(1, 1);
    int t = 0;
    for (; t + 1 < ntile; t += 2) {
      step(t, 0);
      step(t + 1, 1);
    }
    if (t < ntile) step(t, 0);
  }
  // the two slot groups' sums (d = 64), in group order
  if (NSG == 2) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float a0 = __shfl_xor(o0[h], 32, WAVE), a1 = __shfl_xor(o1[h], 32, WAVE);
      if (vg == 0) { o0[h] += a0; o1[h] += a1; }
    }
  }
  if (lane < G) {
    sm[wave][lane] = mrun;
    sl[wave][lane] = lrun;
  }
  if (vg == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      so[wave][h][2 * (lane % DP)] = o0[h];
      so[wave][h][2 * (lane % DP) + 1] = o1[h];
    }
  }
  __syncthreads();
  // the block's partial: its quarters combined in order (an empty quarter has
  // max -inf and adds nothing; quarter 0 always holds the block's first slot)
  for (int i = threadIdx.x; i < G * (D + 2); i += 256) {
    const int h = i / (D + 2), j = i % (D + 2);
    float M = sm[0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, sm[w][h]);
    float val = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = expf(sm[w][h] - M);
      val += f * (j == 0 ? 0.f : j == 1 ? sl[w][h] : so[w][h][j - 2]);
    }
    if (j == 0) val = M;
    part[(((size_t)rt * nq + (size_t)g * G + h) * MAXB + b) * (D + 2) + j] = val;
  }
}

template <int D>
__global__ __launch_bounds__(D) void attn_merge_kernel(const float* __restrict__ part,
                                                       RowTable tab, int nq,
                                                       bf16_t* __restrict__ out,
                                                       float* __restrict__ out32) {
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
  for (int b = j; b < nb; b += D) {
    wts[b] = pp[(size_t)b * (D + 2)];
    lsum[b] = pp[(size_t)b * (D + 2) + 1];
  }
  __syncthreads();
  float M = -INFINITY;
  for (int b = 0; b < nb; ++b) M = fmaxf(M, wts[b]);
  __syncthreads();
  for (int b = j; b < nb; b += D) wts[b] = expf(wts[b] - M);
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
  if (out32) out32[((size_t)rt * nq + h) * D + j] = O / L;  // parity probe
}

template <int D, int G>
void launch_dg(const void* q, const RowTable& tab, int rows, int nq, int nkv, float* part,
               int nb_launch, void* out, float* out32, hipStream_t s) {
  // up to four workgroups per CU of the 256 (two rounds at two per CU): the
  // two-wave form; more: the three-wave form
  if ((long)nb_launch * nkv * rows <= 1024)
    launch_k((attn_decode_kernel<D, G, true>), dim3(nb_launch, nkv, rows), dim3(256), 0, s,
             (const bf16_t*)q, tab, nq, nkv, part);
  else
    launch_k((attn_decode_kernel<D, G, false>), dim3(nb_launch, nkv, rows), dim3(256), 0, s,
             (const bf16_t*)q, tab, nq, nkv, part);
  launch_k((attn_merge_kernel<D>), dim3(nq, rows), dim3(D), 0, s, part, tab, nq,
                     (bf16_t*)out, out32);
}

template <int D>
void launch_d(int G, const void* q, const RowTable& tab, int rows, int nq, int nkv, float* part,
              int nb_launch, void* out, float* out32, hipStream_t s) {
  switch (G) {
#define CASE(g) \
  case g: launch_dg<D, g>(q, tab, rows, nq, nkv, part, nb_launch, out, out32, s); break;
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
                        float* part, void* out, float* out32, hipStream_t s) {
  int nb_launch = 1;
  int nseq = (rows + tab.rows_per_seq - 1) / tab.rows_per_seq;
  for (int i = 0; i < nseq; ++i)
    for (int r = 0; r < tab.rows_per_seq; ++r) {
      int p = tab.pos0[i] + r;
      nb_launch = max(nb_launch, p / host_block_slots(p) + 1);
    }
  int G = nq / nkv;
  if (d == 64) launch_d<64>(G, q, tab, rows, nq, nkv, part, nb_launch, out, out32, s);
  else launch_d<128>(G, q, tab, rows, nq, nkv, part, nb_launch, out, out32, s);
}
