// Glue kernels of the forward step: embedding gather, RMSNorm, RoPE with the
// cache write, greedy argmax, the acceptance of a drafted round.  Rounding points follow the pull request
// "llama: Nanbeige4.3-33B on Metal, the bf16 release served as published",
// section "How".
#include "common.h"
#include "launch.h"

__global__ void fill_zero_kernel(int* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

void launch_fill_zero(int* p, int n, hipStream_t s) {
  hipLaunchKernelGGL(fill_zero_kernel, dim3(1), dim3(64), 0, s, p, n);
}

// ------------------------------------------------------------ embedding ----
// h[r] = E[tok[r]] (a copy); an id outside [0, vocab) yields a NaN row, which
// the greedy draw then refuses, rather than an out-of-bounds read.
__global__ __launch_bounds__(256) void embed_kernel(const bf16_t* __restrict__ E, int vocab,
                                                    int H, const int32_t* __restrict__ tok,
                                                    bf16_t* __restrict__ h) {
  int r = blockIdx.x;
  int t = tok[r];
  uint4* dst = (uint4*)(h + (size_t)r * H);
  int nv = H / 8;
  if (t < 0 || t >= vocab) {
    uint4 nan = make_uint4(0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u, 0x7FC07FC0u);
    for (int i = threadIdx.x; i < nv; i += blockDim.x) dst[i] = nan;
    return;
  }
  const uint4* src = (const uint4*)(E + (size_t)t * H);
  for (int i = threadIdx.x; i < nv; i += blockDim.x) dst[i] = src[i];
}

void launch_embed(const void* E, int vocab, int H, const int32_t* tok, void* h, int rows,
                  hipStream_t s) {
  hipLaunchKernelGGL(embed_kernel, dim3(rows), dim3(256), 0, s, (const bf16_t*)E, vocab, H, tok,
                     (bf16_t*)h);
}

// -------------------------------------------------------------- RMSNorm ----
// out = bf16(w * bf16(x * r)) with r and x * r as row_inv_rms and norm8 form
// them: one wave per row, four rows per workgroup.  In place (out == h) is allowed: each
// element is read and then written by the same lane, after the row's sum.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const bf16_t* h, const bf16_t* __restrict__ w,
                                                      bf16_t* out, int rows, int H, float eps) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;  // uniform per wave; no barrier follows
  const bf16_t* x = h + (size_t)r * H;
  const double rs = row_inv_rms(x, H, eps);
  const u32x4_t* xv = (const u32x4_t*)x;
  const u32x4_t* wv = (const u32x4_t*)w;
  u32x4_t* o = (u32x4_t*)(out + (size_t)r * H);
  for (int v = lane_id(); v < H / 8; v += WAVE) o[v] = norm8(xv[v], wv[v], rs);
}

void launch_rmsnorm(const void* h, const void* w, void* out, int rows, int H, float eps,
                    hipStream_t s) {
  hipLaunchKernelGGL(rmsnorm_kernel, dim3((rows + 3) / 4), dim3(256), 0, s, (const bf16_t*)h,
                     (const bf16_t*)w, (bf16_t*)out, rows, H, eps);
}

// ------------------------------------------------------- RoPE + caching ----
// Unscaled NeoX RoPE (Nanbeige4.3-33B NInfer card, "Provenance and
// representation": half-head pairs (i, i + d/2), theta 1.2e8):
//   inv_i = fp32(1 / fp32(theta^(2i/d))), angle a = fp32(p * inv_i),
//   c, s = bf16(fp32(cos a)), bf16(fp32(sin a)),
//   x'_i = bf16(bf16(x_i c) + bf16(-x_{i+d/2} s)),
//   x'_{i+d/2} = bf16(bf16(x_{i+d/2} c) + bf16(x_i s)).
// The power and cos / sin are evaluated in binary64 and rounded to fp32.
// Every execution of a pass uses the same positions, so the table of (c, s)
// per row is computed once per pass.
__global__ void rope_table_kernel(RowTable tab, int rows, int d, float theta, float2* table) {
  const int half = d / 2;
  const int n = rows * half;
  for (int t = blockIdx.x * blockDim.x + threadIdx.x; t < n; t += gridDim.x * blockDim.x) {
    const int rt = t / half, i = t % half;
    const int seq = rt / tab.rows_per_seq;
    const int p = tab.pos0[seq] + rt % tab.rows_per_seq;
    const float e = (float)(2 * i) / (float)d;
    const float inv = 1.0f / (float)pow((double)theta, (double)e);
    const float a = __fmul_rn((float)p, inv);
    table[t] = make_float2(rbf((float)cos((double)a)), rbf((float)sin((double)a)));
  }
}

void launch_rope_table(const RowTable& tab, int rows, int d, float theta, void* table,
                       hipStream_t s) {
  int n = rows * (d / 2);
  int grid = (n + 255) / 256;
  if (grid > 1024) grid = 1024;
  hipLaunchKernelGGL(rope_table_kernel, dim3(grid), dim3(256), 0, s, tab, rows, d, theta,
                     (float2*)table);
}

// Prompt chunks: RoPE on the q and k heads of each row of the projection
// output qkv [rows][qd + 2*kvd], then k and v stored at slot p of the row's
// cache.  One workgroup per row; a thread takes eight neighbouring pairs of
// one head (16-byte loads and stores of both halves).
__global__ __launch_bounds__(256) void rope_kv_kernel(const bf16_t* __restrict__ qkv,
                                                      bf16_t* __restrict__ qout, RowTable tab,
                                                      int nq, int nkv, int d,
                                                      const float2* __restrict__ table) {
  const int rt = blockIdx.x;
  const int seq = rt / tab.rows_per_seq;
  const int p = tab.pos0[seq] + rt % tab.rows_per_seq;
  const int half = d / 2, ng = half / 8;  // eight-pair groups per head
  const int qd = nq * d, kvd = nkv * d;
  const bf16_t* src = qkv + (size_t)rt * (qd + 2 * kvd);
  bf16_t* kdst = tab.k[seq] + (size_t)p * kvd;
  bf16_t* vdst = tab.v[seq] + (size_t)p * kvd;
  const float2* cs = table + (size_t)rt * half;
  const int items = (nq + nkv) * ng;
  for (int it = threadIdx.x; it < items; it += blockDim.x) {
    const int hh = it / ng, i0 = 8 * (it % ng);
    const bf16_t* x = src + hh * d;  // q heads then k heads, contiguous
    const u32x4_t a = *(const u32x4_t*)(x + i0), b = *(const u32x4_t*)(x + i0 + half);
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
    uint32_t o1w[4], o2w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t r1 = 0, r2 = 0;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const float x1 = __uint_as_float(k ? aw[e] & 0xFFFF0000u : aw[e] << 16);
        const float x2 = __uint_as_float(k ? bw[e] & 0xFFFF0000u : bw[e] << 16);
        const float2 c = cs[i0 + 2 * e + k];
        r1 |= (uint32_t)f2bf(rbf(x1 * c.x) + rbf(-x2 * c.y)) << (16 * k);
        r2 |= (uint32_t)f2bf(rbf(x2 * c.x) + rbf(x1 * c.y)) << (16 * k);
      }
      o1w[e] = r1;
      o2w[e] = r2;
    }
    bf16_t* dst = hh < nq ? qout + (size_t)rt * qd + hh * d : kdst + (hh - nq) * d;
    *(u32x4_t*)(dst + i0) = u32x4_t{o1w[0], o1w[1], o1w[2], o1w[3]};
    *(u32x4_t*)(dst + i0 + half) = u32x4_t{o2w[0], o2w[1], o2w[2], o2w[3]};
  }
  const u32x4_t* vs = (const u32x4_t*)(src + qd + kvd);
  u32x4_t* vd = (u32x4_t*)vdst;
  for (int i = threadIdx.x; i < kvd / 8; i += blockDim.x) vd[i] = vs[i];
}

void launch_rope_kv(const void* qkv, void* qout, const RowTable& tab, int rows, int nq, int nkv,
                    int d, const void* table, hipStream_t s) {
  hipLaunchKernelGGL(rope_kv_kernel, dim3(rows), dim3(256), 0, s, (const bf16_t*)qkv,
                     (bf16_t*)qout, tab, nq, nkv, d, (const float2*)table);
}

// --------------------------------------------------------------- argmax ----
// Greedy draw over bf16 logits: largest value, ties to the lowest id (review
// reply "Teacher-forced misses"); a row holding NaN or +-Inf yields -1 and
// raises the model's non-finite flag.  Stage 1: each workgroup scans one
// chunk of a row.  Stage 2: one wave merges a row's chunks in order.
#define ARGMAX_CHUNK 4096

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

__global__ __launch_bounds__(256) void argmax_partial_kernel(const bf16_t* __restrict__ logits,
                                                             int V, int ld, float* pv, int* pi,
                                                             int nchunk) {
  __shared__ float sv[4];
  __shared__ int si[4], sbad[4];
  int c = blockIdx.x, r = blockIdx.y;
  const bf16_t* row = logits + (size_t)r * ld;
  int beg = c * ARGMAX_CHUNK, end = min(V, beg + ARGMAX_CHUNK);
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF, bad = 0;
  for (int i = beg + threadIdx.x; i < end; i += 256) {
    float v = bf2f(row[i]);
    if (!isfinite(v)) bad = 1;
    if (better(v, i, bv, bi)) { bv = v; bi = i; }
  }
  for (int m = 32; m >= 1; m >>= 1) {
    float ov = __shfl_xor(bv, m, WAVE);
    int oi = __shfl_xor(bi, m, WAVE);
    bad |= __shfl_xor(bad, m, WAVE);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  int w = threadIdx.x >> 6;
  if (lane_id() == 0) { sv[w] = bv; si[w] = bi; sbad[w] = bad; }
  __syncthreads();
  if (threadIdx.x == 0) {
    bv = sv[0]; bi = si[0]; bad = sbad[0];
    for (int k = 1; k < 4; ++k) {
      if (better(sv[k], si[k], bv, bi)) { bv = sv[k]; bi = si[k]; }
      bad |= sbad[k];
    }
    pv[r * nchunk + c] = bad ? NAN : bv;
    pi[r * nchunk + c] = bi;
  }
}

__global__ __launch_bounds__(64) void argmax_final_kernel(const float* pv, const int* pi,
                                                          int nchunk, int32_t* out, int* flag) {
  int r = blockIdx.x;
  float bv = -INFINITY;
  int bi = 0x7FFFFFFF, bad = 0;
  for (int c = lane_id(); c < nchunk; c += WAVE) {
    float v = pv[r * nchunk + c];
    if (isnan(v)) bad = 1;
    else if (better(v, pi[r * nchunk + c], bv, bi)) { bv = v; bi = pi[r * nchunk + c]; }
  }
  for (int m = 32; m >= 1; m >>= 1) {
    float ov = __shfl_xor(bv, m, WAVE);
    int oi = __shfl_xor(bi, m, WAVE);
    bad |= __shfl_xor(bad, m, WAVE);
    if (better(ov, oi, bv, bi)) { bv = ov; bi = oi; }
  }
  if (lane_id() == 0) {
    if (out) out[r] = bad ? -1 : bi;
    if (bad) atomicOr(flag, 1);
  }
}

int argmax_chunks(int V) { return (V + ARGMAX_CHUNK - 1) / ARGMAX_CHUNK; }

void launch_argmax(const void* logits, int V, int ld, int rows, float* pv, int* pi,
                   int32_t* out, int* flag, hipStream_t s) {
  int nchunk = argmax_chunks(V);
  hipLaunchKernelGGL(argmax_partial_kernel, dim3(nchunk, rows), dim3(256), 0, s,
                     (const bf16_t*)logits, V, ld, pv, pi, nchunk);
  hipLaunchKernelGGL(argmax_final_kernel, dim3(rows), dim3(64), 0, s, pv, pi, nchunk, out, flag);
}

// ------------------------------------------------------- drafted rounds ----
// One drafted round (issue "A llama family on Metal", follow-ups: a smaller
// Llama on the same tokenizer drafting with replies unchanged; pull request,
// reply "Drafting": drafted greedy equals plain greedy).  win = [last, d_1 ..
// d_k] are the window's input tokens (d_i the draft's proposals), t[0..k] the
// target's greedy tokens after each of them.  The target agrees with the
// first a proposals where d_{i+1} == t_i for all i < a (a valid id); the
// round yields d_1 .. d_a and then t_a, the target's own next token, so the
// reply is the one plain greedy steps give.  One lane; writes a to *count.
__global__ void draft_accept_kernel(const int32_t* __restrict__ win, const int32_t* __restrict__ t,
                                    int k, int32_t* __restrict__ out, int32_t* __restrict__ count) {
  if (threadIdx.x != 0) return;
  int a = 0;
  while (a < k && t[a] >= 0 && win[a + 1] == t[a]) {
    out[a] = t[a];
    ++a;
  }
  out[a] = t[a];
  *count = a;
}

void launch_draft_accept(const int32_t* win, const int32_t* t, int k, int32_t* out,
                         int32_t* count, hipStream_t s) {
  hipLaunchKernelGGL(draft_accept_kernel, dim3(1), dim3(64), 0, s, win, t, k, out, count);
}
