// Seeded sampling of bf16 logit rows on the GPU (issue "A llama family on
// Metal", the served sampling checks; pull request "llama: Nanbeige4.3-33B on
// Metal, the bf16 release served as published", section "How": tokens drawn
// on the GPU; model card "Nanbeige4.3-33B EXL3", upstream's recommended
// temperature, top_p and top_k).  Temperature, top-k, top-p in that order,
// then one draw against a caller-given uniform u in [0, 1):
//   z = logit / T; the top_k largest z ordered by value (descending), then id;
//   e_i = exp(z_i - z_0), S = sum e_i; candidate i stays while the weight of
//   the candidates before it is below top_p * S (the first always stays); the
//   token is the first remaining candidate whose running weight exceeds
//   u * (remaining weight).
// Top-k selects on the bf16 logits themselves (T > 0 keeps the order), so the
// candidate set is exact.  Stage 1: each workgroup extracts the top_k of one
// 4,096-logit chunk of a row, largest first, by repeated block-wide maxima.
// Stage 2: one workgroup per row extracts the row's top_k from the chunks'
// candidates the same way, then one lane forms the weights and draws in fp32
// in candidate order.  A row holding NaN or +-Inf yields -1 and raises the
// model's non-finite flag.
#include "common.h"
#include "launch.h"

#include <mutex>

namespace {

constexpr int CHUNK = 4096;
constexpr int PER_THREAD = CHUNK / 256;

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// Block-wide best (value desc, id asc) of the 256 threads' offers.
__device__ __forceinline__ void block_best(float& v, int& i, float* sv, int* si) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(v, m, WAVE);
    const int oi = __shfl_xor(i, m, WAVE);
    if (better(ov, oi, v, i)) { v = ov; i = oi; }
  }
  const int w = threadIdx.x >> 6;
  if (lane_id() == 0) { sv[w] = v; si[w] = i; }
  __syncthreads();
  v = sv[0];
  i = si[0];
#pragma unroll
  for (int k = 1; k < 4; ++k)
    if (better(sv[k], si[k], v, i)) { v = sv[k]; i = si[k]; }
  __syncthreads();
}

__global__ __launch_bounds__(256) void sample_partial_kernel(const bf16_t* __restrict__ logits,
                                                             int V, int64_t ld, int k,
                                                             float* cv, int* ci, int* bad,
                                                             int nchunk) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int c = blockIdx.x, r = blockIdx.y;
  const bf16_t* row = logits + (size_t)r * ld;
  const int beg = c * CHUNK + threadIdx.x;
  float v[PER_THREAD];
  int nonfinite = 0;
#pragma unroll
  for (int j = 0; j < PER_THREAD; ++j) {
    const int i = beg + 256 * j;
    v[j] = i < V ? bf2f(row[i]) : -INFINITY;
    if (i < V && !isfinite(v[j])) nonfinite = 1;
  }
  const size_t o = ((size_t)r * nchunk + c) * k;
  if (__syncthreads_or(nonfinite)) {
    if (threadIdx.x == 0) bad[r * nchunk + c] = 1;
    return;  // uniform per workgroup
  }
  if (threadIdx.x == 0) bad[r * nchunk + c] = 0;
  uint32_t taken = 0;
  for (int t = 0; t < k; ++t) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int j = 0; j < PER_THREAD; ++j) {
      const int i = beg + 256 * j;
      if (i < V && !(taken >> j & 1u) && better(v[j], i, bv, bi)) { bv = v[j]; bi = i; }
    }
    float wv = bv;
    int wi = bi;
    block_best(wv, wi, sv, si);
    if (wi == bi && bi != 0x7FFFFFFF) taken |= 1u << ((bi - beg) / 256);
    if (threadIdx.x == 0) { cv[o + t] = wv; ci[o + t] = wi; }
  }
}

__global__ __launch_bounds__(256) void sample_final_kernel(const float* __restrict__ cv,
                                                           const int* __restrict__ ci,
                                                           const int* __restrict__ bad, int nchunk,
                                                           int k, float temperature, float top_p,
                                                           const float* __restrict__ u,
                                                           int32_t* out, int* flag) {
  constexpr int PT = (64 * 64 + 255) / 256;  // candidates per thread (nchunk * k <= 4096)
  __shared__ float sv[4], tv[64];
  __shared__ int si[4], ti[64];
  const int r = blockIdx.x;
  int isbad = 0;
  for (int c = threadIdx.x; c < nchunk; c += 256) isbad |= bad[r * nchunk + c];
  if (__syncthreads_or(isbad)) {
    if (threadIdx.x == 0) {
      out[r] = -1;
      atomicOr(flag, 1);
    }
    return;
  }
  const int n = nchunk * k;
  const float* rv = cv + (size_t)r * n;
  const int* ri = ci + (size_t)r * n;
  float v[PT];
  int id[PT];
#pragma unroll
  for (int j = 0; j < PT; ++j) {
    const int e = threadIdx.x + 256 * j;
    v[j] = e < n ? rv[e] : -INFINITY;
    id[j] = e < n ? ri[e] : 0x7FFFFFFF;
  }
  uint32_t taken = 0;
  for (int t = 0; t < k; ++t) {
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF, bj = -1;
#pragma unroll
    for (int j = 0; j < PT; ++j)
      if (!(taken >> j & 1u) && id[j] != 0x7FFFFFFF && better(v[j], id[j], bv, bi)) {
        bv = v[j];
        bi = id[j];
        bj = j;
      }
    float wv = bv;
    int wi = bi;
    block_best(wv, wi, sv, si);
    if (bj >= 0 && wi == bi) taken |= 1u << bj;
    if (threadIdx.x == 0) { tv[t] = wv; ti[t] = wi; }
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  // weights and the draw, in candidate order (each weight is recomputed
  // where it is used: the same inputs give the same bits)
  const float z0 = tv[0] / temperature;
  float S = 0.f;
  for (int i = 0; i < k; ++i) S += expf(tv[i] / temperature - z0);
  int kept = 1;
  float cum = expf(tv[0] / temperature - z0);
  while (kept < k && cum < top_p * S) {
    cum += expf(tv[kept] / temperature - z0);
    ++kept;
  }
  const float target = u[r] * cum;
  float c = 0.f;
  int pick = kept - 1;
  for (int i = 0; i < kept; ++i) {
    c += expf(tv[i] / temperature - z0);
    if (c > target) { pick = i; break; }
  }
  out[r] = ti[pick];
}

}  // namespace

int sample_chunks(int V) { return (V + CHUNK - 1) / CHUNK; }

// ---------------------------------------------------------------------------
// Scratch of the variant that allocates nothing (llama_sample_noalloc): the
// candidates, the per-chunk non-finite marks and a flag word live in this
// fixed device array, one copy per GPU for the life of the process.  Host
// code never uses the symbol itself (on the host it only names a stand-in):
// each device's address comes from hipGetSymbolAddress, looked up once per
// device with that device current.
constexpr size_t SCRATCH_CAND = (size_t)SAMPLE_NOALLOC_MAX_ROWS * SAMPLE_NOALLOC_MAX_CAND;
constexpr size_t SCRATCH_BYTES =
    2 * SCRATCH_CAND * 4 + (size_t)SAMPLE_NOALLOC_MAX_ROWS * SAMPLE_NOALLOC_MAX_CHUNKS * 4 + 256;
static __device__ __align__(256) uint8_t scratch[SCRATCH_BYTES];

size_t sample_noalloc_scratch_bytes() { return SCRATCH_BYTES; }

// Device address of this device's scratch array, or nullptr (*err set) if the
// lookup fails.  Cached per device; the lookup runs once per device.
static uint8_t* scratch_ptr(hipError_t* err) {
  static std::mutex mu;
  static uint8_t* ptrs[64] = {};
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= 64) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!ptrs[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess) return nullptr;
    ptrs[dev] = (uint8_t*)p;
  }
  return ptrs[dev];
}

hipError_t launch_sample_noalloc(const void* logits, int V, int64_t ld, int rows, int k,
                                 float temperature, float top_p, const float* u, int32_t* out,
                                 hipStream_t s) {
  hipError_t err;
  uint8_t* base = scratch_ptr(&err);
  if (!base) return err;
  float* cv = (float*)base;
  int* ci = (int*)(base + SCRATCH_CAND * 4);
  int* bad = (int*)(base + 2 * SCRATCH_CAND * 4);
  int* flag = (int*)(base + SCRATCH_BYTES - 256);
  // every candidate and mark is written before it is read; the flag word is
  // only ever raised, so it is cleared on each call (a fill kernel, not a
  // memset, so the call may sit in a captured graph)
  launch_fill_zero(flag, 1, s);
  launch_sample(logits, V, ld, rows, k, temperature, top_p, u, cv, ci, bad, out, flag, s);
  return hipGetLastError();
}

void launch_sample(const void* logits, int V, int64_t ld, int rows, int k, float temperature,
                   float top_p, const float* u, float* cv, int* ci, int* bad, int32_t* out,
                   int* flag, hipStream_t s) {
  const int nchunk = sample_chunks(V);
  hipLaunchKernelGGL(sample_partial_kernel, dim3(nchunk, rows), dim3(256), 0, s,
                     (const bf16_t*)logits, V, ld, k, cv, ci, bad, nchunk);
  hipLaunchKernelGGL(sample_final_kernel, dim3(rows), dim3(256), 0, s, cv, ci, bad, nchunk, k,
                     temperature, top_p, u, out, flag);
}
