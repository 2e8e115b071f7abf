// Host-side launchers of the gfx950 kernels (defined in the k_*.hip files and
// called by the C-ABI layer in llama_abi.cpp).
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

// Kernel timing for benchmarks: while a timer is set on the calling thread,
// each kernel launched through launch_k records the start and the end of its
// own execution in the timer's next event pair (hipExtLaunchKernel), so the
// pair spans the kernel alone, not the dispatch around it; once the pool is
// used up, launches are not recorded.  The timer pointer is `__thread`, not
// `thread_local`: a hidden thread_local used across files makes the compiler
// test a thread-local init function by its address, and in a shared object an
// undefined one reads as the load base rather than zero.
struct LaunchTimer {
  hipEvent_t* ev;
  size_t cap;
  size_t* used;
};
extern __thread LaunchTimer* launch_timer __attribute__((visibility("hidden")));
template <typename F, typename... A>
inline void launch_k(F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t s, A... args) {
  LaunchTimer* t = launch_timer;
  if (t && *t->used + 2 <= t->cap) {
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, t->ev[*t->used], t->ev[*t->used + 1], 0,
                          args...);
    *t->used += 2;
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
  }
}

#define LLAMA_MAX_SEQS 16

// Where each row of a step lives: row rt belongs to sequence rt / rows_per_seq
// at position pos0[seq] + rt % rows_per_seq; k / v are that sequence's key and
// value slabs for the execution being run ([max_positions][n_kv_heads][d]).
struct RowTable {
  uint16_t* k[LLAMA_MAX_SEQS];
  uint16_t* v[LLAMA_MAX_SEQS];
  int pos0[LLAMA_MAX_SEQS];
  int rows_per_seq;
};

void launch_fill_zero(int* p, int n, hipStream_t s);
void launch_embed(const void* E, int vocab, int H, const int32_t* tok, void* h, int rows,
                  hipStream_t s);
void launch_rmsnorm(const void* h, const void* w, void* out, int rows, int H, float eps,
                    hipStream_t s);
// (cos, sin) of every row's position, [rows][d/2] float2 of bf16 values,
// computed once per pass and read by every execution.
void launch_rope_table(const RowTable& tab, int rows, int d, float theta, void* table,
                       hipStream_t s);
void launch_rope_kv(const void* qkv, void* qout, const RowTable& tab, int rows, int nq, int nkv,
                    int d, const void* table, hipStream_t s);
int argmax_chunks(int V);
// Seeded top-k / top-p sampling of bf16 logit rows (k <= 64); cv / ci / bad
// hold rows * sample_chunks(V) * k candidates and rows * sample_chunks(V)
// flags.
int sample_chunks(int V);
void launch_sample(const void* logits, int V, int64_t ld, int rows, int k, float temperature,
                   float top_p, const float* u, float* cv, int* ci, int* bad, int32_t* out,
                   int* flag, hipStream_t s);
// The same draw with its candidates in a fixed per-device scratch array
// instead of a workspace (no allocation, no workspace): rows <=
// SAMPLE_NOALLOC_MAX_ROWS, sample_chunks(V) * k <= SAMPLE_NOALLOC_MAX_CAND,
// sample_chunks(V) <= SAMPLE_NOALLOC_MAX_CHUNKS (checked by the caller).
#define SAMPLE_NOALLOC_MAX_ROWS 64
#define SAMPLE_NOALLOC_MAX_CAND 4096
#define SAMPLE_NOALLOC_MAX_CHUNKS 256
size_t sample_noalloc_scratch_bytes();
hipError_t launch_sample_noalloc(const void* logits, int V, int64_t ld, int rows, int k,
                                 float temperature, float top_p, const float* u, int32_t* out,
                                 hipStream_t s);
void launch_argmax(const void* logits, int V, int ld, int rows, float* pv, int* pi, int32_t* out,
                   int* flag, hipStream_t s);
// Acceptance of a drafted round: win[0..k] window inputs, t[0..k] the
// target's greedy tokens; out[0..a] the round's tokens, *count = a.
void launch_draft_accept(const int32_t* win, const int32_t* t, int k, int32_t* out,
                         int32_t* count, hipStream_t s);

// Decode projections (1..16 rows).  Output columns [0, N) are the
// concatenation of up to three weight matrices (segments), each [rows][K].
enum GemvEpilogue { GEMV_STORE = 0, GEMV_RESIDUAL = 1, GEMV_SWIGLU = 2, GEMV_QKV_ROPE = 3 };
struct GemvSeg {
  const uint16_t* W;
  int n_begin, n_end;
};
// STORE:    out[r*ldo + n] = bf16(acc); out32 (nullable) gets the fp32 sum.
// RESIDUAL: out[r*ldo + n] = bf16(out + bf16(acc))  (the residual stream).
// SWIGLU:   seg[0] = gate, seg[1] = up, both with n in [0, F):
//           out[r*ldo + n] = bf16(bf16(silu(bf16(g))) * bf16(u)).
// normw (nullable): the input rows are raw residuals to be normalised with
// this RMSNorm weight -- done inside the projection when rows <=
// GEMV_NORM_ROWS; callers normalise larger windows first and pass NULL.
#define GEMV_NORM_ROWS 4
void launch_gemv(int epi, const GemvSeg* seg, int nseg, int N, int K, const void* x, int ldx,
                 int rows, void* out, int ldo, float* out32, int ld32, const void* normw,
                 float eps, hipStream_t s);
// q/k/v decode projection with RoPE and the cache write fused (seg = q, k, v
// weights); rows are rows row0.. of the pass tab describes; q goes to qout.
void launch_gemv_qkv_rope(const GemvSeg* seg, int K, const void* x, int ldx, int rows, int row0,
                          void* qout, const RowTable& tab, const void* rope, int nq, int nkv,
                          int d, const void* normw, float eps, hipStream_t s);

// Prompt-chunk projections on the matrix cores; ncols tile columns (N, or
// 2F for SWIGLU, whose tiles interleave 32 gate and 32 up rows).
// exact: the projections' running sums restart every 128 terms (slower).
void launch_gemm(int epi, const void* A, int lda, int M, int K, const GemvSeg* seg, int nseg,
                 const void* gate, const void* up, void* out, int ldo, float* out32, int ld32,
                 int ncols, bool exact, hipStream_t s);
// Prompt-chunk attention: rows at positions [pos0, pos0 + rows) against the
// cache slabs kc / vc of one sequence; out32 (nullable) also receives the
// output before its rounding.
// exact: three-part weights, per-tile sums (slower).
void launch_attn_prefill(const void* q, const void* kc, const void* vc, int rows, int pos0, int nq,
                         int nkv, int d, void* out, float* out32, bool exact, hipStream_t s);

// Decode attention: split over key blocks at absolute positions, then
// merged in block order; out32 (nullable) as for prompt chunks.
int attn_max_blocks();
void launch_attn_decode(const void* q, const RowTable& tab, int rows, int nq, int nkv, int d,
                        float* part, void* out, float* out32, hipStream_t s);
