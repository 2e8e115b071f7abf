/* llama_mi355x.h -- C ABI of the MI355X (gfx950) forward step of a dense
 * grouped-query Llama decoder served from bf16 weights with a bf16
 * position-major key/value cache.
 *
 * The step is Hugging Face modeling_llama in bf16 at its rounding points, as
 * the pull request "llama: Nanbeige4.3-33B on Metal, the bf16 release served
 * as published" states them (section "How"): each residual add rounded to
 * bf16; RMSNorm bf16(w * bf16(x * rsqrt(mean(x^2) + eps))); RoPE
 * bf16(bf16(x c) + bf16(rot(x) s)) with bf16 cos and sin of the fp32 angle;
 * SwiGLU bf16(bf16(silu(g)) * u); row projections with fp32 sums rounded
 * once.  Attention scores, softmax and the weighted sum of values are fp32
 * and the attention output is rounded once.  Greedy tokens are drawn on the
 * GPU, ties to the lower id (review reply "Teacher-forced misses").
 *
 * Memory.  Every pointer named *_dev, every weight and the workspace and
 * cache buffers are device addresses owned by the caller; the library only
 * borrows them and they must outlive the handles that hold them.  Handles are
 * host objects freed by llama_free / llama_kv_free.  No call allocates device
 * memory.
 *
 * Layouts.  bf16 values are 16-bit patterns.  Projection weights are
 * [out][in] row-major, as published: q [n_q_heads*head_dim][hidden],
 * k and v [n_kv_heads*head_dim][hidden], o [hidden][n_q_heads*head_dim],
 * gate and up [ffn][hidden], down [hidden][ffn], embed and lm_head
 * [vocab][hidden]; norm weights [hidden].  Activations are [row][width].
 * The cache of one sequence holds, for every execution e (block b of loop l
 * is e = l*n_blocks + b), keys then values, each [max_positions][n_kv_heads]
 * [head_dim] with position p at slot p (keys after RoPE).
 *
 * Asynchrony and errors.  Every call validates its arguments on the host
 * before it enqueues anything on `hip_stream` (a hipStream_t; NULL is the
 * default stream) and returns without blocking.  On a refusal it returns a
 * negative LLAMA_E_* code, changes no state, and llama_last_error() (per
 * thread) names the reason.  A launch failure reports LLAMA_E_DEVICE.
 * Cache lengths advance on the host when a step is enqueued.
 */
#ifndef LLAMA_MI355X_H
#define LLAMA_MI355X_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  LLAMA_OK = 0,
  LLAMA_E_ARG = -1,        /* NULL or inconsistent argument */
  LLAMA_E_GEOMETRY = -2,   /* geometry the kernels do not serve (refused at load) */
  LLAMA_E_CAPACITY = -3,   /* a position would reach past the cache */
  LLAMA_E_POSITION = -4,   /* pos0 differs from the cache length */
  LLAMA_E_DEVICE = -5,     /* a HIP call or launch failed */
  LLAMA_E_NONFINITE = -6,  /* a logit row held NaN or +-Inf */
  LLAMA_E_WORKSPACE = -7   /* workspace or buffer smaller than required */
};

/* Geometry.  Served set (others are refused with LLAMA_E_GEOMETRY):
 * head_dim 64 or 128; hidden, ffn, n_q_heads*head_dim, n_kv_heads*head_dim
 * and vocab multiples of 128; n_q_heads a multiple of n_kv_heads with at
 * most 8 query heads per KV head; rope_theta > 0; vocab 0 means a model of
 * blocks only (no embedding, final norm or lm_head: rows enter and leave as
 * hidden states).  The final norm, when present, is applied at the end of
 * every loop (the looped architecture of the Nanbeige4.2-3B card, section
 * "About the architecture"). */
typedef struct {
  int32_t n_blocks;        /* blocks with their own weights */
  int32_t n_loops;         /* passes over the block stack per step (>= 1) */
  int32_t hidden;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t ffn;
  int32_t vocab;           /* 0: blocks only */
  double rope_theta;       /* unscaled RoPE base */
  float rms_eps;
  int32_t max_chunk_rows;  /* largest llama_prefill_chunk, 1..2048 */
  int32_t max_window_rows; /* largest llama_decode_step window, 1..16 */
  int32_t max_seqs;        /* largest n_seq of llama_decode_step, 1..16 */
  /* Prompt chunks' arithmetic (decode windows are unaffected): 0, the fast
   * form, keeps each projection's fp32 sum in one matrix-unit chain over K
   * and the attention weights in two bf16 parts (16 significant bits);
   * 1, the exact form, restarts the projection sums every 128 terms into
   * fp32 totals and keeps the weights in three bf16 parts (24 bits), at
   * about 2x the projection time and 1.4x the attention time.  Both are fp32
   * sums rounded once, as the spec asks; the exact form's per-element error
   * is close to the decode kernels'. */
  int32_t prompt_exact;
} llama_config;

/* Device addresses of one block's bf16 weights. */
typedef struct {
  const void *attn_norm, *q, *k, *v, *o, *mlp_norm, *gate, *up, *down;
} llama_block_weights;

typedef struct llama_model llama_model; /* opaque */
typedef struct llama_kv llama_kv;       /* opaque: one sequence, every execution */

/* Bytes of device workspace a model needs for caches of up to
 * `max_positions` positions; 0 if the configuration is refused (reason in
 * llama_last_error).  Memory is sized up front from the positions the caller
 * budgets, as the pull request "llama: Nanbeige4.3-33B on Metal, the bf16
 * release served as published" sizes its caches from a context budget
 * (section "How").  The workspace holds the residual, normed rows, q/k/v,
 * attention output and SwiGLU rows of the largest pass (max(max_chunk_rows,
 * max_seqs * max_window_rows) rows), decode attention partials, the per-pass
 * RoPE table, logits scratch, argmax and sampling partials and the
 * non-finite flag.  Host-only. */
size_t llama_workspace_bytes(const llama_config* cfg, int32_t max_positions);

/* Checks the geometry and records the weight and workspace addresses.
 * blocks[n_blocks]; embed, final_norm and lm_head must be NULL when vocab is
 * 0 and non-NULL otherwise; a tied head (lm_head == embed) is refused, as on
 * the pull request's "Checks" list.  Host-only: nothing is enqueued; the
 * first step on the model initialises the workspace on its own stream.
 * workspace_bytes must be at least llama_workspace_bytes(cfg, max_positions),
 * and caches of this model may hold at most max_positions positions. */
int llama_load_weights(const llama_config* cfg, const llama_block_weights* blocks,
                       const void* embed, const void* final_norm, const void* lm_head,
                       void* workspace_dev, size_t workspace_bytes, int32_t max_positions,
                       llama_model** out);

/* Cache bytes for one sequence of up to max_positions positions:
 * executions * max_positions * n_kv_heads * head_dim * 2 (K, V) * 2 bytes --
 * 16-bit keys and values, 208 KiB per position for the 33B shape (the card
 * "Nanbeige4.3-33B EXL3", section "Which rung should I use?", prices the
 * model's 16-bit cache at that).  Host-only; 0 for a NULL model or a
 * non-positive count. */
size_t llama_kv_bytes(const llama_model* model, int32_t max_positions);

/* Wraps a caller-owned device buffer of at least llama_kv_bytes() bytes as an
 * empty cache (length 0) of one sequence: the cache a budget of
 * max_positions positions buys (pull request section "How": caches sized from
 * the context budget).  The buffer stays owned by the caller and must outlive
 * the handle.  Refusals: LLAMA_E_ARG (NULL model, buffer or out),
 * LLAMA_E_CAPACITY (max_positions outside 1..the model's max_positions),
 * LLAMA_E_WORKSPACE (bytes below llama_kv_bytes).  Host-only: nothing is
 * enqueued and the buffer is not touched (its contents are never read before
 * they are written). */
int llama_kv_alloc(llama_model* model, int32_t max_positions, void* device_buf, size_t bytes,
                   llama_kv** out);

int32_t llama_kv_length(const llama_kv* kv);

/* Resumes from a kept prompt state (pull request "llama: Nanbeige4.3-33B on
 * Metal, the bf16 release served as published", section "Measured": a
 * resumed turn keeps the cached prefix and prefills only the rest): the
 * cache keeps positions [0, n_positions) and the next prompt chunk starts at
 * n_positions.  Shortens only: 0 <= n_positions <= llama_kv_length(kv), else
 * LLAMA_E_POSITION and nothing changes.  Host-only, no device work. */
int llama_kv_truncate(llama_kv* kv, int32_t n_positions);

/* Test hook, not for serving: declares that positions [0, n_positions) of
 * every execution hold keys and values the caller wrote itself through
 * llama_kv_slab (synthetic caches for parity tests and benchmarks).  The
 * library cannot check what the buffer holds; steps then read those slots
 * as written.  n_positions 0..max_positions of the cache, else
 * LLAMA_E_CAPACITY. */
int llama_test_kv_declare(llama_kv* kv, int32_t n_positions);

/* Device address of execution e's keys (which = 0) or values (which = 1). */
void* llama_kv_slab(const llama_kv* kv, int32_t exec, int32_t which);

/* One prompt chunk of n_rows (1..max_chunk_rows) rows of one sequence at
 * positions [pos0, pos0 + n_rows); pos0 must equal the cache length.  Rows
 * come from exactly one of tokens_dev (int32 [n_rows], through the
 * embedding) and hidden_in_dev (bf16 [n_rows][hidden], entering the first
 * execution as they are); a blocks-only model takes hidden rows.  Outputs,
 * each optional (NULL): hidden_out_dev bf16 [n_rows][hidden], the residual
 * after the last execution, before the final norm; logits_bf16_dev and
 * logits_f32_dev ([n_rows or 1][vocab]: every row when all_rows != 0, else
 * the last) with the fp32 sums before their rounding; next_token_dev (int32
 * [n_rows or 1]) the greedy id of each logit row, -1 for a row holding NaN
 * or +-Inf.  Prompt chunks of up to 2,048 rows follow the pull request's
 * section "How". */
int llama_prefill_chunk(llama_model* model, llama_kv* kv, const int32_t* tokens_dev,
                        const void* hidden_in_dev, int32_t n_rows, int32_t pos0,
                        void* hidden_out_dev, void* logits_bf16_dev, float* logits_f32_dev,
                        int32_t all_rows, int32_t* next_token_dev, void* hip_stream);

/* One decode window of `rows` (1..max_window_rows) rows for each of n_seq
 * sequences (1..max_seqs, distinct caches), all batched into one pass: the
 * rows of sequence s sit at positions [len_s, len_s + rows).  Rows come
 * from exactly one of tokens_dev (int32 [n_seq][rows]) and hidden_in_dev
 * (bf16 [n_seq][rows][hidden]); hidden_out_dev, logits_bf16_dev, logits_f32_dev and
 * next_tokens_dev are laid out [n_seq][rows][...], each optional.  Every row
 * is computed exactly as a one-row step at its position would compute it, so
 * windows equal one-row steps and batched sequences equal solo runs bit for
 * bit (pull request, section "Measured"). */
int llama_decode_step(llama_model* model, llama_kv* const* kvs, int32_t n_seq,
                      const int32_t* tokens_dev, const void* hidden_in_dev, int32_t rows,
                      void* hidden_out_dev, void* logits_bf16_dev, float* logits_f32_dev,
                      int32_t* next_tokens_dev, void* hip_stream);

/* Test hook: while set, every step also writes each execution's residuals to
 * buf_dev as bf16 [executions][2][rows][hidden] ([0] after the attention
 * half, [1] after the MLP half; rows = the step's total rows).  NULL clears
 * it.  A later step whose capture would not fit is refused. */
int llama_set_capture(llama_model* model, void* buf_dev, size_t bytes);

/* Test hook for parity of single kernels.  While set, every step also writes
 * the intermediate values of one execution `exec` into the caller's device
 * buffers below (each nullable; rows = the step's total rows, at most
 * max_rows, else the step is refused with LLAMA_E_WORKSPACE):
 *   h_in      bf16 [rows][hidden]         residual entering the execution
 *                                         (after a loop boundary: the
 *                                         final-normed state)
 *   x_attn    bf16 [rows][hidden]         RMSNorm output feeding q/k/v
 *   qkv32     fp32 [rows][nq*d + 2*nkv*d] q, k, v sums before rounding
 *   q_rope    bf16 [rows][nq*d]           q after RoPE
 *   attn      bf16 [rows][nq*d]           attention output
 *   attn32    fp32 [rows][nq*d]           attention output before rounding
 *   o32       fp32 [rows][hidden]         o projection sums
 *   x_mlp     bf16 [rows][hidden]         RMSNorm output feeding gate/up
 *   gate_up32 fp32 [rows][2*ffn]          gate sums, then up sums
 *   act       bf16 [rows][ffn]            SwiGLU output
 *   down32    fp32 [rows][hidden]         down projection sums
 * Sums that a fused launch keeps in registers come from an extra launch of
 * the same projection kernel with a storing epilogue (every output's
 * summation order is the same whichever epilogue runs), so the probe reports
 * what the fused step rounds.  NULL clears the hook.  Steps are slower while
 * it is set; their results are unchanged. */
typedef struct {
  void* h_in;
  void* x_attn;
  float* qkv32;
  void* q_rope;
  void* attn;
  float* attn32;
  float* o32;
  void* x_mlp;
  float* gate_up32;
  void* act;
  float* down32;
} llama_probe;
int llama_set_probe(llama_model* model, int32_t exec, const llama_probe* probe, int32_t max_rows);

/* Test hooks for parity of single kernels on caller-given operands (the
 * oracle's inputs), outside any step.  prompt_kernel selects the kernel a
 * decode window runs (0), the one a prompt chunk runs in the fast form (1) or
 * in the exact form (2; see llama_config.prompt_exact).
 *
 * llama_test_linear: y[r][j] = sum_k w[j][k] x[r][k] for rows r < rows
 * (bf16 x [rows][k], bf16 w [n][k]) with the step's projection kernel and a
 * storing epilogue: y_dev bf16 [rows][n] (the sums rounded once) and y32_dev
 * fp32 [rows][n] (the sums).  n and k multiples of 128; rows 1..2048 for the
 * prompt kernel, 1..16 for the decode kernel.  Row projections with fp32
 * sums rounded once: pull request "llama: Nanbeige4.3-33B on Metal, the bf16
 * release served as published", section "How".
 *
 * llama_test_attention: causal grouped-query attention of rows q_dev (bf16
 * [rows][n_q_heads][head_dim], after RoPE) at positions [pos0, pos0 + rows)
 * against execution `exec` of cache kv, which must hold positions
 * [0, pos0 + rows); out_dev bf16 [rows][n_q_heads][head_dim] and out32_dev
 * (nullable) the output before rounding.  rows 1..max_chunk_rows for the
 * prompt kernel, 1..max_seqs * max_window_rows for the decode kernel (its
 * partial sums use the model's workspace, so calls on one model are
 * serialised by their stream).  Asynchronous on hip_stream; refusals return
 * LLAMA_E_ARG or LLAMA_E_POSITION before anything is enqueued. */
int llama_test_linear(llama_model* model, int32_t prompt_kernel, const void* x_dev, int32_t rows,
                      const void* w_dev, int32_t n, int32_t k, void* y_dev, float* y32_dev,
                      void* hip_stream);
int llama_test_attention(llama_model* model, int32_t prompt_kernel, llama_kv* kv, int32_t exec,
                         const void* q_dev, int32_t rows, int32_t pos0, void* out_dev,
                         float* out32_dev, void* hip_stream);

/* Measurement hook for benchmarks.  While `kernel` is one of the classes
 * below, every kernel of that class that a step launches records the start
 * and the end of its own execution in a HIP event pair (hipExtLaunchKernel,
 * on the step's stream), from a pool of max_launches pairs created by this
 * call (host-side event objects; no device memory).  A class may launch more
 * than one kernel per block (decode attention: the split pass and the merge;
 * prompt q/k/v: up to two launches; prompt gate/up and down are one class).
 * Launches beyond the pool are not recorded.  kernel = LLAMA_TIMING_OFF
 * releases the pool.  llama_timing_read synchronises on the recorded events
 * and returns the summed milliseconds of the recorded kernels and their
 * number since the previous read.  While the hook is on, one host thread
 * drives the model (the pool's cursor is not shared safely between threads). */
enum {
  LLAMA_TIMING_OFF = 0,
  LLAMA_TIMING_GATE_UP = 1,   /* decode gate/up projection with SwiGLU */
  LLAMA_TIMING_DOWN = 2,      /* decode down projection + residual */
  LLAMA_TIMING_QKV = 3,       /* decode q/k/v projection */
  LLAMA_TIMING_O = 4,         /* decode o projection + residual */
  LLAMA_TIMING_LM_HEAD = 5,   /* decode lm_head projection */
  LLAMA_TIMING_ATTN = 6,      /* decode attention, both passes */
  LLAMA_TIMING_PREFILL_GEMM = 7, /* every prompt-chunk projection */
  LLAMA_TIMING_PREFILL_ATTN = 8  /* prompt-chunk attention */
};
int llama_set_timing(llama_model* model, int32_t kernel, int32_t max_launches);
int llama_timing_read(llama_model* model, double* total_ms, int64_t* launches);

/* Seeded sampling (issue "A llama family on Metal", the served sampling
 * checks; pull request, section "How": tokens drawn on the GPU; model card
 * "Nanbeige4.3-33B EXL3": upstream's recommended temperature 0.6, top_p 0.95,
 * top_k 20).  For each of `rows` rows of bf16 logits (row r at
 * logits_bf16_dev + r * ld elements, `vocab` entries, e.g. the logits a step
 * call wrote) it draws one token into tokens_dev[r] (int32, device):
 *   z = logit / temperature; keep the top_k largest (ties to the lower id),
 *   ordered largest first; weights e_i = exp(z_i - z_0); candidate i stays
 *   while the weight of those before it is below top_p times the total (the
 *   first always stays); the token is the first remaining candidate whose
 *   running weight exceeds u_dev[r] times the remaining weight.
 * u_dev holds one uniform in [0, 1) per row (float, device), drawn by the
 * caller from its seed, so equal seeds give equal tokens.  Weights and draw
 * are fp32.  rows 1..LLAMA_SAMPLE_MAX_ROWS; temperature > 0 and finite (a
 * greedy draw is the step calls' next_tokens); top_k 1..LLAMA_SAMPLE_MAX_TOP_K
 * (and at most vocab); 0 < top_p <= 1.  A row holding NaN or +-Inf yields -1
 * and raises the non-finite flag (llama_check_finite).  Refusals return
 * LLAMA_E_ARG before anything is enqueued.  Asynchronous on hip_stream; uses
 * the model's workspace, so calls on one model are serialised by its
 * stream. */
#define LLAMA_SAMPLE_MAX_ROWS 64
#define LLAMA_SAMPLE_MAX_TOP_K 64
int llama_sample(llama_model* model, const void* logits_bf16_dev, int32_t rows, int64_t ld,
                 float temperature, int32_t top_k, float top_p, const float* u_dev,
                 int32_t* tokens_dev, void* hip_stream);

/* Seeded sampling that allocates nothing, for callers that cannot allocate
 * device memory or keep a workspace (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): llama_sample's draw (same
 * rule, same bits) on rows of bf16 logits with `vocab` entries, with no model
 * handle.  Its candidates live in a fixed scratch array of about 2.1 MiB
 * (LLAMA_SAMPLE_NOALLOC_SCRATCH_BYTES) that the library keeps on every GPU it
 * runs on until the process ends; the first call on a device looks up that
 * device's copy.  Limits: rows 1..LLAMA_SAMPLE_MAX_ROWS, vocab
 * 1..LLAMA_SAMPLE_NOALLOC_MAX_VOCAB, top_k 1..LLAMA_SAMPLE_MAX_TOP_K (and at
 * most vocab) with ceil(vocab / 4096) * top_k <= 4096; temperature, top_p, u
 * and ld as llama_sample.  A row holding NaN or +-Inf yields -1 (there is no
 * model flag to raise).  Every call on one GPU shares that GPU's scratch and
 * it keeps the last call's contents: calls that overlap on one GPU (other
 * streams or threads) race and must be serialised by the caller; calls on one
 * stream are ordered.  Refusals return LLAMA_E_ARG before anything is
 * enqueued; a failed scratch lookup returns LLAMA_E_DEVICE. */
#define LLAMA_SAMPLE_NOALLOC_MAX_VOCAB 1048576
#define LLAMA_SAMPLE_NOALLOC_SCRATCH_BYTES (2u * 64u * 4096u * 4u + 64u * 256u * 4u + 256u)
int llama_sample_noalloc(const void* logits_bf16_dev, int32_t vocab, int32_t rows, int64_t ld,
                         float temperature, int32_t top_k, float top_p, const float* u_dev,
                         int32_t* tokens_dev, void* hip_stream);

/* One round of drafted greedy decoding (issue "A llama family on Metal:
 * Nanbeige4.3-33B served from its bf16 release", follow-ups: a smaller Llama
 * on the same tokenizer drafting for the served model with replies
 * unchanged; pull request "llama: Nanbeige4.3-33B on Metal, the bf16 release
 * served as published", reply "Drafting": drafted greedy equals plain
 * greedy).  Both caches hold the same p positions (the tokens before
 * last_token_dev[0], the next input, int32 on the device).  The draft model
 * proposes d_1 .. d_n by n_draft greedy one-row steps from that token; the
 * target reads [last, d_1 .. d_n] as one window at positions p .. p + n and
 * draws its greedy token after each; the round yields the a leading
 * proposals the target agrees with, then the target's own token after them:
 * tokens_out_dev[0 .. a] (int32, device, room for n_draft + 1), *n_out = a + 1
 * (host).  Windows equal one-row steps bit for bit, so the reply equals the
 * target's plain greedy steps whatever the draft proposes.  Afterwards both
 * caches hold p + a + 1 positions (last, d_1 .. d_a) and the next round's
 * input is tokens_out_dev[a].  n_draft 1..(target max_window_rows - 1); both
 * models have the same vocabulary; both caches need room for p + n_draft + 1
 * positions.  Refusals (LLAMA_E_ARG, LLAMA_E_POSITION, LLAMA_E_CAPACITY)
 * change nothing.  Unlike the other step calls it synchronises hip_stream
 * once, to read a; both models' work runs on that stream and the target's
 * workspace holds the round's token buffers.  A non-finite logit row shows
 * as a -1 token and in llama_check_finite of the model that met it. */
int llama_draft_round(llama_model* target, llama_kv* target_kv, llama_model* draft,
                      llama_kv* draft_kv, int32_t n_draft, const int32_t* last_token_dev,
                      int32_t* tokens_out_dev, int32_t* n_out, void* hip_stream);

/* The same round with seeded sampling (model card "Nanbeige4.3-33B EXL3",
 * section on its draft model: the target samples and accepts matching draft
 * tokens, so the output follows the target's own sampling).  The draft still
 * proposes its greedy tokens; the target draws its token after each window
 * row i with llama_sample's rule (temperature, top_k, top_p) against u_dev[i]
 * (n_draft + 1 floats in [0, 1), device), and the round keeps the leading
 * proposals equal to those draws, then the target's own draw after them.
 * With u_dev[i] the uniform of position p + i, the reply equals seeded
 * sampling by plain steps with the same uniforms, whatever the draft
 * proposes.  Sampling arguments as llama_sample; the rest as
 * llama_draft_round. */
int llama_draft_round_sampled(llama_model* target, llama_kv* target_kv, llama_model* draft,
                              llama_kv* draft_kv, int32_t n_draft, const int32_t* last_token_dev,
                              float temperature, int32_t top_k, float top_p, const float* u_dev,
                              int32_t* tokens_out_dev, int32_t* n_out, void* hip_stream);

/* Synchronises hip_stream, then reports LLAMA_E_NONFINITE if any greedy or
 * sampled draw since the last call met a non-finite logit row (and clears
 * the flag), else LLAMA_OK.  A row holding NaN or +-Inf is refused rather than
 * given a token, as the pull request's teacher-forced checker refuses such
 * rows before it chooses or compares tokens (review reply "Non-finite
 * rows"); the draw itself yields -1 for that row.  LLAMA_E_DEVICE if the
 * flag cannot be read. */
int llama_check_finite(llama_model* model, void* hip_stream);

void llama_kv_free(llama_kv* kv);
void llama_free(llama_model* model);

/* Reason for the calling thread's last refusal ("" if none). */
const char* llama_last_error(void);

#ifdef __cplusplus
}
#endif
#endif
