/* Plain CPU oracle of the dense grouped-query Llama forward step.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library; the HIP path
 * shares no code with it and never calls it.
 *
 * Data: bf16 values are passed as their uint16 bit patterns.  Activations are
 * row-major [rows][width]; projection weights are [out][in] row-major; caches
 * are position-major [T][n_kv_heads][head_dim] for one layer execution.
 *
 * Arithmetic: binary64 between rounding points, round-to-nearest-even to bf16
 * at exactly the points of Hugging Face modeling_llama in bf16, as listed in
 * the pull request "llama: Nanbeige4.3-33B on Metal, the bf16 release served
 * as published", section "How":
 *   residual adds rounded; RMSNorm bf16(w * bf16(x * rsqrt(mean(x^2)+eps)));
 *   RoPE bf16(bf16(x c) + bf16(rot(x) s)) with bf16 cos/sin of the fp32 angle;
 *   SwiGLU bf16(bf16(silu(g)) * u); row projections summed wide, rounded once.
 * Each operation is exact (binary64) before its rounding point, as in the
 * float64 "--bf16-points" reference described in the same pull request's
 * review thread.
 */
#ifndef LLAMA_ORACLE_H
#define LLAMA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int64_t hidden, n_q_heads, n_kv_heads, head_dim, ffn;
  double rope_theta;
  float rms_eps;
} orc_geom;

typedef struct {
  const uint16_t *attn_norm, *q, *k, *v, *o, *mlp_norm, *gate, *up, *down;
} orc_block_weights;

/* bf16 <-> binary64. */
uint16_t orc_bf16(double x);
double orc_f64(uint16_t b);
void orc_bf16_array(const double* x, int64_t n, uint16_t* out);

/* Planted mistakes, for tests that must see a self-check fail. 0 = none,
 * 1 = RoPE inverse frequencies left at zero (the non-persistent inv_freq
 * pitfall named on the Nanbeige4.2-3B card, section "Verification"). */
void orc_plant(int code);

void orc_embed(const uint16_t* E, int64_t vocab, int64_t H, const int32_t* tok, int64_t rows,
               uint16_t* out);
void orc_rmsnorm(const uint16_t* h, const uint16_t* w, int64_t rows, int64_t H, float eps,
                 uint16_t* out);
void orc_linear(const uint16_t* x, const uint16_t* W, int64_t rows, int64_t N, int64_t K,
                uint16_t* y, double* y64);
void orc_rope_inv_freq(int64_t d, double theta, float* inv);
void orc_rope(uint16_t* x, const int32_t* pos, int64_t rows, int64_t heads, int64_t d,
              double theta);
void orc_attention(const uint16_t* q, const uint16_t* kc, const uint16_t* vc, const int32_t* pos,
                   int64_t rows, int64_t nq, int64_t nkv, int64_t d, uint16_t* out,
                   double* out64);
void orc_swiglu(const uint16_t* g, const uint16_t* u, int64_t n, uint16_t* out);
void orc_residual_add(uint16_t* h, const uint16_t* y, int64_t n);
int32_t orc_argmax(const uint16_t* logits, int64_t V);
/* Seeded top-k / top-p sampling of one row against the uniform u (definition
 * at the function); *margin (nullable) is the decisions' relative margin. */
int32_t orc_sample(const uint16_t* logits, int64_t V, double temperature, int32_t top_k,
                   double top_p, double u, double* margin);

/* One block execution over `rows` rows at absolute positions pos[]: keys and
 * values of every row are stored at their slots first, then each row attends
 * causally to [0, pos[r]].  h is updated in place; h_mid (nullable) receives
 * the residual after the attention half. Returns 0, or -1 if a position is
 * outside [0, cache_positions). */
int orc_block(const orc_geom* g, const orc_block_weights* w, uint16_t* kc, uint16_t* vc,
              int64_t cache_positions, const int32_t* pos, int64_t rows, uint16_t* h,
              uint16_t* h_mid);

#ifdef __cplusplus
}
#endif
#endif
