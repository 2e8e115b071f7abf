/* Plain CPU oracle of the dense grouped-query Llama forward step.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h): loaded by the tests, the smoke
 * check and the benchmark's CPU-baseline leg, never by the HIP path.
 *
 * Everything here is the definition written out: binary64 arithmetic, one
 * round-to-nearest-even to bf16 at each rounding point of the pull request
 * "llama: Nanbeige4.3-33B on Metal, the bf16 release served as published",
 * section "How".  OpenMP only splits independent output elements across
 * threads; no sum is reassociated by it.  Build without -ffast-math and with
 * -ffp-contract=off so every binary64 operation rounds once.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static int g_plant = 0;
void orc_plant(int code) { g_plant = code; }

/* ---------------------------------------------------------------- bf16 --- */

/* Round to bf16 (8 significant bits, binary32 exponent range, subnormals down
 * to 2^-133, overflow to infinity), ties to even. */
uint16_t orc_bf16(double x) {
  if (isnan(x)) return 0x7FC0;
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (isinf(a)) return sign | 0x7F80;
  if (a == 0.0) return sign;
  int e;
  frexp(a, &e);            /* a = m * 2^e with 0.5 <= m < 1 */
  int q = e - 8;           /* weight of the 8th significant bit */
  if (q < -133) q = -133;  /* subnormal quantum */
  double r = nearbyint(ldexp(a, -q)); /* default rounding mode: nearest, ties to even */
  double v = ldexp(r, q);
  if (v > 0x1.FEp127) return sign | 0x7F80;
  float f = (float)v; /* exact: at most 8 significant bits */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(sign | ((u >> 16) & 0x7FFF));
}

double orc_f64(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return (double)f;
}

void orc_bf16_array(const double* x, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16(x[i]);
}

/* ----------------------------------------------------------- embedding --- */

void orc_embed(const uint16_t* E, int64_t vocab, int64_t H, const int32_t* tok, int64_t rows,
               uint16_t* out) {
  for (int64_t r = 0; r < rows; ++r) {
    int64_t t = tok[r];
    if (t < 0 || t >= vocab) { /* out-of-range ids give a NaN row, never a read */
      for (int64_t i = 0; i < H; ++i) out[r * H + i] = 0x7FC0;
      continue;
    }
    memcpy(out + r * H, E + t * H, (size_t)H * 2);
  }
}

/* ------------------------------------------------------------- RMSNorm --- */

/* bf16(w * bf16(x * rsqrt(mean(x^2) + eps))), the mean over the row.  eps is
 * the binary32 value the reference adds to its fp32 variance. */
void orc_rmsnorm(const uint16_t* h, const uint16_t* w, int64_t rows, int64_t H, float eps,
                 uint16_t* out) {
  for (int64_t r = 0; r < rows; ++r) {
    const uint16_t* x = h + r * H;
    double ss = 0.0;
    for (int64_t i = 0; i < H; ++i) {
      double v = orc_f64(x[i]);
      ss += v * v;
    }
    double inv = 1.0 / sqrt(ss / (double)H + (double)eps);
    for (int64_t i = 0; i < H; ++i) {
      double n = orc_f64(orc_bf16(orc_f64(x[i]) * inv));
      out[r * H + i] = orc_bf16(orc_f64(w[i]) * n);
    }
  }
}

/* ---------------------------------------------------------- projection --- */

/* y[r][n] = bf16(sum_k W[n][k] x[r][k]); bf16 products are exact in binary64
 * and the sum is binary64, rounded once.  y64 (nullable) keeps the sums. */
void orc_linear(const uint16_t* x, const uint16_t* W, int64_t rows, int64_t N, int64_t K,
                uint16_t* y, double* y64) {
  double* xd = (double*)malloc(sizeof(double) * (size_t)(rows * K));
  for (int64_t i = 0; i < rows * K; ++i) xd[i] = orc_f64(x[i]);
#pragma omp parallel
  {
    double* wd = (double*)malloc(sizeof(double) * (size_t)K);
#pragma omp for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
      for (int64_t k = 0; k < K; ++k) wd[k] = orc_f64(W[n * K + k]);
      for (int64_t r = 0; r < rows; ++r) {
        const double* xr = xd + r * K;
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) acc += wd[k] * xr[k];
        y[r * N + n] = orc_bf16(acc);
        if (y64) y64[r * N + n] = acc;
      }
    }
    free(wd);
  }
  free(xd);
}

/* ---------------------------------------------------------------- RoPE --- */

/* inv_i = fp32(1 / fp32(theta^(2i/d))) for i < d/2: the exponent 2i/d and the
 * power are binary32 values, the reciprocal a binary32 division. */
void orc_rope_inv_freq(int64_t d, double theta, float* inv) {
  float th = (float)theta;
  for (int64_t i = 0; i < d / 2; ++i) {
    float e = (float)(2 * i) / (float)d;
    float p = (float)pow((double)th, (double)e);
    inv[i] = 1.0f / p;
    if (g_plant == 1) inv[i] = 0.0f;
  }
}

/* Unscaled NeoX (half-head) rotary embedding, in place on x[rows][heads][d].
 * Element j uses frequency j mod d/2 and its partner across the half:
 * rot_j = -x_{j+d/2} for j < d/2, +x_{j-d/2} otherwise.  The angle is the
 * binary32 product p * inv_i; c and s are bf16 of the binary32 cos and sin. */
void orc_rope(uint16_t* x, const int32_t* pos, int64_t rows, int64_t heads, int64_t d,
              double theta) {
  int64_t half = d / 2;
  float* inv = (float*)malloc(sizeof(float) * (size_t)half);
  double* c = (double*)malloc(sizeof(double) * (size_t)half);
  double* s = (double*)malloc(sizeof(double) * (size_t)half);
  uint16_t* tmp = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)d);
  orc_rope_inv_freq(d, theta, inv);
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t i = 0; i < half; ++i) {
      float a = (float)((double)pos[r] * (double)inv[i]);
      c[i] = orc_f64(orc_bf16((double)(float)cos((double)a)));
      s[i] = orc_f64(orc_bf16((double)(float)sin((double)a)));
    }
    for (int64_t h = 0; h < heads; ++h) {
      uint16_t* v = x + (r * heads + h) * d;
      for (int64_t j = 0; j < d; ++j) {
        int64_t i = j % half;
        double xj = orc_f64(v[j]);
        double rot = j < half ? -orc_f64(v[j + half]) : orc_f64(v[j - half]);
        double a = orc_f64(orc_bf16(xj * c[i]));
        double b = orc_f64(orc_bf16(rot * s[i]));
        tmp[j] = orc_bf16(a + b);
      }
      memcpy(v, tmp, (size_t)d * 2);
    }
  }
  free(inv);
  free(c);
  free(s);
  free(tmp);
}

/* ----------------------------------------------------------- attention --- */

/* Causal grouped-query attention for rows at absolute positions pos[]:
 * query head h reads KV head h / (nq/nkv); scores (q . k_t)/sqrt(d) for
 * t <= pos[r]; softmax; output sum_t P_t v_t rounded to bf16 once. */
void orc_attention(const uint16_t* q, const uint16_t* kc, const uint16_t* vc, const int32_t* pos,
                   int64_t rows, int64_t nq, int64_t nkv, int64_t d, uint16_t* out,
                   double* out64) {
  int64_t group = nq / nkv;
  double scale = 1.0 / sqrt((double)d);
#pragma omp parallel for schedule(dynamic)
  for (int64_t rh = 0; rh < rows * nq; ++rh) {
    int64_t r = rh / nq, h = rh % nq, g = h / group;
    int64_t T = (int64_t)pos[r] + 1;
    const uint16_t* qv = q + (r * nq + h) * d;
    double* p = (double*)malloc(sizeof(double) * (size_t)T);
    double m = -INFINITY;
    for (int64_t t = 0; t < T; ++t) {
      const uint16_t* kv = kc + (t * nkv + g) * d;
      double dot = 0.0;
      for (int64_t j = 0; j < d; ++j) dot += orc_f64(qv[j]) * orc_f64(kv[j]);
      p[t] = dot * scale;
      if (p[t] > m) m = p[t];
    }
    double z = 0.0;
    for (int64_t t = 0; t < T; ++t) {
      p[t] = exp(p[t] - m);
      z += p[t];
    }
    for (int64_t t = 0; t < T; ++t) p[t] /= z;
    for (int64_t j = 0; j < d; ++j) {
      double o = 0.0;
      for (int64_t t = 0; t < T; ++t) o += p[t] * orc_f64(vc[(t * nkv + g) * d + j]);
      out[(r * nq + h) * d + j] = orc_bf16(o);
      if (out64) out64[(r * nq + h) * d + j] = o;
    }
    free(p);
  }
}

/* ---------------------------------------------------------- SwiGLU etc --- */

/* bf16(bf16(silu(g)) * u) with silu(g) = g / (1 + e^-g). */
void orc_swiglu(const uint16_t* g, const uint16_t* u, int64_t n, uint16_t* out) {
  for (int64_t i = 0; i < n; ++i) {
    double gv = orc_f64(g[i]);
    double sg = orc_f64(orc_bf16(gv / (1.0 + exp(-gv))));
    out[i] = orc_bf16(sg * orc_f64(u[i]));
  }
}

/* h = bf16(h + y), y already a bf16 projection output. */
void orc_residual_add(uint16_t* h, const uint16_t* y, int64_t n) {
  for (int64_t i = 0; i < n; ++i) h[i] = orc_bf16(orc_f64(h[i]) + orc_f64(y[i]));
}

/* Greedy choice over bf16 logits: the largest value, ties to the lowest id.
 * A row holding NaN or +-Inf anywhere is refused (-1). */
int32_t orc_argmax(const uint16_t* logits, int64_t V) {
  int32_t best = -1;
  double bv = 0.0;
  for (int64_t v = 0; v < V; ++v) {
    double x = orc_f64(logits[v]);
    if (!isfinite(x)) return -1;
    if (best < 0 || x > bv) {
      best = (int32_t)v;
      bv = x;
    }
  }
  return best;
}

/* Seeded sampling over bf16 logits (issue "A llama family on Metal", the
 * served sampling checks; pull request, section "How": tokens drawn on the
 * GPU; model card "Nanbeige4.3-33B EXL3", upstream's recommended temperature,
 * top_p and top_k).  Hugging Face's logits warpers in their default order --
 * temperature, top-k, top-p -- then one draw against the uniform u in [0, 1):
 *   1. z_v = logit_v / temperature;
 *   2. keep the top_k largest z, ordered by value (descending), then id;
 *   3. p_i = exp(z_i - z_0) / sum_j exp(z_j - z_0) over the kept;
 *   4. top-p: candidate i stays while the probability of the candidates
 *      before it is below top_p (the first always stays);
 *   5. the first remaining candidate whose cumulative probability, over the
 *      remaining ones renormalised, exceeds u.
 * A row holding NaN or +-Inf is refused (-1).  *margin (nullable) receives
 * the smallest distance, relative to the sum it is taken against, between a
 * decision threshold (the top-p cut, the draw target) and the cumulative sum
 * compared with it: a perturbation of the weights smaller than that cannot
 * change the token. */
int32_t orc_sample(const uint16_t* logits, int64_t V, double temperature, int32_t top_k,
                   double top_p, double u, double* margin) {
  if (top_k < 1 || V < 1 || !(temperature > 0.0)) return -1;
  int64_t k = top_k < V ? top_k : V;
  int32_t* id = (int32_t*)malloc(sizeof(int32_t) * (size_t)k);
  double* val = (double*)malloc(sizeof(double) * (size_t)k);
  double* e = (double*)malloc(sizeof(double) * (size_t)k);
  int64_t n_in = 0;
  int32_t tok = -1;
  for (int64_t v = 0; v < V; ++v) {
    double x = orc_f64(logits[v]);
    if (!isfinite(x)) goto done;
    /* insertion into the kept list (value descending, then id ascending) */
    if (n_in == k && !(x > val[k - 1])) continue;
    int64_t pos = n_in < k ? n_in : k - 1;
    while (pos > 0 && x > val[pos - 1]) {
      val[pos] = val[pos - 1];
      id[pos] = id[pos - 1];
      --pos;
    }
    val[pos] = x;
    id[pos] = (int32_t)v;
    if (n_in < k) ++n_in;
  }
  {
    double z0 = val[0] / temperature, S = 0.0;
    for (int64_t i = 0; i < k; ++i) {
      e[i] = exp(val[i] / temperature - z0);
      S += e[i];
    }
    int64_t n = 1;
    double cum = e[0];
    while (n < k && cum < top_p * S) cum += e[n++];
    double mp = HUGE_VAL;
    if (n > 1) mp = (top_p * S - (cum - e[n - 1])) / S;
    if (n < k) mp = fmin(mp, (cum - top_p * S) / S);
    double target = u * cum, c = 0.0, md = HUGE_VAL;
    int64_t i = 0;
    for (; i < n; ++i) {
      double prev = c;
      c += e[i];
      if (c > target) {
        md = (c - target) / cum;
        if (i > 0) md = fmin(md, (target - prev) / cum);
        break;
      }
    }
    if (i == n) i = n - 1;
    tok = id[i];
    if (margin) *margin = fmin(mp, md);
  }
done:
  free(id);
  free(val);
  free(e);
  return tok;
}

/* --------------------------------------------------------------- block --- */

int orc_block(const orc_geom* g, const orc_block_weights* w, uint16_t* kc, uint16_t* vc,
              int64_t cache_positions, const int32_t* pos, int64_t rows, uint16_t* h,
              uint16_t* h_mid) {
  int64_t H = g->hidden, d = g->head_dim, nq = g->n_q_heads, nkv = g->n_kv_heads, F = g->ffn;
  int64_t qd = nq * d, kvd = nkv * d;
  for (int64_t r = 0; r < rows; ++r)
    if (pos[r] < 0 || pos[r] >= cache_positions) return -1;

  uint16_t* x = (uint16_t*)malloc(2 * (size_t)(rows * H));
  uint16_t* q = (uint16_t*)malloc(2 * (size_t)(rows * qd));
  uint16_t* k = (uint16_t*)malloc(2 * (size_t)(rows * kvd));
  uint16_t* v = (uint16_t*)malloc(2 * (size_t)(rows * kvd));
  uint16_t* a = (uint16_t*)malloc(2 * (size_t)(rows * qd));
  uint16_t* y = (uint16_t*)malloc(2 * (size_t)(rows * H));
  uint16_t* gt = (uint16_t*)malloc(2 * (size_t)(rows * F));
  uint16_t* up = (uint16_t*)malloc(2 * (size_t)(rows * F));
  uint16_t* m = (uint16_t*)malloc(2 * (size_t)(rows * F));

  /* attention half */
  orc_rmsnorm(h, w->attn_norm, rows, H, g->rms_eps, x);
  orc_linear(x, w->q, rows, qd, H, q, NULL);
  orc_linear(x, w->k, rows, kvd, H, k, NULL);
  orc_linear(x, w->v, rows, kvd, H, v, NULL);
  orc_rope(q, pos, rows, nq, d, g->rope_theta);
  orc_rope(k, pos, rows, nkv, d, g->rope_theta);
  for (int64_t r = 0; r < rows; ++r) {
    memcpy(kc + (int64_t)pos[r] * kvd, k + r * kvd, (size_t)kvd * 2);
    memcpy(vc + (int64_t)pos[r] * kvd, v + r * kvd, (size_t)kvd * 2);
  }
  orc_attention(q, kc, vc, pos, rows, nq, nkv, d, a, NULL);
  orc_linear(a, w->o, rows, H, qd, y, NULL);
  orc_residual_add(h, y, rows * H);
  if (h_mid) memcpy(h_mid, h, 2 * (size_t)(rows * H));

  /* MLP half */
  orc_rmsnorm(h, w->mlp_norm, rows, H, g->rms_eps, x);
  orc_linear(x, w->gate, rows, F, H, gt, NULL);
  orc_linear(x, w->up, rows, F, H, up, NULL);
  orc_swiglu(gt, up, rows * F, m);
  orc_linear(m, w->down, rows, H, F, y, NULL);
  orc_residual_add(h, y, rows * H);

  free(x); free(q); free(k); free(v); free(a); free(y); free(gt); free(up); free(m);
  return 0;
}
