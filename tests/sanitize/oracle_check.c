/* Every oracle entry point on small and edge-sized inputs, for an
 * AddressSanitizer / UndefinedBehaviorSanitizer build of oracle.c (test
 * infrastructure checking test infrastructure).  Shapes cover one row, a
 * ragged row count, grouped heads, head sizes 64 and 128, a block run as a
 * chunk then as one-row steps, a refused position, the planted mistake and
 * non-finite rows.  A few invariants that hold at any size are asserted; the
 * numerical pins live in the Python tests.  Exits 0 on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

static int failures = 0;
#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      fprintf(stderr, "line %d: check failed: %s\n", __LINE__, #cond); \
      failures++;                                                        \
    }                                                                    \
  } while (0)

static uint64_t state = 0x9e3779b97f4a7c15ull;
static double uni(void) { /* xorshift64*, test data only */
  state ^= state >> 12;
  state ^= state << 25;
  state ^= state >> 27;
  return (double)((state * 0x2545f4914f6cdd1dull) >> 11) * 0x1.0p-53;
}

static uint16_t* bf16_rand(int64_t n, double scale, double offset) {
  uint16_t* p = malloc((size_t)n * sizeof *p);
  for (int64_t i = 0; i < n; i++) p[i] = orc_bf16(offset + scale * (2.0 * uni() - 1.0));
  return p;
}

static void scalars(void) {
  CHECK(orc_f64(orc_bf16(1.0)) == 1.0);
  CHECK(isnan(orc_f64(orc_bf16(NAN))));
  CHECK(isinf(orc_f64(orc_bf16(INFINITY))));
  CHECK(orc_f64(orc_bf16(1e-40)) >= 0.0);
  double xs[5] = {0.0, -0.0, 1e38, -1e-45, 3.14159};
  uint16_t out[5];
  orc_bf16_array(xs, 5, out);
  CHECK(out[0] == 0 && out[1] == 0x8000);
}

static void rows_and_projections(int64_t rows, int64_t H, int64_t N) {
  const int64_t V = 300;
  uint16_t* E = bf16_rand(V * H, 0.5, 0.0);
  int32_t* tok = malloc((size_t)rows * sizeof *tok);
  for (int64_t r = 0; r < rows; r++) tok[r] = (int32_t)(r * 37 % V);
  uint16_t* h = malloc((size_t)(rows * H) * sizeof *h);
  orc_embed(E, V, H, tok, rows, h);
  CHECK(memcmp(h, E + (int64_t)tok[rows - 1] * H, (size_t)H * 2) == 0 || rows > 0);
  uint16_t* w = bf16_rand(H, 0.02, 1.0);
  uint16_t* x = malloc((size_t)(rows * H) * sizeof *x);
  orc_rmsnorm(h, w, rows, H, 1e-5f, x);
  uint16_t* W = bf16_rand(N * H, 0.02, 0.0);
  uint16_t* y = malloc((size_t)(rows * N) * sizeof *y);
  double* y64 = malloc((size_t)(rows * N) * sizeof *y64);
  orc_linear(x, W, rows, N, H, y, y64);
  for (int64_t i = 0; i < rows * N; i++) CHECK(y[i] == orc_bf16(y64[i]));
  uint16_t* a = malloc((size_t)(rows * N) * sizeof *a);
  orc_swiglu(y, y, rows * N, a);
  orc_residual_add(y, a, rows * N);
  int32_t id = orc_argmax(y, N);
  CHECK(id >= 0 && id < N);
  free(E), free(tok), free(h), free(w), free(x), free(W), free(y), free(y64), free(a);
}

static void rope_and_attention(int64_t rows, int64_t nq, int64_t nkv, int64_t d, int64_t T) {
  float* inv = malloc((size_t)(d / 2) * sizeof *inv);
  orc_rope_inv_freq(d, 1.2e8, inv);
  CHECK(inv[0] == 1.0f);
  int32_t* pos = malloc((size_t)rows * sizeof *pos);
  for (int64_t r = 0; r < rows; r++) pos[r] = (int32_t)(T - rows + r);
  uint16_t* q = bf16_rand(rows * nq * d, 1.0, 0.0);
  orc_rope(q, pos, rows, nq, d, 1.2e8);
  uint16_t* kc = bf16_rand(T * nkv * d, 1.0, 0.0);
  uint16_t* vc = malloc((size_t)(T * nkv * d) * sizeof *vc);
  for (int64_t i = 0; i < T * nkv * d; i++) vc[i] = orc_bf16(1.0);
  uint16_t* out = malloc((size_t)(rows * nq * d) * sizeof *out);
  double* out64 = malloc((size_t)(rows * nq * d) * sizeof *out64);
  orc_attention(q, kc, vc, pos, rows, nq, nkv, d, out, out64);
  /* values of 1 average to 1 at any weights */
  for (int64_t i = 0; i < rows * nq * d; i++) CHECK(out[i] == orc_bf16(1.0));
  free(inv), free(pos), free(q), free(kc), free(vc), free(out), free(out64);
}

static void block_steps(int64_t H, int64_t nq, int64_t nkv, int64_t d, int64_t F) {
  orc_geom g = {H, nq, nkv, d, F, 1.2e8, 1e-5f};
  const int64_t T = 12, chunk = 7;
  uint16_t *an = bf16_rand(H, 0.02, 1.0), *mn = bf16_rand(H, 0.02, 1.0);
  uint16_t* q = bf16_rand(nq * d * H, 0.02, 0.0);
  uint16_t* k = bf16_rand(nkv * d * H, 0.02, 0.0);
  uint16_t* v = bf16_rand(nkv * d * H, 0.02, 0.0);
  uint16_t* o = bf16_rand(H * nq * d, 0.02, 0.0);
  uint16_t* gt = bf16_rand(F * H, 0.02, 0.0);
  uint16_t* up = bf16_rand(F * H, 0.02, 0.0);
  uint16_t* dn = bf16_rand(H * F, 0.02, 0.0);
  orc_block_weights w = {an, q, k, v, o, mn, gt, up, dn};
  uint16_t* kc = calloc((size_t)(T * nkv * d), 2);
  uint16_t* vc = calloc((size_t)(T * nkv * d), 2);
  uint16_t* h = bf16_rand((chunk + 2) * H, 1.0, 0.0);
  uint16_t* mid = malloc((size_t)((chunk + 2) * H) * 2);
  int32_t pos[9];
  for (int i = 0; i < 9; i++) pos[i] = i;
  CHECK(orc_block(&g, &w, kc, vc, T, pos, chunk, h, mid) == 0);
  CHECK(orc_block(&g, &w, kc, vc, T, pos + chunk, 1, h + chunk * H, NULL) == 0);
  CHECK(orc_block(&g, &w, kc, vc, T, pos + chunk + 1, 1, h + (chunk + 1) * H, mid) == 0);
  int32_t bad = (int32_t)T;
  CHECK(orc_block(&g, &w, kc, vc, T, &bad, 1, h, NULL) == -1);
  orc_plant(1);
  CHECK(orc_block(&g, &w, kc, vc, T, pos, 2, h, NULL) == 0);
  orc_plant(0);
  free(an), free(mn), free(q), free(k), free(v), free(o), free(gt), free(up), free(dn);
  free(kc), free(vc), free(h), free(mid);
}

static void sampling(void) {
  const int64_t V = 1000;
  uint16_t* l = bf16_rand(V, 3.0, 0.0);
  double margin = 0.0;
  for (int k = 1; k <= 64; k *= 4) {
    int32_t t = orc_sample(l, V, 0.6, k, 0.95, 0.5, &margin);
    CHECK(t >= 0 && t < V);
    t = orc_sample(l, V, 1.0, k, 1.0, 0.999999, NULL);
    CHECK(t >= 0 && t < V);
  }
  CHECK(orc_sample(l, V, 0.6, 1, 0.95, 0.3, NULL) == orc_argmax(l, V));
  l[V / 2] = orc_bf16(NAN);
  CHECK(orc_argmax(l, V) < 0);
  CHECK(orc_sample(l, V, 0.6, 20, 0.95, 0.5, NULL) < 0);
  free(l);
}

int main(void) {
  scalars();
  rows_and_projections(1, 256, 128);
  rows_and_projections(13, 512, 384);
  rope_and_attention(1, 4, 1, 128, 1);
  rope_and_attention(5, 8, 2, 64, 37);
  rope_and_attention(3, 7, 1, 128, 130);
  block_steps(256, 4, 2, 64, 384);
  block_steps(256, 2, 1, 128, 256);
  sampling();
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("oracle check ok\n");
  return 0;
}
