/* Host-side walk of the C ABI for an AddressSanitizer / UndefinedBehavior-
 * Sanitizer build of llama_abi.cpp: sizing, loading, cache handles, and the
 * refusal of every bad argument before anything is enqueued.  No call here
 * reaches the device (device addresses are host-side stand-ins that the
 * refusal paths never touch), so it runs without a GPU.  Exits 0 when every
 * call returned what the header states; the sanitizers abort on any invalid
 * memory access or undefined operation in the library's host code. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "llama_mi355x.h"

#define FAKE(off) ((void*)(uintptr_t)(0x10000 + (off)))

static int failures = 0;

#define EXPECT(code, call)                                                              \
  do {                                                                                  \
    int rc_ = (call);                                                                   \
    if (rc_ != (code)) {                                                                \
      fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", __LINE__, #call, rc_, \
              (code), llama_last_error());                                              \
      failures++;                                                                       \
    } else if ((code) != LLAMA_OK && !llama_last_error()[0]) {                          \
      fprintf(stderr, "line %d: refusal without a reason\n", __LINE__);                 \
      failures++;                                                                       \
    }                                                                                   \
  } while (0)

static llama_config tiny(void) {
  llama_config c;
  memset(&c, 0, sizeof c);
  c.n_blocks = 2;
  c.n_loops = 1;
  c.hidden = 512;
  c.n_q_heads = 8;
  c.n_kv_heads = 2;
  c.head_dim = 64;
  c.ffn = 1408;
  c.vocab = 4096;
  c.rope_theta = 10000.0;
  c.rms_eps = 1e-5f;
  c.max_chunk_rows = 64;
  c.max_window_rows = 16;
  c.max_seqs = 2;
  c.prompt_exact = 0;
  return c;
}

static llama_config big(void) {
  llama_config c = tiny();
  c.n_blocks = 52;
  c.hidden = 7168;
  c.n_q_heads = 56;
  c.n_kv_heads = 8;
  c.head_dim = 128;
  c.ffn = 22016;
  c.vocab = 166912;
  c.rope_theta = 1.2e8;
  c.max_chunk_rows = 2048;
  return c;
}

static void fill_blocks(llama_block_weights* b, int n) {
  for (int i = 0; i < n; i++) {
    const void** f = (const void**)&b[i];
    for (size_t j = 0; j < sizeof(llama_block_weights) / sizeof(void*); j++) f[j] = FAKE(64 * j);
  }
}

static void geometry(void) {
  llama_config c = big();
  if (llama_workspace_bytes(&c, 131072 + 256) == 0) {
    fprintf(stderr, "33B geometry refused: %s\n", llama_last_error());
    failures++;
  }
  for (int i = 0; i < 14; i++) {
    llama_config b = big();
    switch (i) {
      case 0: b.head_dim = 96; break;
      case 1: b.hidden = 7000; break;
      case 2: b.n_q_heads = 50; break;
      case 3: b.n_q_heads = 72; break;
      case 4: b.vocab = 166913; break;
      case 5: b.rope_theta = 0.0; break;
      case 6: b.max_chunk_rows = 4096; break;
      case 7: b.max_window_rows = 17; break;
      case 8: b.max_seqs = 0; break;
      case 9: b.ffn = 22000; break;
      case 10: b.n_loops = 0; break;
      case 11: b.rms_eps = -1.0f; break;
      case 12: b.prompt_exact = 2; break;
      case 13: b.rope_theta = NAN; break;
    }
    if (llama_workspace_bytes(&b, 4096) != 0 || !llama_last_error()[0]) {
      fprintf(stderr, "geometry change %d not refused\n", i);
      failures++;
    }
  }
}

static void model_and_caches(void) {
  llama_config c = tiny();
  llama_block_weights b[2];
  fill_blocks(b, 2);
  size_t ws = llama_workspace_bytes(&c, 512);
  llama_model* m = NULL;
  EXPECT(LLAMA_E_GEOMETRY, llama_load_weights(&c, b, FAKE(0), FAKE(8), FAKE(0), FAKE(16), ws, 512, &m));
  EXPECT(LLAMA_E_ARG, llama_load_weights(&c, b, FAKE(0), FAKE(8), NULL, FAKE(16), ws, 512, &m));
  EXPECT(LLAMA_E_WORKSPACE,
         llama_load_weights(&c, b, FAKE(0), FAKE(8), FAKE(24), FAKE(16), ws - 1, 512, &m));
  EXPECT(LLAMA_OK, llama_load_weights(&c, b, FAKE(0), FAKE(8), FAKE(24), FAKE(16), ws, 512, &m));
  if (!m) return;
  size_t kvb = llama_kv_bytes(m, 128);
  if (kvb != (size_t)2 * 128 * 2 * 64 * 2 * 2) {
    fprintf(stderr, "kv bytes %zu\n", kvb);
    failures++;
  }
  llama_kv *kv = NULL, *kv2 = NULL;
  EXPECT(LLAMA_E_CAPACITY, llama_kv_alloc(m, 513, FAKE(0), (size_t)1 << 30, &kv));
  EXPECT(LLAMA_E_WORKSPACE, llama_kv_alloc(m, 128, FAKE(0), kvb - 1, &kv));
  EXPECT(LLAMA_OK, llama_kv_alloc(m, 128, FAKE(0), kvb, &kv));
  EXPECT(LLAMA_OK, llama_kv_alloc(m, 128, FAKE(kvb), kvb, &kv2));
  if (llama_kv_slab(kv, 2, 0) != NULL) failures++;
  if (llama_kv_slab(kv, 1, 1) != FAKE((2 * 1 + 1) * 128 * 2 * 64 * 2)) failures++;

  llama_kv* one[1] = {kv};
  llama_kv* two[2] = {kv, kv};
  llama_kv* three[3] = {kv, kv2, kv};
  EXPECT(LLAMA_E_ARG, llama_decode_step(m, one, 1, FAKE(0), NULL, 17, NULL, NULL, NULL, NULL, NULL));
  EXPECT(LLAMA_E_ARG, llama_decode_step(m, one, 1, FAKE(0), NULL, 0, NULL, NULL, NULL, NULL, NULL));
  EXPECT(LLAMA_E_ARG, llama_decode_step(m, two, 2, FAKE(0), NULL, 1, NULL, NULL, NULL, NULL, NULL));
  EXPECT(LLAMA_E_ARG, llama_decode_step(m, three, 3, FAKE(0), NULL, 1, NULL, NULL, NULL, NULL, NULL));
  EXPECT(LLAMA_E_ARG, llama_decode_step(m, one, 1, FAKE(0), FAKE(0), 1, NULL, NULL, NULL, NULL, NULL));
  EXPECT(LLAMA_E_ARG, llama_decode_step(m, one, 1, NULL, NULL, 1, NULL, NULL, NULL, NULL, NULL));
  EXPECT(LLAMA_OK, llama_test_kv_declare(kv, 127));
  EXPECT(LLAMA_E_CAPACITY, llama_decode_step(m, one, 1, FAKE(0), NULL, 2, NULL, NULL, NULL, NULL, NULL));
  EXPECT(LLAMA_OK, llama_test_kv_declare(kv, 128));
  EXPECT(LLAMA_E_CAPACITY, llama_test_kv_declare(kv, 129));
  EXPECT(LLAMA_OK, llama_kv_truncate(kv, 100));
  EXPECT(LLAMA_E_POSITION, llama_kv_truncate(kv, 101));
  EXPECT(LLAMA_E_POSITION, llama_kv_truncate(kv, -1));
  if (llama_kv_length(kv) != 100) failures++;
  EXPECT(LLAMA_E_POSITION, llama_prefill_chunk(m, kv, FAKE(0), NULL, 8, 3, NULL, NULL, NULL, 0, NULL, NULL));
  EXPECT(LLAMA_OK, llama_kv_truncate(kv, 0));
  EXPECT(LLAMA_E_ARG, llama_prefill_chunk(m, kv, FAKE(0), NULL, 65, 0, NULL, NULL, NULL, 0, NULL, NULL));
  EXPECT(LLAMA_E_ARG, llama_prefill_chunk(m, kv, NULL, NULL, 8, 0, NULL, NULL, NULL, 0, NULL, NULL));

  /* capture and probe bounds */
  EXPECT(LLAMA_OK, llama_set_capture(m, FAKE(0), 16));
  EXPECT(LLAMA_E_WORKSPACE, llama_decode_step(m, one, 1, FAKE(0), NULL, 1, NULL, NULL, NULL, NULL, NULL));
  EXPECT(LLAMA_OK, llama_set_capture(m, NULL, 0));
  llama_probe p;
  memset(&p, 0, sizeof p);
  p.attn = FAKE(0);
  EXPECT(LLAMA_E_ARG, llama_set_probe(m, 2, &p, 4));
  EXPECT(LLAMA_E_ARG, llama_set_probe(m, -1, &p, 4));
  EXPECT(LLAMA_E_ARG, llama_set_probe(m, 0, &p, 0));
  EXPECT(LLAMA_OK, llama_set_probe(m, 1, &p, 4));
  EXPECT(LLAMA_E_WORKSPACE, llama_prefill_chunk(m, kv, FAKE(0), NULL, 5, 0, NULL, NULL, NULL, 0, NULL, NULL));
  EXPECT(LLAMA_OK, llama_set_probe(m, 0, NULL, 0));

  /* single-kernel test entries */
  EXPECT(LLAMA_E_ARG, llama_test_linear(m, 3, FAKE(0), 4, FAKE(0), 128, 128, FAKE(0), NULL, NULL));
  EXPECT(LLAMA_E_ARG, llama_test_linear(m, 1, FAKE(0), 4, FAKE(0), 100, 128, FAKE(0), NULL, NULL));
  EXPECT(LLAMA_E_ARG, llama_test_linear(m, 0, FAKE(0), 17, FAKE(0), 128, 128, FAKE(0), NULL, NULL));
  EXPECT(LLAMA_E_ARG, llama_test_attention(m, 1, kv, 2, FAKE(0), 4, 0, FAKE(0), NULL, NULL));
  EXPECT(LLAMA_E_POSITION, llama_test_attention(m, 1, kv, 0, FAKE(0), 4, 0, FAKE(0), NULL, NULL));

  /* sampling arguments */
  EXPECT(LLAMA_E_ARG, llama_sample(m, FAKE(0), 0, 4096, 0.6f, 20, 0.95f, FAKE(0), FAKE(0), NULL));
  EXPECT(LLAMA_E_ARG, llama_sample(m, FAKE(0), 4, 4095, 0.6f, 20, 0.95f, FAKE(0), FAKE(0), NULL));
  EXPECT(LLAMA_E_ARG, llama_sample(m, FAKE(0), 4, 4096, NAN, 20, 0.95f, FAKE(0), FAKE(0), NULL));
  EXPECT(LLAMA_E_ARG, llama_sample(m, FAKE(0), 4, 4096, 0.6f, 65, 0.95f, FAKE(0), FAKE(0), NULL));
  EXPECT(LLAMA_E_ARG, llama_sample(m, FAKE(0), 4, 4096, 0.6f, 20, 1.5f, FAKE(0), FAKE(0), NULL));

  /* drafting: same model as draft is refused; lengths unchanged */
  EXPECT(LLAMA_E_ARG, llama_draft_round(m, kv, m, kv, 4, FAKE(0), FAKE(0), NULL, NULL));

  /* another model's cache */
  llama_model* m2 = NULL;
  EXPECT(LLAMA_OK, llama_load_weights(&c, b, FAKE(0), FAKE(8), FAKE(24), FAKE(16), ws, 512, &m2));
  EXPECT(LLAMA_E_ARG, llama_decode_step(m2, one, 1, FAKE(0), NULL, 1, NULL, NULL, NULL, NULL, NULL));
  llama_free(m2);
  llama_kv_free(kv);
  llama_kv_free(kv2);
  llama_free(m);
}

static void blocks_only(void) {
  llama_config c = big();
  c.n_blocks = 1;
  c.vocab = 0;
  c.max_chunk_rows = 16;
  c.max_seqs = 1;
  llama_block_weights b[1];
  fill_blocks(b, 1);
  size_t ws = llama_workspace_bytes(&c, 64);
  llama_model* m = NULL;
  EXPECT(LLAMA_E_ARG, llama_load_weights(&c, b, FAKE(0), NULL, NULL, FAKE(16), ws, 64, &m));
  EXPECT(LLAMA_OK, llama_load_weights(&c, b, NULL, NULL, NULL, FAKE(16), ws, 64, &m));
  if (!m) return;
  llama_kv* kv = NULL;
  EXPECT(LLAMA_OK, llama_kv_alloc(m, 64, FAKE(0), llama_kv_bytes(m, 64), &kv));
  llama_kv* one[1] = {kv};
  EXPECT(LLAMA_E_ARG, llama_decode_step(m, one, 1, FAKE(0), NULL, 1, NULL, NULL, NULL, NULL, NULL));
  EXPECT(LLAMA_E_ARG, llama_sample(m, FAKE(0), 1, 128, 1.0f, 1, 1.0f, FAKE(0), FAKE(0), NULL));
  llama_kv_free(kv);
  llama_free(m);
}

int main(void) {
  geometry();
  model_and_caches();
  blocks_only();
  if (failures) {
    fprintf(stderr, "%d unexpected results\n", failures);
    return 1;
  }
  printf("abi host check ok\n");
  return 0;
}
