/* Host side of the synthetic-input generator (definitions in synth_core.h).
 * Element values depend only on (seed, tensor id, index), never on the
 * thread count. */
#include <stddef.h>
#include "synth_core.h"

void synth_normal_bf16(uint16_t* out, int64_t n, uint64_t seed, uint64_t tensor_id,
                       int64_t offset, double mean, double std) {
  uint64_t key = synth_key(seed, tensor_id);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = synth_normal_elem(key, (uint64_t)(offset + i), mean, std);
}

void synth_tokens(int32_t* out, int64_t n, uint64_t seed, uint64_t tensor_id, int64_t offset,
                  int32_t vocab) {
  uint64_t key = synth_key(seed, tensor_id);
  for (int64_t i = 0; i < n; ++i) out[i] = synth_token_elem(key, (uint64_t)(offset + i), vocab);
}

void synth_uniform_f32(float* out, int64_t n, uint64_t seed, uint64_t tensor_id, int64_t offset) {
  uint64_t key = synth_key(seed, tensor_id);
  for (int64_t i = 0; i < n; ++i) out[i] = synth_uniform_elem(key, (uint64_t)(offset + i));
}
