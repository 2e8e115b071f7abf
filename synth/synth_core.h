/* Seeded, counter-based synthetic inputs (weights, caches, prompt tokens).
 *
 * This is the one module that both the CPU oracle's tests and the HIP path's
 * tests and benchmark draw their inputs from.  It holds none of the forward
 * step's arithmetic: it only turns (seed, tensor id, element index) into a
 * bf16 bit pattern or a token id, identically on the host and on the GPU.
 *
 * Generator (published definitions):
 *   - SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
 *     generators", OOPSLA 2014; finaliser constants as in Vigna's public
 *     splitmix64.c).  The j-th output of a stream whose state starts at `key`
 *     is mix(key + (j+1)*GAMMA); that makes every element independently
 *     addressable.
 *   - Stream key for (seed, tensor id): mix(mix(seed + GAMMA) + (id+1)*GAMMA).
 *   - Approximately normal deviates by the Irwin-Hall sum of twelve uniforms
 *     (the classic "sum of 12 uniforms minus 6" generator): element i takes the
 *     outputs 3i, 3i+1, 3i+2 of its stream, splits each into four 16-bit
 *     fields u_k, and forms z = (sum u_k - 393210) / 65536, which has mean 0,
 *     variance 1 - 2^-32 and support [-6, 6].  z is exact in binary64, and the
 *     value mean + std*z is formed with two correctly rounded binary64
 *     operations (no fused multiply-add), then rounded to bf16 to nearest-even.
 *     Only integer operations and IEEE-exact binary64 arithmetic are used, so
 *     host and device produce the same bits.
 *   - Uniform token ids in [0, V): the high 32 bits of output i, times V,
 *     shifted right by 32 (Lemire's multiply-shift range reduction).
 *   - Uniform binary32 values in [0, 1): the high 24 bits of output i times
 *     2^-24 (exact in binary32).
 */
#ifndef SYNTH_CORE_H
#define SYNTH_CORE_H
#include <stdint.h>

#ifdef __HIPCC__
#define SYNTH_FN __host__ __device__ static inline
#else
#define SYNTH_FN static inline
#endif

#define SYNTH_GAMMA 0x9E3779B97F4A7C15ULL

SYNTH_FN uint64_t synth_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

SYNTH_FN uint64_t synth_key(uint64_t seed, uint64_t tensor_id) {
  return synth_mix(synth_mix(seed + SYNTH_GAMMA) + (tensor_id + 1) * SYNTH_GAMMA);
}

SYNTH_FN uint64_t synth_draw(uint64_t key, uint64_t j) {
  return synth_mix(key + (j + 1) * SYNTH_GAMMA);
}

/* Sum of the four 16-bit fields of a 64-bit word. */
SYNTH_FN uint32_t synth_fields(uint64_t w) {
  return (uint32_t)(w & 0xFFFF) + (uint32_t)((w >> 16) & 0xFFFF) +
         (uint32_t)((w >> 32) & 0xFFFF) + (uint32_t)(w >> 48);
}

/* Irwin-Hall deviate for element i, exact in binary64. */
SYNTH_FN double synth_z(uint64_t key, uint64_t i) {
  uint32_t s = synth_fields(synth_draw(key, 3 * i)) + synth_fields(synth_draw(key, 3 * i + 1)) +
               synth_fields(synth_draw(key, 3 * i + 2));
  return ((double)(int32_t)(s - 393210u)) * (1.0 / 65536.0);
}

/* Round a binary64 value to bf16 bits, nearest-even, using only integer
 * operations on its encoding.  Inputs here are finite and far inside the
 * binary32 normal range (|v| <= 7 and either 0 or >= 2^-30), so the 8-bit
 * significand is taken straight from the binary64 one.  Anything else maps to
 * a quiet NaN, which the callers never produce. */
SYNTH_FN uint16_t synth_bf16(double v) {
  union { double d; uint64_t u; } c;
  c.d = v;
  uint64_t sign = c.u >> 63;
  int32_t e = (int32_t)((c.u >> 52) & 0x7FF);
  uint64_t frac = c.u & 0xFFFFFFFFFFFFFULL;
  if (e == 0 && frac == 0) return (uint16_t)(sign << 15);
  if (e < 1023 - 100 || e > 1023 + 100) return 0x7FC0;
  /* keep 7 fraction bits: drop 45 */
  uint64_t keep = frac >> 45, rest = frac & ((1ULL << 45) - 1), half = 1ULL << 44;
  int32_t e32 = e - 1023 + 127;
  uint32_t mag = ((uint32_t)e32 << 7) | (uint32_t)keep;
  if (rest > half || (rest == half && (keep & 1))) mag += 1; /* carries into the exponent */
  return (uint16_t)((sign << 15) | mag);
}

/* No fused multiply-add may contract mean + std*z; the two helpers below are
 * kept apart so each rounds once. */
SYNTH_FN uint16_t synth_normal_elem(uint64_t key, uint64_t i, double mean, double std) {
  double z = synth_z(key, i);
#ifdef __HIP_DEVICE_COMPILE__
  double v = __dadd_rn(mean, __dmul_rn(std, z));
#else
  volatile double p = std * z;
  double v = mean + p;
#endif
  return synth_bf16(v);
}

SYNTH_FN float synth_uniform_elem(uint64_t key, uint64_t i) {
  return (float)(uint32_t)(synth_draw(key, i) >> 40) * (1.0f / 16777216.0f);
}

SYNTH_FN int32_t synth_token_elem(uint64_t key, uint64_t i, int32_t vocab) {
  uint64_t hi = synth_draw(key, i) >> 32;
  return (int32_t)((hi * (uint64_t)vocab) >> 32);
}

#endif
