// Device helpers shared by the gfx950 kernels: bf16 conversions, packed
// bf16 dot products, wave64 reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

#define WAVE 64

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf2f(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ bf16_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (bf16_t)0x7FC0;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}
// fp32 -> nearest bf16 value, as fp32.
__device__ __forceinline__ float rbf(float f) { return bf2f(f2bf(f)); }

__device__ __forceinline__ uint32_t pack_bf2(bf16_t lo, bf16_t hi) {
  return (uint32_t)lo | ((uint32_t)hi << 16);
}

// acc + a.lo*b.lo + a.hi*b.hi on packed bf16 pairs (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// Butterfly sum over the 64 lanes; every lane ends with the same value, and
// the association order is fixed (xor 32, 16, 8, 4, 2, 1).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, WAVE);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, WAVE));
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (WAVE - 1); }

// RMSNorm, bf16(w * bf16(x * r)) with r = 1/sqrt(sum(x^2)/H + eps) (pull
// request "llama: Nanbeige4.3-33B on Metal, the bf16 release served as
// published", section "How").  The sum of squares, r and x * r are binary64:
// a bf16 square is exact there and a row's sum of them is exact for any
// spread of magnitudes a normalised activation has (16 bits per square plus
// the row's exponent range and log2(H) bits of growth fit in 53), so the
// order of the sum does not change it; sqrt and the division are correctly
// rounded, and x * r is rounded once to bf16 (via round-to-odd to fp32).  The
// normed value is therefore the correctly rounded one, the same from the
// standalone norm kernel and from every projection that normalises its own
// input rows.  A full wave sums a row, lane l taking 16-byte vectors l,
// l+64, ..., then the xor butterfly.  H is a multiple of 8.

// binary64 -> bf16 bits, round to nearest even.  Inside bf16's normal range
// (biased binary64 exponent 897..1150) the rounding is done on the bits: add
// half an ulp of bit 45 (less one, plus the kept lsb: ties to even), keep
// sign, exponent and the top 7 mantissa bits, rebias the exponent by
// 1023 - 127 (a carry into the exponent rounds up correctly, to Inf past the
// largest value).  Elsewhere (zero, bf16 subnormals, Inf, NaN) through fp32
// with round to odd -- truncate and set the last bit if anything was dropped,
// 24 bits >= 8 + 2 making the second rounding exact -- then fp32 -> bf16.
__device__ __forceinline__ bf16_t d2bf(double x) {
  uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint32_t e = (uint32_t)(b >> 52) & 0x7FFu;
  if (e >= 897u && e <= 1150u) {
    b += 0x00000FFFFFFFFFFFull + ((b >> 45) & 1ull);
    const uint32_t t = (uint32_t)(b >> 45);  // sign | exponent (11) | mantissa (7)
    return (bf16_t)((((t >> 18) & 1u) << 15) | ((t & 0x3FFFFu) - (896u << 7)));
  }
  float f = __double2float_rz(x);
  if ((double)f != x) f = __uint_as_float(__float_as_uint(f) | 1u);
  return f2bf(f);
}

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, WAVE);
  return v;
}

// One 16-byte vector's squares added to a running binary64 sum.
__device__ __forceinline__ double sumsq8(u32x4_t q, double ss) {
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const double a = bf_lo(w[j]), b = bf_hi(w[j]);
    ss = fma(a, a, ss);
    ss = fma(b, b, ss);
  }
  return ss;
}

__device__ __forceinline__ double inv_rms(double lane_ss, int H, float eps) {
  const double ss = wave_sum_d(lane_ss);
  return 1.0 / sqrt(ss / (double)H + (double)eps);
}

__device__ __forceinline__ double row_inv_rms(const bf16_t* __restrict__ x, int H, float eps) {
  const u32x4_t* xv = (const u32x4_t*)x;
  const int nv = H / 8;
  double ss = 0.0;
  // loads are issued eight at a time
  for (int v0 = lane_id(); v0 < nv; v0 += 8 * WAVE) {
    u32x4_t q[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int v = v0 + i * WAVE;
      q[i] = v < nv ? xv[v] : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (v0 + i * WAVE >= nv) break;
      ss = sumsq8(q[i], ss);
    }
  }
  return inv_rms(ss, H, eps);
}

// The same sum over a row already staged in LDS (nv = H / 8 vectors).
__device__ __forceinline__ double row_inv_rms_lds(const u32x4_t* xv, int H, float eps) {
  const int nv = H / 8;
  double ss = 0.0;
  for (int v = lane_id(); v < nv; v += WAVE) ss = sumsq8(xv[v], ss);
  return inv_rms(ss, H, eps);
}

// Eight normalised elements: bf16(w * bf16(x * r)), packed.
__device__ __forceinline__ u32x4_t norm8(u32x4_t x, u32x4_t w, double r) {
  const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ws[4] = {w.x, w.y, w.z, w.w};
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float n0 = bf2f(d2bf((double)bf_lo(xs[j]) * r));
    const float n1 = bf2f(d2bf((double)bf_hi(xs[j]) * r));
    o[j] = pack_bf2(f2bf(bf_lo(ws[j]) * n0), f2bf(bf_hi(ws[j]) * n1));
  }
  return u32x4_t{o[0], o[1], o[2], o[3]};
}
