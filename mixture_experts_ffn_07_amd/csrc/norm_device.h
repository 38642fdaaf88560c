// Pre-FFN RMSNorm device code: x_n = bf16(x / sqrt(mean(x^2) + eps) * gamma),
// eps 1e-20 (DeepseekV41Config rms_norm_eps in the max.pipelines API
// reference; norm_eps in the checkpoint config.json on the "DeepSeek V4.1"
// atlas page).
//
// Every step before the final rounding is done in f64: the squares of bf16
// values are exact there, 1/sqrt of the mean is one correctly rounded divide
// of a correctly rounded square root, and (x * r) * gamma are two f64
// products.  The one rounding to bf16 then decides the same value as a
// definition in exact arithmetic unless the f64 product lies within a few
// f64 ulps of a bf16 midpoint.
#pragma once

#include "moe_device.h"

namespace moe {

// Nearest bf16 to d (ties to an even significand), as its bit pattern.  A
// normal result keeps 7 stored significand bits: add 2^44 - 1 plus the lowest
// kept bit to the f64 pattern and clear the 45 bits below it.  Below 2^-126
// bf16 is subnormal with the fixed step 2^-133.  Either result has at most 8
// significant bits, so the f64 -> f32 conversion that follows is exact.
__device__ __forceinline__ uint32_t f64_to_bf16_rne(double d) {
  if (__builtin_expect(__builtin_fabs(d) < 0x1p-126, 0)) {
    d = __builtin_rint(d * 0x1p133) * 0x1p-133;
  } else {
    uint64_t b = __builtin_bit_cast(uint64_t, d);
    b = (b + 0x00000FFFFFFFFFFFull + ((b >> 45) & 1u)) & ~0x00001FFFFFFFFFFFull;
    d = __builtin_bit_cast(double, b);
  }
  return __builtin_bit_cast(uint32_t, (float)d) >> 16;
}

// Sum over the wave, the same value in every lane (lane 0's butterfly result).
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// Sum of squares of four bf16 packed in two dwords, added to acc in f64.
__device__ __forceinline__ double add_squares4(uint32_t a, uint32_t b, double acc) {
  const double v0 = (double)__uint_as_float(a << 16), v1 = (double)__uint_as_float(a & 0xffff0000u);
  const double v2 = (double)__uint_as_float(b << 16), v3 = (double)__uint_as_float(b & 0xffff0000u);
  acc = __builtin_fma(v0, v0, acc);
  acc = __builtin_fma(v1, v1, acc);
  acc = __builtin_fma(v2, v2, acc);
  return __builtin_fma(v3, v3, acc);
}

// r = 1 / sqrt(sum_sq / hidden + eps), wave-uniform.
__device__ __forceinline__ double rms_recip(double sum_sq, int hidden, double eps) {
  return 1.0 / __builtin_sqrt(sum_sq / (double)hidden + eps);
}

// Normalised bf16 bits of bf16 x with gain bf16 g: bf16((x * r) * g).
__device__ __forceinline__ uint32_t norm_one(uint32_t x_bits16, uint32_t g_bits16, double r) {
  const double xv = (double)__uint_as_float(x_bits16 << 16);
  const double gv = (double)__uint_as_float(g_bits16 << 16);
  return f64_to_bf16_rne((xv * r) * gv);
}

// Two packed bf16 (one dword) normalised, packed the same way.
__device__ __forceinline__ uint32_t norm_pair(uint32_t x2, uint32_t g2, double r) {
  return norm_one(x2 & 0xffffu, g2 & 0xffffu, r) | (norm_one(x2 >> 16, g2 >> 16, r) << 16);
}

}  // namespace moe
