// Device-side helpers shared by the gfx950 kernels of the MoE FFN layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x2_t __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float f32x4_t __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4_t __attribute__((__vector_size__(4 * sizeof(uint32_t))));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ __bf16 bits_to_bf16(uint16_t b) { return __builtin_bit_cast(__bf16, b); }

// E8M0 scale byte as the fp32 whose exponent field is that byte; the fp4
// converts below use only the exponent of their scale operand, so this
// multiplies by 2^(s-127).
__device__ __forceinline__ float e8m0_scale_operand(uint32_t s) { return __uint_as_float(s << 23); }

// Eight E2M1 codes of one dword (element 2i in the low nibble of byte i) to
// eight bf16 values, each multiplied by the block scale.  One gfx950
// v_cvt_scalef32_pk_bf16_fp4 per byte.
__device__ __forceinline__ bf16x8_t dequant_fp4x8(uint32_t w, float scale) {
  bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0);
  bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1);
  bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2);
  bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3);
  bf16x8_t r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return r;
}

// Eight E4M3 codes (byte i = element i of lo, then of hi) to eight bf16
// values times the block scale: one gfx950 v_cvt_scalef32_pk_bf16_fp8 per
// two codes.  Exact whenever the scaled value is inside bf16's range (an E4M3
// value has 4 significant bits).
__device__ __forceinline__ bf16x8_t dequant_fp8x8(uint32_t lo, uint32_t hi, float scale) {
  bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, false);
  bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, true);
  bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, false);
  bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, true);
  bf16x8_t r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  return r;
}

// D = A(16x32) * B(32x16) + C with fp32 accumulation.  Lane l supplies
// A[l%16][8*(l/16) .. +7] and B[8*(l/16) .. +7][l%16] and holds
// C[4*(l/16) + i][l%16], i = 0..3.
__device__ __forceinline__ f32x4_t mfma_16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8_t zero_bf16x8() {
  bf16x8_t z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = bits_to_bf16(0);
  return z;
}

// silu(min(g, L)) * clamp(u, -L, L)
__device__ __forceinline__ float clamped_swiglu(float g, float u, float limit) {
  g = fminf(g, limit);
  u = fminf(fmaxf(u, -limit), limit);
  return g / (1.0f + __expf(-g)) * u;
}

// Wave-wide max / min without LDS traffic: DPP permutations within each row
// of 16 lanes (pairs, quads, half-row mirror, row mirror), then the four row
// results read into scalar registers.  The result is wave-uniform.  All 64
// lanes must be active.
__device__ __forceinline__ int dpp_quad_1032(int v) { return __builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true); }
__device__ __forceinline__ int dpp_quad_2301(int v) { return __builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true); }
__device__ __forceinline__ int dpp_row_half_mirror(int v) { return __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true); }
__device__ __forceinline__ int dpp_row_mirror(int v) { return __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, true); }

__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, __int_as_float(dpp_quad_1032(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_quad_2301(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_row_half_mirror(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_row_mirror(__float_as_int(v))));
  const int b = __float_as_int(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(b, 0)), r1 = __int_as_float(__builtin_amdgcn_readlane(b, 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(b, 32)), r3 = __int_as_float(__builtin_amdgcn_readlane(b, 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ int wave_min_i32(int v) {
  v = min(v, dpp_quad_1032(v));
  v = min(v, dpp_quad_2301(v));
  v = min(v, dpp_row_half_mirror(v));
  v = min(v, dpp_row_mirror(v));
  const int r0 = __builtin_amdgcn_readlane(v, 0), r1 = __builtin_amdgcn_readlane(v, 16);
  const int r2 = __builtin_amdgcn_readlane(v, 32), r3 = __builtin_amdgcn_readlane(v, 48);
  return min(min(r0, r1), min(r2, r3));
}

// Wave-wide float sum in a fixed association (pairs, quads, half rows, rows,
// then (row0 + row1) + (row2 + row3)): the same bits on every run.
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += __int_as_float(dpp_quad_1032(__float_as_int(v)));
  v += __int_as_float(dpp_quad_2301(__float_as_int(v)));
  v += __int_as_float(dpp_row_half_mirror(__float_as_int(v)));
  v += __int_as_float(dpp_row_mirror(__float_as_int(v)));
  const int b = __float_as_int(v);
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(b, 0)), r1 = __int_as_float(__builtin_amdgcn_readlane(b, 16));
  const float r2 = __int_as_float(__builtin_amdgcn_readlane(b, 32)), r3 = __int_as_float(__builtin_amdgcn_readlane(b, 48));
  return (r0 + r1) + (r2 + r3);
}

// Inclusive prefix sum over a wave.
__device__ __forceinline__ int wave_inclusive_scan(int v) {
  const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

// Exclusive prefix sum over a block of up to 1024 threads; `scratch` holds
// 16 ints of shared memory.  Every thread of the block must call it.
__device__ __forceinline__ int block_exclusive_scan(int v, int* scratch, int* block_total) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int nwaves = (blockDim.x + kWave - 1) / kWave;
  int inc = wave_inclusive_scan(v);
  __syncthreads();
  if (lane == kWave - 1) scratch[wave] = inc;
  __syncthreads();
  int before = 0, total = 0;
  for (int w = 0; w < nwaves; ++w) {
    int s = scratch[w];
    if (w < wave) before += s;
    total += s;
  }
  if (block_total) *block_total = total;
  return before + inc - v;
}

}  // namespace moe
