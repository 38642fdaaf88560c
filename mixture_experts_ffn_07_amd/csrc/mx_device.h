// Two-term MXFP8 (E4M3) form of bf16 activation rows for gfx950's
// block-scaled matrix instructions.
//
// For a block of 32 consecutive values: scale exponent e = floor(log2 max|x|)
// - 8 (8 = largest E4M3 exponent), stored as the E8M0 byte e + 127 (an
// all-zero block gets 127); hi = E4M3(x / 2^e) rounded to nearest even and
// held within +-448; lo = E4M3(x / 2^e - hi), the residual of the unclamped
// scaled value.  hi + lo keeps about 8 significant bits, the precision of the
// bf16 input.  A staged row of K values is laid out as hi codes [K], lo codes
// [K], scale bytes [K/32], then padding to a multiple of 16 bytes plus 16.
#pragma once

#include "moe_device.h"

namespace moe {

constexpr int kMxPad = 16;  // bytes of padding per staged row

__host__ __device__ inline int mx_row_bytes(int K) { return ((2 * K + K / 32 + 15) & ~15) + kMxPad; }

// Four scaled values to four E4M3 codes (byte i = value i).
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  return ((uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu) |
         ((uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, 0, false) << 16);
}

// Converts x[32] (the block) and writes 32 hi codes, 32 lo codes and the
// scale byte.  hi_dst/lo_dst must be 16-byte aligned.
__device__ __forceinline__ void mx_convert_block(const float (&x)[32], uint8_t* hi_dst, uint8_t* lo_dst,
                                                 uint8_t* scale_dst) {
  float amax = 0.f;
#pragma unroll
  for (int t = 0; t < 32; ++t) amax = fmaxf(amax, fabsf(x[t]));
  const int ex = (int)((__float_as_uint(amax) >> 23) & 0xff) - 127;  // floor(log2(amax)) for normal amax
  const int sc = amax > 0.f ? min(max(ex - 8 + 127, 1), 253) : 127;
  const float inv = __uint_as_float((uint32_t)(254 - sc) << 23);  // 2^(127 - sc)
  uint32_t hi[8], lo[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    float s4[4], c4[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      s4[u] = x[4 * t + u] * inv;  // in (-512, 512)
      c4[u] = fminf(fmaxf(s4[u], -448.f), 448.f);
    }
    const uint32_t h = e4m3x4(c4[0], c4[1], c4[2], c4[3]);
    hi[t] = h;
    lo[t] = e4m3x4(s4[0] - __builtin_amdgcn_cvt_f32_fp8((int)h, 0), s4[1] - __builtin_amdgcn_cvt_f32_fp8((int)h, 1),
                   s4[2] - __builtin_amdgcn_cvt_f32_fp8((int)h, 2), s4[3] - __builtin_amdgcn_cvt_f32_fp8((int)h, 3));
  }
  u32x4_t* dh = reinterpret_cast<u32x4_t*>(hi_dst);
  u32x4_t* dl = reinterpret_cast<u32x4_t*>(lo_dst);
  dh[0] = u32x4_t{hi[0], hi[1], hi[2], hi[3]};
  dh[1] = u32x4_t{hi[4], hi[5], hi[6], hi[7]};
  dl[0] = u32x4_t{lo[0], lo[1], lo[2], lo[3]};
  dl[1] = u32x4_t{lo[4], lo[5], lo[6], lo[7]};
  *scale_dst = (uint8_t)sc;
}

// The 32 bf16 values held in four 16-byte pieces, as floats.
__device__ __forceinline__ void unpack_bf16x32(const u32x4_t (&v)[4], float (&x)[32]) {
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      x[8 * q + 2 * w] = __uint_as_float(v[q][w] << 16);
      x[8 * q + 2 * w + 1] = __uint_as_float(v[q][w] & 0xffff0000u);
    }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

constexpr uint32_t kOob = 0x7ffffff0u;  // a buffer offset past any matrix: the load returns 0

typedef int i32x8_t __attribute__((__vector_size__(8 * sizeof(int))));

// D += A(16x128, E4M3 with E8M0 per 32) * B(128x16, E2M1 with E8M0 per 32), fp32.
// Lane l = 16g + m: A row m, chunk offsets [16g,16g+16) in dwords 0-3 and
// [64+16g,64+16g+16) in dwords 4-7, scale of A block g (rows m); B column m,
// offsets [32g,32g+32) (low nibble first) and the scale of that block.
__device__ __forceinline__ f32x4_t mfma_mx(const i32x8_t& a, const u32x4_t& b, int sa, int sb, f32x4_t c) {
  const i32x8_t bw = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bw, c, 0, 4, 0, sa, 0, sb);
}

}  // namespace moe
