// Two-term MXFP6 (E2M3) rows: the activation operand of the block-scaled
// matrix instruction v_mfma_scale_f32_16x16x128_f8f6f4 in the grouped GEMMs
// for many tokens.
//
// A bf16 row is cut into blocks of 32 consecutive values.  Per block:
//   hi = E2M3(x / 2^e1), e1 = floor(log2 max|x|) - 2 (2: largest E2M3
//        exponent), rounded to nearest even, saturating at +-7.5;
//   r  = x - 2^e1 hi (exact in fp32: both terms are multiples of the
//        smaller one's unit in the last place);
//   lo = E2M3(r / 2^e2), e2 = floor(log2 max|r|) - 2.
// x = 2^e1 hi + 2^e2 lo + (a rounding error of lo), about 8 significant
// bits, the precision of the bf16 input.  An all-zero block (or residual)
// gets the scale byte 127 and zero codes.  Scale bytes are E8M0 (e + 127),
// held in [0, 254].
//
// Storage: per 128-wide chunk of K a record of kMx6Rec = 208 bytes laid out
// for the MFMA's lane order (lane 16 g + m reads row m, K values
// [32 g, 32 g + 32) of the chunk as 32 sequential 6-bit fields in 6 dwords):
//   [  0,  64)  hi, dwords 0-3 of lane group g at 16 g
//   [ 64,  96)  hi, dwords 4-5 of lane group g at 64 + 8 g
//   [ 96, 160)  lo, dwords 0-3 at 96 + 16 g
//   [160, 192)  lo, dwords 4-5 at 160 + 8 g
//   [192, 208)  scales, one dword per lane group at 192 + 4 g: byte 0 the
//               hi scale, byte 1 the lo scale (the instruction's op_sel
//               picks the byte), bytes 2-3 zero.
#pragma once

#include "moe_device.h"

namespace moe {

constexpr int kMx6Rec = 208;  // bytes per row and 128-wide chunk
constexpr int kMx6TileRows = 96;  // rows per tile of the grouped GEMM
__host__ __device__ inline int64_t mx6_row_bytes(int K) { return (int64_t)(K / 128) * kMx6Rec; }

}  // namespace moe
