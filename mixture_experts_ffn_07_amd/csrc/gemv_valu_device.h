// Weight-streaming GEMV on the vector ALUs for one or two tokens: one wave
// computes NR whole output rows.  At this size the projections are pure
// weight streaming, and many waves that each read one contiguous row with
// all of its loads in flight keep more memory requests outstanding across the
// chip than a few waves streaming long ranges (a 75 MB read: ~20 us from 864
// streaming waves, ~14 us from a few thousand light ones).  The arithmetic,
// 2 flops per weight, is far below the vector-ALU rate.
//
// Each lane takes the 16-byte weight vectors v = lane, lane + 64, ... of its
// rows (KV per row, issued together; raw buffer loads past the row read
// zero), multiplies them in fp32 with the matching activation elements of
// the T rows staged in LDS (bf16), and the lanes' sums are added in a fixed
// order (wave_sum_f32), so the result does not depend on scheduling.
#pragma once

#include "moe_device.h"
#include "mx_device.h"

namespace moe {

constexpr int kValuMaxTokens = 2;

// EPV weights per 16-byte vector: 8 (bf16) or 4 (fp32).
template <int EPV, int KV, int NR>
struct ValuRows {
  u32x4_t w[NR][KV];
};

// Issue the weight loads of rows at byte offsets row_off[r] of `rw`
// (a row is K weights).
template <int EPV, int KV, int NR>
__device__ __forceinline__ void valu_issue(ValuRows<EPV, KV, NR>& st, const __amdgpu_buffer_rsrc_t& rw,
                                           const uint32_t (&row_off)[NR], int K) {
  const int lane = threadIdx.x & 63;
  const int nv = K / EPV;
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int i = 0; i < KV; ++i) {
      const int v = lane + 64 * i;
      const uint32_t off = v < nv ? row_off[r] + 16u * (uint32_t)v : kOob;
      st.w[r][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)off, 0, 0));
    }
}

// out[r][t] += this lane's part of sum_k W[r][k] * x[t][k] for t < T (TM >=
// T), x_lds: T rows of K bf16 at stride x_stride elements.
template <int EPV, int KV, int NR, int TM>
__device__ __forceinline__ void valu_accumulate(const ValuRows<EPV, KV, NR>& st, const uint16_t* x_lds,
                                                int x_stride, int T, int K, float (&out)[NR][TM]) {
  const int lane = threadIdx.x & 63;
  const int nv = K / EPV;
#pragma unroll
  for (int i = 0; i < KV; ++i) {
    const int v = min(lane + 64 * i, nv - 1);  // past the row the weights are zero; keep the read in range
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      if (t >= T) break;
      float xv[EPV];
      if constexpr (EPV == 8) {
        const u32x4_t xx = *reinterpret_cast<const u32x4_t*>(x_lds + t * x_stride + 8 * v);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          xv[2 * q] = __uint_as_float(xx[q] << 16);
          xv[2 * q + 1] = __uint_as_float(xx[q] & 0xffff0000u);
        }
      } else {
        const uint2 xx = *reinterpret_cast<const uint2*>(x_lds + t * x_stride + 4 * v);
        xv[0] = __uint_as_float(xx.x << 16);
        xv[1] = __uint_as_float(xx.x & 0xffff0000u);
        xv[2] = __uint_as_float(xx.y << 16);
        xv[3] = __uint_as_float(xx.y & 0xffff0000u);
      }
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        float a = out[r][t];
        if constexpr (EPV == 8) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            a = fmaf(__uint_as_float(st.w[r][i][q] << 16), xv[2 * q], a);
            a = fmaf(__uint_as_float(st.w[r][i][q] & 0xffff0000u), xv[2 * q + 1], a);
          }
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) a = fmaf(__uint_as_float(st.w[r][i][q]), xv[q], a);
        }
        out[r][t] = a;
      }
    }
  }
}

// out[r][t] = sum_k W[r][k] * x[t][k] for t < T (TM >= T), x_lds: T rows of
// K bf16 at stride x_stride elements.  Every lane ends with the full sums.
template <int EPV, int KV, int NR, int TM>
__device__ __forceinline__ void valu_compute(const ValuRows<EPV, KV, NR>& st, const uint16_t* x_lds, int x_stride,
                                             int T, int K, float (&out)[NR][TM]) {
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int t = 0; t < TM; ++t) out[r][t] = 0.f;
  valu_accumulate<EPV, KV, NR, TM>(st, x_lds, x_stride, T, K, out);
#pragma unroll
  for (int r = 0; r < NR; ++r)
#pragma unroll
    for (int t = 0; t < TM; ++t) out[r][t] = wave_sum_f32(out[r][t]);
}

// One MXFP4 block (32 E2M1 codes in a 16-byte vector, element 2i in the low
// nibble of byte i) times 32 bf16 activations at x (LDS, 16-byte aligned),
// added to acc.  Each code pair becomes two bf16 values times the block
// scale (v_cvt_scalef32_pk_bf16_fp4, exact), multiplied with the matching
// activation pair by one v_dot2 with fp32 accumulation.
//
// The activation vector goes through an empty asm register constraint first:
// without it, this hipcc folds the element extraction away and feeds dword 0
// of the 16-byte vector to all four v_dot2c of it (visible in the assembly;
// the results are wrong).
template <int SEL>
__device__ __forceinline__ float mx4_dot_pair(uint32_t codes, float scale, uint32_t xi, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(codes, scale, SEL),
                                         __builtin_bit_cast(bf16x2_t, xi), acc, false);
}

__device__ __forceinline__ float mx4_dot32(const u32x4_t& q, float scale, const uint16_t* x, float acc) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    u32x4_t xx = *reinterpret_cast<const u32x4_t*>(x + 8 * d);
    asm("" : "+v"(xx));
    acc = mx4_dot_pair<0>(q[d], scale, xx[0], acc);
    acc = mx4_dot_pair<1>(q[d], scale, xx[1], acc);
    acc = mx4_dot_pair<2>(q[d], scale, xx[2], acc);
    acc = mx4_dot_pair<3>(q[d], scale, xx[3], acc);
  }
  return acc;
}

// Half an MXFP8 block: 16 E4M3 codes in a 16-byte vector (byte i = element
// i) times 16 bf16 activations at x, added to acc; each code pair becomes two
// bf16 values times the block scale (v_cvt_scalef32_pk_bf16_fp8, exact) for
// one v_dot2.  Same register constraint on the activations as mx4_dot32.
template <bool HI>
__device__ __forceinline__ float mx8_dot_pair(uint32_t codes, float scale, uint32_t xi, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(codes, scale, HI),
                                         __builtin_bit_cast(bf16x2_t, xi), acc, false);
}

__device__ __forceinline__ float mx8_dot16(const u32x4_t& q, float scale, const uint16_t* x, float acc) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    u32x4_t xx = *reinterpret_cast<const u32x4_t*>(x + 8 * h);
    asm("" : "+v"(xx));
    acc = mx8_dot_pair<false>(q[2 * h], scale, xx[0], acc);
    acc = mx8_dot_pair<true>(q[2 * h], scale, xx[1], acc);
    acc = mx8_dot_pair<false>(q[2 * h + 1], scale, xx[2], acc);
    acc = mx8_dot_pair<true>(q[2 * h + 1], scale, xx[3], acc);
  }
  return acc;
}

// One 16-byte vector of codes of either codec against its activations:
// MXFP4 32 elements, MXFP8 16.
template <bool FP8>
__device__ __forceinline__ float mx_dot_vec(const u32x4_t& q, float scale, const uint16_t* x, float acc) {
  if constexpr (FP8)
    return mx8_dot16(q, scale, x, acc);
  else
    return mx4_dot32(q, scale, x, acc);
}

// Copying `pieces` 16-byte pieces into LDS (dst + 16 * q) with all threads
// of the block; piece q is read from byte offset off(q) of `rs`.  A batch
// holds NP pieces per thread, loaded before any is stored, so it costs one
// round trip; issue and commit are separate so that other loads can be
// issued in between.
template <int NP>
struct StageBatch {
  u32x4_t v[NP];
};

template <int NP, typename Off>
__device__ __forceinline__ void stage_issue(StageBatch<NP>& b, const __amdgpu_buffer_rsrc_t& rs, int pieces, int q0,
                                            Off off) {
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int q = q0 + (int)threadIdx.x + (int)blockDim.x * i;
    b.v[i] = __builtin_bit_cast(u32x4_t,
                                __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(q < pieces ? off(q) : kOob), 0, 0));
  }
}

template <int NP>
__device__ __forceinline__ void stage_commit(const StageBatch<NP>& b, int pieces, int q0, uint8_t* dst) {
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const int q = q0 + (int)threadIdx.x + (int)blockDim.x * i;
    if (q < pieces) *reinterpret_cast<u32x4_t*>(dst + 16 * q) = b.v[i];
  }
}

// pieces [q_begin, pieces), batch by batch
template <int NP, typename Off>
__device__ __forceinline__ void stage_pieces(const __amdgpu_buffer_rsrc_t& rs, int pieces, uint8_t* dst, Off off,
                                             int q_begin = 0) {
  for (int q0 = q_begin; q0 < pieces; q0 += NP * (int)blockDim.x) {
    StageBatch<NP> b;
    stage_issue<NP>(b, rs, pieces, q0, off);
    stage_commit<NP>(b, pieces, q0, dst);
  }
}

// Stage T rows of K bf16 (row stride ld elements in global memory) into LDS
// at stride K.
__device__ __forceinline__ void valu_stage_rows(const uint16_t* src, int64_t ld, int T, int K, uint16_t* x_lds) {
  const int per_row = K / 8;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, (uint32_t)((int64_t)T * ld * 2));
  stage_pieces<4>(rs, T * per_row, reinterpret_cast<uint8_t*>(x_lds), [&](int q) {
    const int t = q / per_row, c = q - t * per_row;
    return (uint32_t)(((int64_t)t * ld + 8 * c) * 2);
  });
}

// One gate/up row pair of the shared expert (gate row nrow and up row
// I_s + nrow of sh_gu [2 I_s][H] bf16) against the T rows of x, by the
// calling wave; the block stages x into x_lds (every thread of the block must
// call it).  h_sh[t][nrow] = bf16(clamped SwiGLU).  Rows past I_s read zero
// and write nothing.
__device__ __forceinline__ void shared_gate_up_pair(const uint16_t* x, const uint16_t* sh_gu, uint16_t* h_sh, int T,
                                                    int H, int Is, float limit, int nrow, uint16_t* x_lds) {
  const int lane = threadIdx.x & 63;
  const bool ok = nrow < Is;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(sh_gu, (uint32_t)((int64_t)2 * Is * H * 2));
  const uint32_t off[2] = {ok ? (uint32_t)nrow * (uint32_t)H * 2u : kOob,
                           ok ? (uint32_t)(Is + nrow) * (uint32_t)H * 2u : kOob};
  ValuRows<8, 10, 2> st;
  valu_issue<8, 10, 2>(st, rw, off, H);
  valu_stage_rows(x, H, T, H, x_lds);
  __syncthreads();
  float out2[2][kValuMaxTokens];
  valu_compute<8, 10, 2, kValuMaxTokens>(st, x_lds, H, T, H, out2);
  if (lane == 0 && ok)
    for (int t = 0; t < T; ++t)
      h_sh[(int64_t)t * Is + nrow] = f32_to_bf16(clamped_swiglu(out2[0][t], out2[1][t], limit));
}

}  // namespace moe
