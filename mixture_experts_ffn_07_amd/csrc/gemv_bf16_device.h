// Weight-streaming projection with bf16 weights (the shared expert) for few
// tokens, as a block-level device function: used by the standalone bf16
// kernel and by the fused few-token kernels, which run it beside the router
// and the routing step.
//
// Weights are read with raw buffer loads (a load past the end of the matrix
// returns zero without touching memory, so every load is issued
// unconditionally); v_mfma_f32_16x16x32_bf16 on rows staged in LDS.
#pragma once

#include "moe_device.h"
#include "moe_internal.h"
#include "mx_device.h"

namespace moe {

constexpr int kLdsPad = 8;  // bf16 elements of padding per staged bf16 row
constexpr int kBf16Chunks = 2;  // 128-wide chunks per batch

// Weights of kBf16Chunks 128-wide K chunks for this lane's row(s), as loaded.
template <int NB>
struct Bf16Batch {
  u32x4_t h[kBf16Chunks][NB][4];
};

struct Bf16View {
  __amdgpu_buffer_rsrc_t w;
  uint32_t row_off[2];  // byte offset of this lane's row(s)
  int K, nchunks;
};

template <int NB>
__device__ __forceinline__ void bf16_load(Bf16Batch<NB>& b, const Bf16View& v, int first_chunk, int grp) {
#pragma unroll
  for (int u = 0; u < kBf16Chunks; ++u) {
    const int c = first_chunk + 4 * u;
    const int k0 = c * 128 + grp * 32;
    const bool ok = c < v.nchunks && k0 < v.K;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint32_t ho = ok ? v.row_off[nb] + (uint32_t)(k0 * 2) : kOob;
#pragma unroll
      for (int s = 0; s < 4; ++s)
        b.h[u][nb][s] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(v.w, (int)ho, 16 * s, 0));
    }
  }
}

template <int NB>
__device__ __forceinline__ void bf16_mma(const Bf16Batch<NB>& b, f32x4_t (&acc)[NB], const uint16_t* a_lds,
                                         int a_stride, int rows, int first_chunk, const Bf16View& v, int lane) {
  const int col = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int u = 0; u < kBf16Chunks; ++u) {
    const int c = first_chunk + 4 * u;
    if (c >= v.nchunks) break;  // wave-uniform; no loads below
    const int k0 = c * 128 + grp * 32;
    bf16x8_t a[4];
    if (col < rows && k0 < v.K) {
      const bf16x8_t* src = reinterpret_cast<const bf16x8_t*>(a_lds + col * a_stride + k0);
#pragma unroll
      for (int s = 0; s < 4; ++s) a[s] = src[s];
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) a[s] = zero_bf16x8();
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
      for (int s = 0; s < 4; ++s) acc[nb] = mfma_16x16x32(a[s], __builtin_bit_cast(bf16x8_t, b.h[u][nb][s]), acc[nb]);
    }
  }
}

// The rows' bf16 values into LDS (row stride K + kLdsPad).  All loads of a
// pass are issued before any store; pieces past the rows read zero.
__device__ __forceinline__ void bf16_stage(const GemvProblem& p, int m_begin, int rows, uint16_t* a_lds,
                                           int a_stride) {
  constexpr int kPass = 8;
  const int pieces_per_row = p.K / 8;
  const int total = rows * pieces_per_row;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, (uint32_t)((int64_t)p.a_rows * p.lda * 2));
  for (int base = threadIdx.x; base < total; base += 256 * kPass) {
    u32x4_t v[kPass];
#pragma unroll
    for (int j = 0; j < kPass; ++j) {
      const int i = base + 256 * j;
      const int r = i / pieces_per_row, q = i - r * pieces_per_row;
      const int s = min(m_begin + r, p.a_rows - 1);
      const uint32_t off = i < total ? (uint32_t)(((int64_t)s * p.lda + q * 8) * 2) : kOob;
      v[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)off, 0, 0));
    }
#pragma unroll
    for (int j = 0; j < kPass; ++j) {
      const int i = base + 256 * j;
      if (i < total) {
        const int r = i / pieces_per_row, q = i - r * pieces_per_row;
        *reinterpret_cast<u32x4_t*>(a_lds + r * a_stride + q * 8) = v[j];
      }
    }
  }
}

// One 256-thread block of the bf16 weight-streaming projection: tile `id % p.grid_tiles`
// (dense rows [tile * rows_cap, ...)) x 16 output columns.  The 4 waves split K
// (128-wide chunks dealt round-robin); the partial tiles are added in a fixed
// order through LDS.  `lds` holds the staged rows (gemv_bf16_lds_bytes).
template <bool SWIGLU>
__device__ __forceinline__ void gemv_bf16_block(const GemvProblem& p, int id, int rows_cap, float limit,
                                                uint8_t* lds) {
  constexpr int NB = SWIGLU ? 2 : 1;
  __shared__ f32x4_t red[3][NB][64];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int tile = id % p.grid_tiles;
  const int n0 = (id / p.grid_tiles) * 16;
  if (n0 >= p.N) return;
  const int m_begin = tile * rows_cap;
  const int rows = min(m_begin + rows_cap, p.M) - m_begin;
  if (rows <= 0) return;

  Bf16View v;
  v.K = p.K;
  v.nchunks = (p.K + 127) / 128;
  const int row = n0 + col;
  v.w = make_rsrc(p.bh, (uint32_t)(p.b_expert_rows * p.K * 2));
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) v.row_off[nb] = (uint32_t)(row + nb * p.b_row_second) * (uint32_t)(p.K * 2);

  f32x4_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  {
    constexpr int step = 4 * kBf16Chunks;
    Bf16Batch<NB> b0, b1;
    bf16_load<NB>(b0, v, wave, grp);
    bf16_load<NB>(b1, v, wave + step, grp);
    uint16_t* a_lds = reinterpret_cast<uint16_t*>(lds);
    const int a_stride = p.K + kLdsPad;
    bf16_stage(p, m_begin, rows, a_lds, a_stride);
    __syncthreads();
    for (int c = wave; c < v.nchunks; c += 2 * step) {
      bf16_mma<NB>(b0, acc, a_lds, a_stride, rows, c, v, lane);
      if (c + step >= v.nchunks) break;
      bf16_load<NB>(b0, v, c + 2 * step, grp);
      bf16_mma<NB>(b1, acc, a_lds, a_stride, rows, c + step, v, lane);
      bf16_load<NB>(b1, v, c + 3 * step, grp);
    }
  }

  if (wave > 0) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) red[wave - 1][nb][lane] = acc[nb];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    f32x4_t s = acc[nb];
#pragma unroll
    for (int w = 0; w < 3; ++w) s += red[w][nb][lane];
    acc[nb] = s;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * grp + i;  // row of the MFMA tile held by this lane
    if (r < rows) {
      const float o = SWIGLU ? clamped_swiglu(acc[0][i], acc[NB - 1][i], limit) : acc[0][i];
      p.C[(int64_t)(m_begin + r) * p.ldc + n0 + col] = f32_to_bf16(o);
    }
  }
}

inline size_t gemv_bf16_lds_bytes(int rows_cap, int k_max) {
  return (size_t)rows_cap * (k_max + kLdsPad) * sizeof(uint16_t);
}

}  // namespace moe
