// Expert projections for few tokens (decode): weight streaming at HBM rate.
//
// With T <= 8 tokens an expert receives at most T rows (a token selects an
// expert at most once), so one tile per (expert, 16 output columns) reads
// each weight byte exactly once.  The layer's cost is then the weight bytes
// (MXFP4 routed experts, bf16 shared expert: Strata DEEPSEEK41 notes, opening
// paragraph and the "Where it goes" table), and the kernel is built to keep
// as many of them in flight as the register file allows and to spend as
// little ALU time per weight byte as possible:
//   * MXFP4 weights go straight into gfx950's block-scaled matrix
//     instruction (v_mfma_scale_f32_16x16x128_f8f6f4): E2M1 codes as the B
//     operand with their E8M0 byte as its per-lane scale, no dequantisation.
//     Activation rows are in two-term MXFP8 form (mx_device.h), converted
//     once by the routing kernel or, for the down projection, while staging;
//     each 128-wide chunk is two MFMAs (hi and lo);
//   * the bf16 shared expert uses v_mfma_f32_16x16x32_bf16 on bf16 rows;
//   * one weight format per launch keeps the register footprint of each
//     instantiation small;
//   * weights are read with raw buffer loads: a load past the end of the
//     expert's matrix returns zero without touching memory, so every load
//     is issued unconditionally and the compiler can wait on exactly the
//     batch it needs (vmcnt counts stay precise);
//   * the 4 waves of a block split K (128-wide chunks dealt round-robin) and
//     each wave streams its chunks in double-buffered batches; the first two
//     batches are issued before the activation rows are staged, so staging
//     hides under the weight latency.
// Rows >= T of the 16-row MFMA tile are zero and are never read or written.
// The 4 partial tiles are added in a fixed order through LDS; the epilogue
// applies the clamped SwiGLU (gate/up) or stores bf16 (down).
#include "moe_device.h"
#include "moe_internal.h"
#include "mx_device.h"

namespace moe {

namespace {

constexpr int kLdsPad = 8;  // bf16 elements of padding per staged bf16 row

// Weights of one 128-wide K chunk for this lane, as loaded.
struct Fp4Chunk {
  u32x4_t q;
  uint32_t s;
};
struct Bf16Chunk {
  u32x4_t h[4];
};

template <bool FP4, int NB>
struct Batch;
template <int NB>
struct Batch<true, NB> {
  static constexpr int kChunks = 5;
  Fp4Chunk c[kChunks][NB];
};
template <int NB>
struct Batch<false, NB> {
  static constexpr int kChunks = 2;
  Bf16Chunk c[kChunks][NB];
};

// Per-lane addressing of one problem's weight rows.
struct WeightView {
  __amdgpu_buffer_rsrc_t q, s;  // codes and scales (MXFP4) or bf16 values (q)
  uint32_t row_off[2];          // byte offset of this lane's row(s) in q
  uint32_t srow_off[2];         // byte offset of this lane's row(s) in s
  int K, nchunks;
};

template <bool FP4, int NB>
__device__ __forceinline__ void load_batch(Batch<FP4, NB>& b, const WeightView& v, int first_chunk, int grp) {
  constexpr int C = Batch<FP4, NB>::kChunks;
#pragma unroll
  for (int u = 0; u < C; ++u) {
    const int c = first_chunk + 4 * u;
    const int k0 = c * 128 + grp * 32;
    const bool ok = c < v.nchunks && k0 < v.K;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if constexpr (FP4) {
        const uint32_t qo = ok ? v.row_off[nb] + (uint32_t)(k0 / 2) : kOob;
        const uint32_t so = ok ? v.srow_off[nb] + (uint32_t)(k0 / 32) : kOob;
        b.c[u][nb].q = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(v.q, (int)qo, 0, 0));
        b.c[u][nb].s = __builtin_amdgcn_raw_buffer_load_b8(v.s, (int)so, 0, 0);
      } else {
        const uint32_t ho = ok ? v.row_off[nb] + (uint32_t)(k0 * 2) : kOob;
#pragma unroll
        for (int s = 0; s < 4; ++s)
          b.c[u][nb].h[s] =
              __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(v.q, (int)ho, 16 * s, 0));
      }
    }
  }
}

template <bool FP4, int NB>
__device__ __forceinline__ void mma_batch(const Batch<FP4, NB>& b, f32x4_t (&acc)[NB], const uint8_t* lds,
                                          int rows, int first_chunk, const WeightView& v, int lane) {
  constexpr int C = Batch<FP4, NB>::kChunks;
  const int col = lane & 15, grp = lane >> 4;
#pragma unroll
  for (int u = 0; u < C; ++u) {
    const int c = first_chunk + 4 * u;
    if (c >= v.nchunks) break;  // wave-uniform; no loads below
    if constexpr (FP4) {
      const int kb = c * 128;
      const uint8_t* row = lds + col * mx_row_bytes(v.K);
      const bool r_ok = col < rows;
      const bool h0 = r_ok && kb + 16 * grp < v.K, h1 = r_ok && kb + 64 + 16 * grp < v.K;
      const u32x4_t z = u32x4_t{0u, 0u, 0u, 0u};
      const u32x4_t a0 = h0 ? *reinterpret_cast<const u32x4_t*>(row + kb + 16 * grp) : z;
      const u32x4_t a1 = h1 ? *reinterpret_cast<const u32x4_t*>(row + kb + 64 + 16 * grp) : z;
      const u32x4_t l0 = h0 ? *reinterpret_cast<const u32x4_t*>(row + v.K + kb + 16 * grp) : z;
      const u32x4_t l1 = h1 ? *reinterpret_cast<const u32x4_t*>(row + v.K + kb + 64 + 16 * grp) : z;
      const int sa = (r_ok && kb + 32 * grp < v.K) ? (int)row[2 * v.K + kb / 32 + grp] : 127;
      const i32x8_t ahi = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
      const i32x8_t alo = {(int)l0[0], (int)l0[1], (int)l0[2], (int)l0[3], (int)l1[0], (int)l1[1], (int)l1[2], (int)l1[3]};
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int sb = (int)b.c[u][nb].s;
        acc[nb] = mfma_mx(ahi, b.c[u][nb].q, sa, sb, acc[nb]);
        acc[nb] = mfma_mx(alo, b.c[u][nb].q, sa, sb, acc[nb]);
      }
    } else {
      const uint16_t* a_lds = reinterpret_cast<const uint16_t*>(lds);
      const int a_stride = v.K + kLdsPad;
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
        for (int s = 0; s < 4; ++s)
          acc[nb] = mfma_16x16x32(a[s], __builtin_bit_cast(bf16x8_t, b.c[u][nb].h[s]), acc[nb]);
      }
    }
  }
}

// Source row of A for tile row r.
__device__ __forceinline__ int a_source_row(const GemvProblem& p, int m_begin, int r) {
  int s = p.gather ? p.gather[m_begin + r] / p.gather_div : m_begin + r;
  return min(max(s, 0), p.a_rows - 1);
}

// MXFP8 staging.  Pre-converted rows (p.amx) are copied; bf16 rows (p.A)
// are converted, one thread per block of 32 values.  All loads of a pass
// are issued before any conversion or store.
__device__ __forceinline__ void stage_rows_mx(const GemvProblem& p, int m_begin, int rows, uint8_t* lds) {
  const int K = p.K, stride = mx_row_bytes(K);
  if (p.amx) {
    constexpr int kPass = 4;
    const int pieces = stride / 16;
    const int total = rows * pieces;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.amx, (uint32_t)((int64_t)p.a_rows * stride));
    for (int base = threadIdx.x; base < total; base += 256 * kPass) {
      u32x4_t v[kPass];
#pragma unroll
      for (int j = 0; j < kPass; ++j) {
        const int i = base + 256 * j;
        const int r = i / pieces, q = i - r * pieces;
        const uint32_t off =
            i < total ? (uint32_t)((int64_t)a_source_row(p, m_begin, r) * stride + 16 * q) : kOob;
        v[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)off, 0, 0));
      }
#pragma unroll
      for (int j = 0; j < kPass; ++j) {
        const int i = base + 256 * j;
        if (i < total) *reinterpret_cast<u32x4_t*>(lds + 16 * i) = v[j];  // rows are contiguous
      }
    }
    return;
  }
  constexpr int kPass = 2;
  const int nblk = K / 32;
  const int total = rows * nblk;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, (uint32_t)((int64_t)p.a_rows * p.lda * 2));
  for (int base = threadIdx.x; base < total; base += 256 * kPass) {
    u32x4_t v[kPass][4];
#pragma unroll
    for (int j = 0; j < kPass; ++j) {
      const int i = base + 256 * j;
      const int r = i / nblk, b = i - r * nblk;
      const int src = i < total ? a_source_row(p, m_begin, r) : 0;
      const uint32_t off = i < total ? (uint32_t)(((int64_t)src * p.lda + 32 * b) * 2) : kOob;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        v[j][q] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)off, 16 * q, 0));
    }
#pragma unroll
    for (int j = 0; j < kPass; ++j) {
      const int i = base + 256 * j;
      if (i >= total) break;
      const int r = i / nblk, b = i - r * nblk;
      float x[32];
      unpack_bf16x32(v[j], x);
      uint8_t* row = lds + r * stride;
      mx_convert_block(x, row + 32 * b, row + K + 32 * b, row + 2 * K + b);
    }
  }
}

// Stage the tile's bf16 activation rows in LDS.  All loads of a pass are
// issued before any store; out-of-range pieces read zero through the buffer.
__device__ __forceinline__ void stage_rows(const GemvProblem& p, int m_begin, int rows, uint16_t* a_lds,
                                           int a_stride) {
  constexpr int kPass = 8;
  const int pieces_per_row = p.K / 8;
  const int total = rows * pieces_per_row;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, (uint32_t)((int64_t)p.a_rows * p.lda * 2));
  int src_row[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) src_row[r] = r < rows ? a_source_row(p, m_begin, r) : 0;
  for (int base = threadIdx.x; base < total; base += 256 * kPass) {
    u32x4_t v[kPass];
#pragma unroll
    for (int j = 0; j < kPass; ++j) {
      const int i = base + 256 * j;
      const int r = i / pieces_per_row, q = i - r * pieces_per_row;
      int s = 0;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) s = (rr == r) ? src_row[rr] : s;
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

// This wave's share of K (chunks wave, wave+4, ...): batches b0/b1 were
// issued by the caller for the first two steps; each iteration multiplies
// one batch and refills it two steps ahead.  The loop body issues its loads
// unconditionally (past the end they read zero), so each wait covers
// exactly the batch about to be used.
template <bool FP4, int NB>
__device__ __forceinline__ void stream_rest(Batch<FP4, NB>& b0, Batch<FP4, NB>& b1, const WeightView& v,
                                            const uint8_t* lds, int rows, f32x4_t (&acc)[NB], int wave, int lane) {
  constexpr int C = Batch<FP4, NB>::kChunks;
  const int grp = lane >> 4;
  const int step = 4 * C;
  for (int c = wave; c < v.nchunks; c += 2 * step) {
    mma_batch<FP4, NB>(b0, acc, lds, rows, c, v, lane);
    if (c + step >= v.nchunks) break;
    load_batch<FP4, NB>(b0, v, c + 2 * step, grp);
    mma_batch<FP4, NB>(b1, acc, lds, rows, c + step, v, lane);
    load_batch<FP4, NB>(b1, v, c + 3 * step, grp);
  }
}

}  // namespace

// 1-D grid: problem 1's blocks first, then problem 0's, tile-major within
// each 16-column tile.  Both problems use the weight format FP4.
template <bool SWIGLU, bool FP4>
__global__ __launch_bounds__(256) void expert_gemv_kernel(GemvParams prm) {
  constexpr int NB = SWIGLU ? 2 : 1;
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  __shared__ f32x4_t red[3][NB][64];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  int id = blockIdx.x;
  const int first = prm.p[1].grid_tiles * prm.p[1].col_tiles;
  const int which = id < first ? 1 : 0;
  if (which == 0) id -= first;
  const GemvProblem& p = prm.p[which];
  const int tile = id % p.grid_tiles;
  const int n0 = (id / p.grid_tiles) * 16;
  if (n0 >= p.N) return;

  int e = 0, m_begin, m_end;
  if (p.tiles) {
    if (tile >= *p.tile_count) return;
    const GemmTile tl = p.tiles[tile];
    e = tl.e;
    m_begin = tl.m_begin;
    m_end = min(tl.m_end, tl.m_begin + prm.rows_cap);
  } else {
    m_begin = tile * prm.rows_cap;
    m_end = min(m_begin + prm.rows_cap, p.M);
  }
  const int rows = m_end - m_begin;
  if (rows <= 0) return;

  WeightView v;
  v.K = p.K;
  v.nchunks = (p.K + 127) / 128;
  const int row = n0 + col;
  if constexpr (FP4) {
    const uint32_t qbytes = (uint32_t)(p.b_expert_rows * (p.K / 2));
    const uint32_t sbytes = (uint32_t)(p.b_expert_rows * (p.K / 32));
    v.q = make_rsrc(p.bq + (int64_t)e * qbytes, qbytes);
    v.s = make_rsrc(p.bs + (int64_t)e * sbytes, sbytes);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      v.row_off[nb] = (uint32_t)(row + nb * p.b_row_second) * (uint32_t)(p.K / 2);
      v.srow_off[nb] = (uint32_t)(row + nb * p.b_row_second) * (uint32_t)(p.K / 32);
    }
  } else {
    const uint32_t hbytes = (uint32_t)(p.b_expert_rows * p.K * 2);
    v.q = make_rsrc(p.bh + (int64_t)e * p.b_expert_rows * p.K, hbytes);
    v.s = v.q;
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      v.row_off[nb] = (uint32_t)(row + nb * p.b_row_second) * (uint32_t)(p.K * 2);
      v.srow_off[nb] = 0;
    }
  }

  f32x4_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  {
    constexpr int C = Batch<FP4, NB>::kChunks;
    Batch<FP4, NB> b0, b1;
    load_batch<FP4, NB>(b0, v, wave, grp);
    load_batch<FP4, NB>(b1, v, wave + 4 * C, grp);
    if constexpr (FP4)
      stage_rows_mx(p, m_begin, rows, lds);
    else
      stage_rows(p, m_begin, rows, reinterpret_cast<uint16_t*>(lds), p.K + kLdsPad);
    __syncthreads();
    stream_rest<FP4, NB>(b0, b1, v, lds, rows, acc, wave, lane);
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
      const float o = SWIGLU ? clamped_swiglu(acc[0][i], acc[NB - 1][i], prm.limit) : acc[0][i];
      p.C[(int64_t)(m_begin + r) * p.ldc + n0 + col] = f32_to_bf16(o);
    }
  }
}

// LDS of one tile: T staged rows, bf16 or two-term MXFP8.
size_t gemv_lds_bytes(int rows_cap, int k_max, bool fp4) {
  return fp4 ? (size_t)rows_cap * mx_row_bytes(k_max) : (size_t)rows_cap * (k_max + kLdsPad) * sizeof(uint16_t);
}

hipError_t launch_expert_gemv(const GemvParams& prm, bool swiglu, bool fp4, hipStream_t stream) {
  int k_max = prm.p[0].K;
  if (prm.p[1].grid_tiles > 0 && prm.p[1].K > k_max) k_max = prm.p[1].K;
  const size_t shm = gemv_lds_bytes(prm.rows_cap, k_max, fp4);
  dim3 grid((unsigned)(prm.p[0].grid_tiles * prm.p[0].col_tiles + prm.p[1].grid_tiles * prm.p[1].col_tiles));
  if (grid.x == 0) return hipSuccess;
  if (swiglu && fp4)
    hipLaunchKernelGGL((expert_gemv_kernel<true, true>), grid, dim3(256), shm, stream, prm);
  else if (swiglu)
    hipLaunchKernelGGL((expert_gemv_kernel<true, false>), grid, dim3(256), shm, stream, prm);
  else if (fp4)
    hipLaunchKernelGGL((expert_gemv_kernel<false, true>), grid, dim3(256), shm, stream, prm);
  else
    hipLaunchKernelGGL((expert_gemv_kernel<false, false>), grid, dim3(256), shm, stream, prm);
  return hipGetLastError();
}

}  // namespace moe
