// Grouped expert GEMMs of the MoE FFN layer on gfx950 matrix cores.
//
// One kernel template serves the routed experts (MXFP4 weights: E2M1 codes
// with an E8M0 scale per 32 elements, Strata DEEPSEEK41 notes: "the experts
// as MXFP4") and the shared expert (bf16 weights), both projections:
//   gate/up: h = silu(min(x W_g^T, L)) * clamp(x W_u^T, -L, L)   (swiglu_limit,
//            DeepseekV41Config), gate rows 0..I-1 and up rows I..2I-1 of the
//            [2I][H] weight; one block computes matching gate and up columns
//            so the activation is applied in the epilogue;
//   down:    o = h W_d^T.
//
// Block = 4 waves, 16 output columns, up to 16*MT rows of one expert.  The
// 4 waves split K (128-wide chunks dealt round-robin) and add their fp32
// partial tiles through LDS in a fixed order.  MXFP4 weights are expanded to
// bf16 in registers (one v_cvt_scalef32_pk_bf16_fp4 per 2 elements, exact)
// and multiplied on v_mfma_f32_16x16x32_bf16 with fp32 accumulation.
//
// K layout within a 128-wide chunk: lane group g = lane/16 owns K offsets
// [32g, 32g+32), exactly one E8M0 block, read as one 16-byte load of codes
// (or 64 bytes of bf16); MFMA step s uses its elements 8s..8s+7 for both
// operands, which permutes K identically on A and B.
#include "moe_device.h"
#include "moe_internal.h"
#include "mx_device.h"

namespace moe {

template <int MT, bool SWIGLU, bool FP4>
__global__ __launch_bounds__(256) void expert_gemm_kernel(GemmParams p) {
  constexpr int NB = SWIGLU ? 2 : 1;
  constexpr int U = 2;  // chunks loaded ahead per wave per batch
  __shared__ f32x4_t red[3][MT][NB][64];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;

  int e = 0, m_begin, m_end;
  if (p.tiles) {
    if ((int)blockIdx.x >= *p.tile_count) return;
    const GemmTile tl = p.tiles[blockIdx.x];
    e = tl.e;
    m_begin = tl.m_begin;
    m_end = tl.m_end;
  } else {
    m_begin = blockIdx.x * 16 * MT;
    m_end = min(m_begin + 16 * MT, p.M);
  }
  const int n0 = blockIdx.y * 16;
  const int K = p.K;

  // A row of each m-subtile for this lane
  const uint16_t* arow[MT];
  bool aok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int r = m_begin + 16 * mt + col;
    aok[mt] = r < m_end;
    int src = 0;
    if (aok[mt]) src = p.gather ? min(max(p.gather[r] / p.gather_div, 0), p.a_rows - 1) : r;
    arow[mt] = p.A + (int64_t)src * p.lda;
  }
  // B rows of this lane: output column n0 + col (and its up row)
  const uint8_t* qrow[NB];
  const uint8_t* srow[NB];
  const uint16_t* hrow[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int64_t brow = (int64_t)e * p.b_expert_rows + n0 + col + nb * p.b_row_second;
    if (FP4) {
      qrow[nb] = p.bq + brow * (K / 2);
      srow[nb] = p.bs + brow * (K / 32);
    } else {
      hrow[nb] = p.bh + brow * K;
    }
  }

  f32x4_t acc[MT][NB];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[mt][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nchunks = (K + 127) / 128;
  for (int c0 = wave; c0 < nchunks; c0 += 4 * U) {
    // ---- loads for U chunks
    u32x4_t q[U][NB];
    uint32_t sc[U][NB];
    bf16x8_t bh[U][NB][4];
    bf16x8_t a[U][MT][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = c0 + 4 * u;
      const int k0 = c * 128 + grp * 32;
      const bool kok = c < nchunks && k0 < K;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        if (FP4) {
          if (kok) {
            q[u][nb] = *reinterpret_cast<const u32x4_t*>(qrow[nb] + k0 / 2);
            sc[u][nb] = srow[nb][k0 / 32];
          } else {
            q[u][nb] = u32x4_t{0u, 0u, 0u, 0u};
            sc[u][nb] = 127u;
          }
        } else {
#pragma unroll
          for (int s = 0; s < 4; ++s)
            bh[u][nb][s] = kok ? reinterpret_cast<const bf16x8_t*>(hrow[nb] + k0)[s] : zero_bf16x8();
        }
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          a[u][mt][s] = (kok && aok[mt]) ? reinterpret_cast<const bf16x8_t*>(arow[mt] + k0)[s] : zero_bf16x8();
      }
    }
    // ---- dequantise and multiply
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        bf16x8_t b[4];
        if (FP4) {
          const float scale = e8m0_scale_operand(sc[u][nb]);
#pragma unroll
          for (int s = 0; s < 4; ++s) b[s] = dequant_fp4x8(q[u][nb][s], scale);
        } else {
#pragma unroll
          for (int s = 0; s < 4; ++s) b[s] = bh[u][nb][s];
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) acc[mt][nb] = mfma_16x16x32(a[u][mt][s], b[s], acc[mt][nb]);
      }
    }
  }

  // ---- fixed-order reduction of the 4 waves' partial tiles
  if (wave > 0) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) red[wave - 1][mt][nb][lane] = acc[mt][nb];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      f32x4_t v = acc[mt][nb];
#pragma unroll
      for (int w = 0; w < 3; ++w) v += red[w][mt][nb][lane];
      acc[mt][nb] = v;
    }
  }
  // ---- epilogue: lane holds rows 4*grp + i of each m-subtile, column n0 + col
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = m_begin + 16 * mt + 4 * grp + i;
      if (r < m_end) {
        float v;
        if (SWIGLU)
          v = clamped_swiglu(acc[mt][0][i], acc[mt][NB - 1][i], p.limit);
        else
          v = acc[mt][0][i];
        p.C[(int64_t)r * p.ldc + n0 + col] = f32_to_bf16(v);
      }
    }
  }
}

// Tiled variant for tiles of up to 128 rows (many tokens per expert): the
// block's activation tile (128 rows x 128 K, bf16) is staged in LDS once per
// K chunk and shared by its 4 waves; wave w owns 32 output columns (and, for
// gate/up, the matching up columns): up to 8 x 4 MFMA tiles of 16x16, the
// row tiles past the tile's rows skipped.  Tiles of 128 rows keep an
// expert's rows in one tile at ~64 tokens per expert, so its weights are
// streamed once.  Weights are read once per block from HBM and dequantised
// in registers; the next chunk's weights and activation tile (double-
// buffered in LDS) load while the current one is multiplied.
// rows per tile: 128 with MXFP4 weights, 64 with bf16 weights (dense rows,
// whose larger weight registers leave room for fewer accumulators)
template <bool FP4>
constexpr int tiled_m() { return FP4 ? 8 : 4; }  // 16-row MFMA tiles per block
// output columns per wave: 32 for gate/up (plus the 32 matching up columns), 64 for down
template <bool SWIGLU>
constexpr int tiled_cols_per_wave() { return SWIGLU ? 32 : 64; }
constexpr int kTiledLdsStride = 128 + 8;  // bf16 elements per staged row (16 bytes of padding)

template <bool SWIGLU, bool FP4>
struct TiledB {
  // 4 column tiles of 16 rows: for gate/up, tiles 0-1 are gate columns and
  // 2-3 the matching up columns
  u32x4_t q[4][FP4 ? 1 : 4];
  uint32_t s[4];
};

template <bool SWIGLU, bool FP4>
__device__ __forceinline__ void tiled_load_b(TiledB<SWIGLU, FP4>& b, const GemmParams& p, int e, int n0w, int col,
                                             int grp, int c, int nchunks) {
  const int K = p.K;
  const int k0 = c * 128 + grp * 32;
  const bool ok = c < nchunks && k0 < K;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // column tile j: gate/up -> (j < 2 ? gate : up) columns n0w + 16 (j % 2); down -> n0w + 16 j
    const int ncol = SWIGLU ? n0w + 16 * (j & 1) + col + (j >> 1) * p.b_row_second : n0w + 16 * j + col;
    const uint32_t r = (uint32_t)ncol;  // row within the expert's matrix (past its end reads zero)
    if constexpr (FP4) {
      const uint32_t qb = (uint32_t)(p.b_expert_rows * (K / 2)), sb = (uint32_t)(p.b_expert_rows * (K / 32));
      const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.bq + (int64_t)e * qb, qb);
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.bs + (int64_t)e * sb, sb);
      b.q[j][0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                                  rq, (int)(ok ? r * (uint32_t)(K / 2) + (uint32_t)(k0 / 2) : kOob), 0, 0));
      b.s[j] = __builtin_amdgcn_raw_buffer_load_b8(rs, (int)(ok ? r * (uint32_t)(K / 32) + (uint32_t)(k0 / 32) : kOob),
                                                    0, 0);
    } else {
      const uint32_t hb = (uint32_t)(p.b_expert_rows * K * 2);
      const __amdgpu_buffer_rsrc_t rh = make_rsrc(p.bh + (int64_t)e * p.b_expert_rows * K, hb);
      const uint32_t off = ok ? (r * (uint32_t)K + (uint32_t)k0) * 2u : kOob;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        b.q[j][q] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rh, (int)off, 16 * q, 0));
      b.s[j] = 0;
    }
  }
}

template <bool SWIGLU, bool FP4>
__global__ __launch_bounds__(256, 2) void expert_gemm_tiled_kernel(GemmParams p) {
  constexpr int kTiledM = tiled_m<FP4>();
  constexpr int kTiledRows = 16 * kTiledM;
  __shared__ __attribute__((aligned(16))) uint16_t a_lds[2][kTiledRows * kTiledLdsStride];
  __shared__ int32_t src_rows[kTiledRows];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;

  int e = 0, m_begin, m_end;
  if (p.tiles) {
    if ((int)blockIdx.x >= *p.tile_count) return;
    const GemmTile tl = p.tiles[blockIdx.x];
    e = tl.e;
    m_begin = tl.m_begin;
    m_end = min(tl.m_end, tl.m_begin + kTiledRows);
  } else {
    m_begin = blockIdx.x * kTiledRows;
    m_end = min(m_begin + kTiledRows, p.M);
  }
  const int rows = m_end - m_begin;
  const int K = p.K, nchunks = (K + 127) / 128;
  // output columns of this wave: [n0w, n0w + 32) (and the up columns for gate/up)
  constexpr int CW = tiled_cols_per_wave<SWIGLU>();
  const int n0w = blockIdx.y * 4 * CW + wave * CW;
  const bool n_ok = n0w < p.N;

  for (int r = threadIdx.x; r < kTiledRows; r += blockDim.x) {
    int src = 0;
    if (r < rows) src = p.gather ? min(max(p.gather[m_begin + r] / p.gather_div, 0), p.a_rows - 1) : m_begin + r;
    src_rows[r] = src;
  }
  __syncthreads();

  // activation staging: 128 rows x 128 K bf16 = 2048 16-byte pieces, 8 per
  // thread (rows tid / 16 + 16 j, piece tid % 16); rows past the tile read zero
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, (uint32_t)((int64_t)p.a_rows * p.lda * 2));
  constexpr int kAP = kTiledRows * 16 / 256;
  const int a_q = threadIdx.x & 15, a_r0 = threadIdx.x >> 4;
  auto a_issue = [&](u32x4_t (&v)[kAP], int c) {
    const int k = c * 128 + 8 * a_q;
#pragma unroll
    for (int j = 0; j < kAP; ++j) {
      const int r = a_r0 + 16 * j;
      const bool ok = r < rows && c < nchunks && k < K;
      const uint32_t off = ok ? (uint32_t)(((int64_t)src_rows[r] * p.lda + k) * 2) : kOob;
      v[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)off, 0, 0));
    }
  };
  auto a_commit = [&](const u32x4_t (&v)[kAP], int buf) {
#pragma unroll
    for (int j = 0; j < kAP; ++j)
      *reinterpret_cast<u32x4_t*>(&a_lds[buf][(a_r0 + 16 * j) * kTiledLdsStride + 8 * a_q]) = v[j];
  };

  f32x4_t acc[kTiledM][4];
#pragma unroll
  for (int m = 0; m < kTiledM; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[m][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int m_tiles = (rows + 15) / 16;  // block-uniform

  // weights and the activation tile one chunk ahead (PD = 1: a 128-row
  // chunk keeps the matrix cores busy long enough to cover the load latency,
  // and the 4 x 32 accumulators leave no registers for a deeper pipeline)
  constexpr int PD = 1;
  TiledB<SWIGLU, FP4> b0, b1, b2;
  u32x4_t av[kAP];
  const int n_src = n_ok ? n0w : 0;
  a_issue(av, 0);
  tiled_load_b<SWIGLU, FP4>(b0, p, e, n_src, col, grp, n_ok ? 0 : nchunks, nchunks);
  if constexpr (PD == 2) tiled_load_b<SWIGLU, FP4>(b1, p, e, n_src, col, grp, n_ok ? 1 : nchunks, nchunks);
  a_commit(av, 0);
  __syncthreads();
  // multiply chunk c (activation tile in a_lds[buf], weights in bc): K step s
  // uses elements 8s..8s+7 of each lane group's 32
  auto multiply = [&](const TiledB<SWIGLU, FP4>& bc, int buf) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8_t bb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (FP4)
          bb[j] = dequant_fp4x8(bc.q[j][0][s], e8m0_scale_operand(bc.s[j]));
        else
          bb[j] = __builtin_bit_cast(bf16x8_t, bc.q[j][s]);
      }
#pragma unroll
      for (int m = 0; m < kTiledM; ++m) {
        if (m >= m_tiles) break;  // block-uniform
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
            &a_lds[buf][(16 * m + col) * kTiledLdsStride + 32 * grp + 8 * s]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[m][j] = mfma_16x16x32(a, bb[j], acc[m][j]);
      }
    }
  };
  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    a_issue(av, c + 1);
    if constexpr (PD == 2)
      tiled_load_b<SWIGLU, FP4>(b2, p, e, n_src, col, grp, n_ok ? c + 2 : nchunks, nchunks);
    else
      tiled_load_b<SWIGLU, FP4>(b1, p, e, n_src, col, grp, n_ok ? c + 1 : nchunks, nchunks);
    multiply(b0, buf);
    a_commit(av, buf ^ 1);
    b0 = b1;
    if constexpr (PD == 2) b1 = b2;
    __syncthreads();
  }

  if (!n_ok) return;
  // epilogue: lane holds rows 16m + 4*grp + i, column 16 jj + col of its 32
#pragma unroll
  for (int m = 0; m < kTiledM; ++m) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * m + 4 * grp + i;
      if (r < rows) {
        if constexpr (SWIGLU) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int n = n0w + 16 * jj + col;
            if (n < p.N)
              p.C[(int64_t)(m_begin + r) * p.ldc + n] = f32_to_bf16(clamped_swiglu(acc[m][jj][i], acc[m][jj + 2][i], p.limit));
          }
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int n = n0w + 16 * j + col;
            if (n < p.N) p.C[(int64_t)(m_begin + r) * p.ldc + n] = f32_to_bf16(acc[m][j][i]);
          }
        }
      }
    }
  }
}

int expert_gemm_mt(int64_t n_rows, int n_groups, bool fp4) {
  const int kTiledRows = 16 * (fp4 ? tiled_m<true>() : tiled_m<false>());
  // rows per group on average decides the row-tile height; 128-row tiles go
  // to the LDS-tiled kernel, which needs enough of them to fill the chip
  // (its blocks are 128 output columns wide)
  const int64_t avg = n_groups > 0 ? (n_rows + n_groups - 1) / n_groups : n_rows;
  const int64_t tiles = (n_rows + kTiledRows - 1) / kTiledRows;
  return (avg > 16 && tiles >= 16) ? kTiledRows / 16 : 1;
}

template <bool SWIGLU, bool FP4>
static void launch_t(const GemmParams& p, int mt, dim3 grid, hipStream_t stream) {
  if (mt == tiled_m<FP4>()) {
    // 128- or 64-row tiles: the LDS-tiled kernel, 4 waves x tiled_cols_per_wave columns per block
    const int cols = 4 * tiled_cols_per_wave<SWIGLU>();
    const dim3 g(grid.x, (unsigned)((p.N + cols - 1) / cols));
    hipLaunchKernelGGL((expert_gemm_tiled_kernel<SWIGLU, FP4>), g, dim3(256), 0, stream, p);
  } else {
    hipLaunchKernelGGL((expert_gemm_kernel<1, SWIGLU, FP4>), grid, dim3(256), 0, stream, p);
  }
}

hipError_t launch_expert_gemm(const GemmParams& p, bool swiglu, bool fp4, int mt, int64_t grid_tiles,
                              hipStream_t stream) {
  dim3 grid((unsigned)grid_tiles, (unsigned)(p.N / 16));
  if (swiglu && fp4)
    launch_t<true, true>(p, mt, grid, stream);
  else if (swiglu)
    launch_t<true, false>(p, mt, grid, stream);
  else if (fp4)
    launch_t<false, true>(p, mt, grid, stream);
  else
    launch_t<false, false>(p, mt, grid, stream);
  return hipGetLastError();
}

}  // namespace moe
