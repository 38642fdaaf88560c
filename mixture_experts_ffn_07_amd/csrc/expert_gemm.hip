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

int expert_gemm_mt(int64_t n_rows, int n_groups) {
  // rows per group on average decides the row-tile height
  const int64_t avg = n_groups > 0 ? (n_rows + n_groups - 1) / n_groups : n_rows;
  return avg > 16 ? 4 : 1;
}

template <bool SWIGLU, bool FP4>
static void launch_t(const GemmParams& p, int mt, dim3 grid, hipStream_t stream) {
  if (mt == 4)
    hipLaunchKernelGGL((expert_gemm_kernel<4, SWIGLU, FP4>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((expert_gemm_kernel<1, SWIGLU, FP4>), grid, dim3(256), 0, stream, p);
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
