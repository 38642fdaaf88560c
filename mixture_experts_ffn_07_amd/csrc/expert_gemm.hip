// Grouped expert GEMMs of the MoE FFN layer on gfx950 matrix cores.
//
// One kernel template serves the routed experts (MXFP4 weights: E2M1 codes
// with an E8M0 scale per 32 elements, the routed experts' format in the Strata
// DEEPSEEK41 notes; or MXFP8: E4M3 codes, float8_e4m3fn in the MAX API's
// SUPPORTED_ENCODINGS, same scales) and the shared expert (bf16 weights),
// both projections:
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
// [32g, 32g+32), exactly one E8M0 block, read as one 16-byte load of MXFP4
// codes (32 bytes of MXFP8 codes, 64 bytes of bf16); MFMA step s uses its
// elements 8s..8s+7 for both operands, which permutes K identically on A and
// B.  MXFP8 codes are expanded with one v_cvt_scalef32_pk_bf16_fp8 per 2.
#include "moe_device.h"
#include "moe_internal.h"
#include "mx_device.h"

namespace moe {

template <int MT, bool SWIGLU, int BF>  // BF: WeightFormat of B
__global__ __launch_bounds__(256) void expert_gemm_kernel(GemmParams p) {
  constexpr bool FP4 = BF == kWMxfp4, FP8 = BF == kWMxfp8, MX = FP4 || FP8;
  constexpr int NQ = FP8 ? 2 : 1;  // 16-byte code loads per lane and block
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
    if (MX) {
      qrow[nb] = p.bq + brow * (FP4 ? K / 2 : K);
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
    u32x4_t q[U][NB][NQ];
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
        if (MX) {
#pragma unroll
          for (int j = 0; j < NQ; ++j)
            q[u][nb][j] = kok ? reinterpret_cast<const u32x4_t*>(qrow[nb] + (FP4 ? k0 / 2 : k0))[j]
                              : u32x4_t{0u, 0u, 0u, 0u};
          sc[u][nb] = kok ? (uint32_t)srow[nb][k0 / 32] : 127u;
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
          for (int s = 0; s < 4; ++s) b[s] = dequant_fp4x8(q[u][nb][0][s], scale);
        } else if (FP8) {
          const float scale = e8m0_scale_operand(sc[u][nb]);
#pragma unroll
          for (int s = 0; s < 4; ++s)
            b[s] = dequant_fp8x8(q[u][nb][s >> 1][2 * (s & 1)], q[u][nb][s >> 1][2 * (s & 1) + 1], scale);
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
// rows per tile: 128 with MXFP4 weights, 96 with MXFP8 and 64 with bf16
// weights (larger weight registers leave room for fewer accumulators at two
// blocks per CU without spilling)
template <int BF>
constexpr int tiled_m() { return BF == kWBf16 ? 4 : BF == kWMxfp8 ? 6 : 8; }  // 16-row MFMA tiles per block
// output columns per wave: 32 for gate/up (plus the 32 matching up columns), 64 for down
template <bool SWIGLU>
constexpr int tiled_cols_per_wave() { return SWIGLU ? 32 : 64; }
constexpr int kTiledLdsStride = 128 + 8;  // bf16 elements per staged row (16 bytes of padding)

template <bool SWIGLU, int BF>
struct TiledB {
  // 4 column tiles of 16 rows: for gate/up, tiles 0-1 are gate columns and
  // 2-3 the matching up columns; a lane's 32 K elements take 1 (MXFP4), 2
  // (MXFP8) or 4 (bf16) 16-byte vectors
  u32x4_t q[4][BF == kWMxfp4 ? 1 : BF == kWMxfp8 ? 2 : 4];
  uint32_t s[4];
};

// with_scale false: the scale bytes come from the kernel's scale groups
template <bool SWIGLU, int BF>
__device__ __forceinline__ void tiled_load_b(TiledB<SWIGLU, BF>& b, const GemmParams& p, int e, int n0w, int col,
                                             int grp, int c, int nchunks, bool with_scale = true) {
  constexpr bool FP4 = BF == kWMxfp4, FP8 = BF == kWMxfp8;
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
    } else if constexpr (FP8) {
      const uint32_t qb = (uint32_t)(p.b_expert_rows * K), sb = (uint32_t)(p.b_expert_rows * (K / 32));
      const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.bq + (int64_t)e * qb, qb);
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.bs + (int64_t)e * sb, sb);
      const uint32_t off = ok ? r * (uint32_t)K + (uint32_t)k0 : kOob;
#pragma unroll
      for (int q = 0; q < 2; ++q)
        b.q[j][q] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)off, 16 * q, 0));
      b.s[j] = with_scale ? __builtin_amdgcn_raw_buffer_load_b8(
                                rs, (int)(ok ? r * (uint32_t)(K / 32) + (uint32_t)(k0 / 32) : kOob), 0, 0)
                          : 0u;
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

template <bool SWIGLU, int BF>
__global__ __launch_bounds__(256, 2) void expert_gemm_tiled_kernel(GemmParams p) {
  constexpr bool FP4 = BF == kWMxfp4, FP8 = BF == kWMxfp8;
  constexpr int kTiledM = tiled_m<BF>();
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
  TiledB<SWIGLU, BF> b0, b1, b2;
  u32x4_t av[kAP];
  const int n_src = n_ok ? n0w : 0;
  // MXFP8, K a multiple of 512 (384): scale groups of sgs = 4 (3) chunks.  A
  // per-chunk byte load per lane and column tile touches 16 scattered rows
  // per instruction; instead lane group g < sgs loads the scale word of
  // chunk sgs G + g of its row once per group, and each chunk takes its byte
  // from that lane (ds_bpermute).
  const int sgs = FP8 ? (K % 512 == 0 ? 4 : K % 384 == 0 ? 3 : 0) : 0;  // block-uniform
  const bool groups = sgs != 0;
  uint32_t sw_cur[4] = {0u, 0u, 0u, 0u}, sw_next[4] = {0u, 0u, 0u, 0u};
  auto load_sw = [&](uint32_t (&sw)[4], int g) {
    const uint32_t sb = (uint32_t)(p.b_expert_rows * (K / 32));
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.bs + (int64_t)e * sb, sb);
    const int ci = sgs * g + grp;
    const bool ok = n_ok && grp < sgs && ci < nchunks;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int ncol = SWIGLU ? n_src + 16 * (j & 1) + col + (j >> 1) * p.b_row_second : n_src + 16 * j + col;
      sw[j] = __builtin_amdgcn_raw_buffer_load_b32(
          rs, (int)(ok ? (uint32_t)ncol * (uint32_t)(K / 32) + 4u * (uint32_t)ci : kOob), 0, 0);
    }
  };
  a_issue(av, 0);
  tiled_load_b<SWIGLU, BF>(b0, p, e, n_src, col, grp, n_ok ? 0 : nchunks, nchunks, !groups);
  if (groups) load_sw(sw_next, 0);
  if constexpr (PD == 2) tiled_load_b<SWIGLU, BF>(b1, p, e, n_src, col, grp, n_ok ? 1 : nchunks, nchunks);
  a_commit(av, 0);
  __syncthreads();
  // multiply chunk c (activation tile in a_lds[buf], weights in bc): K step s
  // uses elements 8s..8s+7 of each lane group's 32
  auto multiply = [&](const TiledB<SWIGLU, BF>& bc, int buf) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8_t bb[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (FP4)
          bb[j] = dequant_fp4x8(bc.q[j][0][s], e8m0_scale_operand(bc.s[j]));
        else if constexpr (FP8)
          bb[j] = dequant_fp8x8(bc.q[j][s >> 1][2 * (s & 1)], bc.q[j][s >> 1][2 * (s & 1) + 1],
                                e8m0_scale_operand(bc.s[j]));
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
    int sub = 0;
    if (groups) {
      sub = c % sgs;
      if (sub == 0) {  // block-uniform
#pragma unroll
        for (int j = 0; j < 4; ++j) sw_cur[j] = sw_next[j];
        load_sw(sw_next, c / sgs + 1);
      }
    }
    a_issue(av, c + 1);
    if constexpr (PD == 2)
      tiled_load_b<SWIGLU, BF>(b2, p, e, n_src, col, grp, n_ok ? c + 2 : nchunks, nchunks, !groups);
    else
      tiled_load_b<SWIGLU, BF>(b1, p, e, n_src, col, grp, n_ok ? c + 1 : nchunks, nchunks, !groups);
    if (groups) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b0.s[j] = ((uint32_t)__builtin_amdgcn_ds_bpermute(4 * (col + 16 * sub), (int)sw_cur[j]) >> (8 * grp)) & 0xffu;
    }
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

// ---------------------------------------------------------------- pipelined MXFP4 kernel
// Tiles of 128 rows, as in the LDS-tiled kernel, or 32 (32 gate + 32 up or 64
// output columns per column group, four column groups per block), with the
// operands brought into LDS by gfx950's global-to-LDS loads (16 bytes per
// lane, no registers) in a multi-stage pipeline, activations and weights
// SA - 1 and SB - 1 chunks ahead.  At ~64 rows per expert the routed
// projections read each expert's weights once; registers cannot hold the
// loads in flight such a stream needs, LDS can.  Per 128-wide K chunk and
// block: activation tile 128 x 256 B (bf16), weight codes 256 rows x 64 B,
// scale words 256 x 4 B (or a share of a scale group).
//
// LDS layouts are XOR-swizzled so that the 16 lanes reading one MFMA operand
// column hit 16 different 16-byte bank groups: activation row r keeps its
// 16-byte piece q in slot q ^ (r & 15); weight row b keeps piece q in slot
// q ^ ((b >> 2) & 3).  A load instruction writes its 64 lanes' pieces to 1 KB
// of consecutive LDS, so each lane fetches the global piece that belongs in
// its slot.
//
// Synchronisation: per chunk each wave issues a fixed number of loads (rows
// past the tile and chunks past K re-read valid addresses, results unused),
// so an exact vmcnt wait retires chunk c while later chunks stay in flight; a
// bare s_barrier (no fence, which would drain every load) then publishes the
// chunk to all waves.
// Global-to-LDS load of 16 (or 4) bytes per lane: lane l's bytes land at LDS
// byte address lds + 16 l (4 l).  Written in asm so that the compiler does not
// treat the LDS it writes as possibly read by every later LDS load (it would
// then wait for all loads in flight before each one); the kernel waits for
// these loads itself.  The loads write no registers; M0 carries the LDS
// address.  It is an input operand of the asm ("{m0}"), so the compiler
// writes M0 itself and knows the asm reads it; the asm opens with one wait
// state, which gfx950 needs between an SALU write of M0 and the load.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p);
}
__device__ __forceinline__ void load_lds16(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}
// 12 bytes per lane; lane l's bytes land at lds + 16 l (the fourth dword of
// each 16-byte slot is left alone; checked on gfx950).
__device__ __forceinline__ void load_lds12(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx3 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void load_lds4(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}

// XCD-aware block order for the pipelined kernels: a 1-D grid of
// ceil(tiles / 8) * 8 * col_blocks blocks; the hardware deals consecutive
// blocks round-robin to the 8 XCDs, so block b runs on XCD b % 8.  Each XCD
// takes the tiles t with t % 8 == its index and runs a tile's column blocks
// back to back, so the tile's activation rows, which every column block
// re-reads, stay in that XCD's L2 instead of crossing the fabric again.
struct PipeBlock {
  int tile, cb;
};
__device__ __forceinline__ PipeBlock pipe_block(int col_blocks) {
  const int b = (int)blockIdx.x, x = b & 7, q = b >> 3;
  return PipeBlock{8 * (q / col_blocks) + x, q % col_blocks};
}

template <int N>
struct IntC {
  static constexpr int value = N;
};

constexpr int kPipeAStage = 128 * 256;  // bytes
constexpr int kPipeBStage = 256 * 64;
constexpr int kPipeSStage = 256 * 4;

// The pipelined kernel has 8 waves: two waves per column group split
// every K chunk (wave w: column group w & 3, K half w >> 2, i.e. steps
// 2 (w >> 2) and 2 (w >> 2) + 1 of each lane group's 32 values), so each SIMD
// runs two waves and one's LDS and dependency stalls overlap the other's
// matrix work.  The halves' accumulators are added through LDS at the end.
// Per chunk each wave issues up to 4 activation loads, then 2 weight-code
// loads, and the waves that carry scales one scale load: a 4-byte word per
// weight row (K-half-0 waves, rows 64 w + lane), or with scale groups (below)
// a 16- or 12-byte load covering several chunks; the waits count these
// (pipe8_wait).  (Loads of 4 bytes or less fill 4-byte LDS slots per lane.)
//
// Tiles of AR = 128 rows serve many rows per expert.  At a few rows per
// expert the kernel streams weights with little matrix work per byte: 32-row
// tiles shrink the activation stages to 8 KB, and with two stages of each
// operand two blocks fit on a CU.
constexpr int kPipe8LoadsA = 4;  // activation loads per wave and chunk at 128-row tiles
constexpr int kPipe8LoadsB = 2;
template <int AR>
struct Pipe8Cfg {
  static constexpr int kA = 3;  // activation stages
  static constexpr int kB = 3;  // weight stages
};
template <>
struct Pipe8Cfg<32> {
  static constexpr int kA = 2;
  static constexpr int kB = 3;
};
// SG = 1 (whole scales): the block's scale bytes, 256 rows x K / 32, go to
// LDS once in the prologue (at most kPipeWholeS bytes), with two weight
// stages so that two blocks still fit on a CU.  Scale groups re-fetched each
// 128-byte scale line once per group (the weight stream evicts it in
// between): the 32-row down projection at 64 tokens moved 1.87 GB against
// 1.53 GB algorithmic, and went 312 -> 290 us this way (320 tokens: 500 -> 470 us).
constexpr int kPipeWholeS = 256 * 80;
template <int AR>
constexpr int pipe8_pool_bytes() {
  return Pipe8Cfg<AR>::kA * AR * 256 + Pipe8Cfg<AR>::kB * (kPipeBStage + kPipeSStage);
}
static_assert(pipe8_pool_bytes<128>() >= 4 * 128 * 256 && pipe8_pool_bytes<32>() >= 4 * 32 * 256,
              "the K-half reduction reuses 4 x AR x 256 B of the stage pool");
// Each iteration c of the main loop issues the stream with the shorter lead
// first (activations: chunk c + SA - 1, weights: chunk c + SB - 1, with SA
// and SB stages).  At the top of iteration c, chunk c of both streams must
// have landed: the wait allows as many loads in flight as were issued after
// the later of the two (la activation and lb weight loads per iteration and
// wave).  Chunks from the prologue are complete already (it ends with a full
// wait).
template <int SA, int SB>
constexpr int pipe8_wait(int la, int lb) {
  constexpr bool kAFirst = SA <= SB;
  const int c = 64;  // any iteration past the prologue
  const int ja = c - (SA - 1), jb = c - (SB - 1);
  const int oa = kAFirst ? 0 : 1, ob = 1 - oa;
  const bool a_later = ja > jb || (ja == jb && oa > ob);
  const int j_last = a_later ? ja : jb, o_last = a_later ? oa : ob;
  int n = 0;
  for (int j = j_last; j < c; ++j)
    for (int o = 0; o < 2; ++o)
      if (j > j_last || o > o_last) n += o == oa ? la : lb;
  return n;
}

// SG = 4 (K a multiple of 512) or 3 (K a multiple of 384): the scale bytes of
// SG chunks come as one 16- or 12-byte load per weight row instead of one
// 4-byte load per row and chunk.  Each such load touches 64 scattered rows,
// and their number per chunk counts (timing copies: one extra 4-byte load of
// that kind per wave and chunk cost 17%).  A scale group (SG chunks of 256
// rows, 16 bytes per row in LDS) is four parts of 64 rows; a ring holds three
// groups, and groups 0 and 1 come in the prologue.  SG = 4: wave 0 issues
// part c & 3 of group (c >> 2) + 2 in iteration c.  SG = 3: waves 0 and 1
// issue parts 2 (c % 3) + wave (mod 4) of group c / 3 + 2, so the third
// iteration repeats parts 0 and 1.  A group's parts land four or more
// iterations before its first chunk is read.  SG = 0: a 4-byte load per row
// and chunk by the K-half-0 waves.
template <bool SWIGLU, int AR, int SG = 0>
__global__ __launch_bounds__(512, AR == 32 ? 2 : 1) void expert_gemm_pipe8_kernel(GemmParams p, int n_tiles, int col_blocks) {
  constexpr bool kWhole = SG == 1;
  constexpr int kSA = Pipe8Cfg<AR>::kA, kSB = kWhole ? 2 : Pipe8Cfg<AR>::kB;
  constexpr bool kAFirst = kSA <= kSB;
  constexpr int kAStage = AR * 256;
  constexpr int kLoadsA = AR / 32;  // activation loads per wave and chunk at full tiles
  constexpr int MTMAX = AR / 16;
  static_assert(SG == 0 || SG == 1 || SG == 3 || SG == 4, "scale groups of 3 or 4 chunks, or whole");
  constexpr int kSGroup = 256 * 16;
  constexpr int kPool =
      kSA * kAStage + kSB * kPipeBStage + (kWhole ? kPipeWholeS : SG ? 3 * kSGroup : kSB * kPipeSStage);
  static_assert(kPool >= 4 * AR * 256, "the K-half reduction reuses 4 x AR x 256 B of the stage pool");
  // one pool: activation stages, weight-code stages, scale stages (the first
  // AR KB also hold the K-half reduction at the end)
  __shared__ __attribute__((aligned(16))) uint8_t pool[kPool];
  __shared__ int32_t src_rows[AR];
  auto a_lds = [&](int i) { return pool + i * kAStage; };
  auto b_lds = [&](int i) { return pool + kSA * kAStage + i * kPipeBStage; };
  auto s_lds = [&](int i) { return pool + kSA * kAStage + kSB * kPipeBStage + i * kPipeSStage; };
  auto sg_lds = [&](int g) { return pool + kSA * kAStage + kSB * kPipeBStage + (g % 3) * kSGroup; };
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int cg = wave & 3, kh = wave >> 2;

  const PipeBlock pb = pipe_block(col_blocks);
  if (pb.tile >= n_tiles) return;
  int e = 0, m_begin, m_end;
  if (p.tiles) {
    if (pb.tile >= *p.tile_count) return;
    const GemmTile tl = p.tiles[pb.tile];
    e = tl.e;
    m_begin = tl.m_begin;
    m_end = min(tl.m_end, tl.m_begin + AR);
  } else {
    m_begin = pb.tile * AR;
    m_end = min(m_begin + AR, p.M);
  }
  const int rows = m_end - m_begin;
  const int K = p.K, nchunks = K / 128;
  constexpr int CW = tiled_cols_per_wave<SWIGLU>();
  const int n0 = pb.cb * 4 * CW;
  for (int r = threadIdx.x; r < AR; r += 512) {
    int src = p.gather ? p.gather[m_begin + min(r, rows - 1)] / p.gather_div : m_begin + min(r, rows - 1);
    src_rows[r] = min(max(src, 0), p.a_rows - 1);
  }
  __syncthreads();

  // activation load t fills rows 4 i .. 4 i + 3, i = wave + 8 t, while 4 i <
  // a_rows_run: the tile's rows rounded up to the row tiles the main loop runs
  // (an even number of 16-row tiles), so that every wave issues MT / 2 of them
  // (rows past the tile re-read its last row); the waits count on that
  const int mt_run = min(2 * ((rows + 31) / 32), MTMAX);
  const int a_rows_run = 16 * mt_run;
  const uint8_t* a_src[kLoadsA];
#pragma unroll
  for (int t = 0; t < kLoadsA; ++t) {
    const int row = 4 * (wave + 8 * t) + (lane >> 4);
    const int piece = (lane & 15) ^ (row & 15);
    a_src[t] = reinterpret_cast<const uint8_t*>(p.A + (int64_t)src_rows[row] * p.lda) + 16 * piece;
  }
  auto brow_col = [&](int brow) {
    int c;
    if constexpr (SWIGLU) {
      const int w = brow >> 6, j = (brow >> 4) & 3, n = brow & 15;
      const int gc = min(n0 + 32 * w + 16 * (j & 1) + n, p.N - 1);
      c = gc + (j >> 1) * p.b_row_second;
    } else {
      c = min(n0 + brow, p.N - 1);
    }
    return (int64_t)c;
  };
  const uint8_t* bq_e = p.bq + (int64_t)e * p.b_expert_rows * (K / 2);
  const uint8_t* bs_e = p.bs + (int64_t)e * p.b_expert_rows * (K / 32);
  const uint8_t* b_src[kPipe8LoadsB];
#pragma unroll
  for (int t = 0; t < kPipe8LoadsB; ++t) {
    const int brow = 16 * (2 * wave + t) + (lane >> 2);
    const int piece = (lane & 3) ^ ((brow >> 2) & 3);
    b_src[t] = bq_e + brow_col(brow) * (K / 2) + 16 * piece;
  }
  const uint8_t* s_src = bs_e + brow_col(64 * (wave & 3) + lane) * (K / 32);
  // scale groups: row 64 i + lane of part i (i = 0..3)
  const uint8_t* sg_src[4];
  if constexpr (SG > 1) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sg_src[i] = bs_e + brow_col(64 * i + lane) * (K / 32);
  }
  const int n_groups = SG > 1 ? nchunks / SG : 1;
  // the waves that issue scale loads in the main loop (wave-uniform)
  const bool s_issuer = SG == 4 ? wave == 0 : SG == 3 ? wave < 2 : SG == 0 ? kh == 0 : false;

  auto issue_a = [&](int c) {
    const int cc = min(c, nchunks - 1);
    const uint32_t dst = lds_addr(a_lds(c % kSA) + 1024 * wave);
#pragma unroll
    for (int t = 0; t < kLoadsA; ++t)
      if (4 * (wave + 8 * t) < a_rows_run) load_lds16(a_src[t] + 256 * cc, dst + 8192 * t);  // wave-uniform
  };
  auto issue_b = [&](int c) {
    const int cc = min(c, nchunks - 1);
    const uint32_t dst = lds_addr(b_lds(c % kSB) + 2048 * wave);
#pragma unroll
    for (int t = 0; t < kPipe8LoadsB; ++t) load_lds16(b_src[t] + 64 * cc, dst + 1024 * t);
    if constexpr (SG == 0)
      if (kh == 0) load_lds4(s_src + 4 * cc, lds_addr(s_lds(c % kSB) + 256 * wave));  // wave-uniform
  };
  // part i of scale group g (groups past the end re-read the last one into a
  // ring slot no longer read)
  auto issue_sg = [&](int g, int i) {
    const int gg = min(g, n_groups - 1);
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      if (ii == i) {
        if constexpr (SG == 4)
          load_lds16(sg_src[ii] + 16 * gg, lds_addr(sg_lds(g) + 1024 * ii));
        else if constexpr (SG == 3)
          load_lds12(sg_src[ii] + 12 * gg, lds_addr(sg_lds(g) + 1024 * ii));
      }
    }
  };
  auto issue_sg_iter = [&](int c) {
    if constexpr (kWhole) {
    } else if constexpr (SG == 4) {
      if (s_issuer) issue_sg((c >> 2) + 2, c & 3);
    } else if constexpr (SG == 3) {
      if (s_issuer) issue_sg(c / 3 + 2, (2 * (c % 3) + wave) & 3);
    }
  };

  f32x4_t acc[MTMAX][4];
#pragma unroll
  for (int m = 0; m < MTMAX; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[m][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int m_tiles = (rows + 15) / 16;

#pragma unroll
  for (int c = 0; c < kSB - 1; ++c) issue_b(c);
#pragma unroll
  for (int c = 0; c < kSA - 1; ++c) issue_a(c);
  if constexpr (kWhole) {
    // the block's weight rows are one run of consecutive rows (n0 ..), so
    // their scale bytes are one contiguous range; a piece past the expert's
    // rows re-reads its first piece into LDS no one reads
    const int run_bytes = 256 * (K / 32);
    const int64_t avail = (int64_t)(p.N - n0) * (K / 32);
    const uint8_t* sbase = bs_e + (int64_t)n0 * (K / 32);
    for (int q0 = 16 * 64 * wave; q0 < run_bytes; q0 += 16 * 512) {
      const int off = q0 + 16 * lane;
      load_lds16(sbase + (off + 16 <= avail ? off : 0), lds_addr(pool + kSA * kAStage + kSB * kPipeBStage + q0));
    }
  } else if constexpr (SG != 0) {
    if (wave == 0) {  // wave-uniform
#pragma unroll
      for (int g = 0; g < 2; ++g)
#pragma unroll
        for (int i = 0; i < 4; ++i) issue_sg(g, i);
    }
  }
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");

  auto run = [&](auto mt_tag) {
    constexpr int MT = decltype(mt_tag)::value;
    for (int c = 0; c < nchunks; ++c) {
      // MT / 2 activation loads per wave, the weight codes, and the scale
      // load of the waves that issue one; a scale group for chunk c was
      // issued before chunk c's weight codes
      constexpr int kWait0 = pipe8_wait<kSA, kSB>(MT / 2, kPipe8LoadsB + 1);
      constexpr int kWait1 = pipe8_wait<kSA, kSB>(MT / 2, kPipe8LoadsB);
      static_assert(kWait0 < 64 && kWait1 < 64, "vmcnt holds at most 63");
      if (c > 0) {
        if (s_issuer)
          asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(kWait0) : "memory");
        else
          asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(kWait1) : "memory");
        asm volatile("s_barrier" ::: "memory");
      }
      const uint8_t* al = a_lds(c % kSA);
      const uint8_t* bl = b_lds(c % kSB);
      const uint8_t* sl = kWhole ? pool + kSA * kAStage + kSB * kPipeBStage + 4 * c
                          : SG ? sg_lds(c / (SG ? SG : 1)) + 4 * (c % (SG ? SG : 1))
                               : s_lds(c % kSB);
      const int kSRow = kWhole ? K / 32 : SG ? 16 : 4;  // scale bytes per row in LDS
      uint32_t q[4][2];
      float sc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int brow = 64 * cg + 16 * j + col;
        const uint2 v = *reinterpret_cast<const uint2*>(bl + 64 * brow + 16 * (grp ^ ((brow >> 2) & 3)) + 8 * kh);
        q[j][0] = v.x;
        q[j][1] = v.y;
        sc[j] = e8m0_scale_operand(sl[kSRow * brow + grp]);
      }
      auto read_a = [&](bf16x8_t (&a)[MT], int s4) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
          a[m] = *reinterpret_cast<const bf16x8_t*>(al + 256 * (16 * m + col) + 16 * ((4 * grp + s4) ^ col));
      };
      bf16x8_t a0[MT], a1[MT];
      read_a(a0, 2 * kh);
      if constexpr (kAFirst) {
        issue_a(c + kSA - 1);
        issue_b(c + kSB - 1);
        issue_sg_iter(c);
      } else {
        issue_b(c + kSB - 1);
        issue_sg_iter(c);
        issue_a(c + kSA - 1);
      }
      read_a(a1, 2 * kh + 1);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bf16x8_t bb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) bb[j] = dequant_fp4x8(q[j][h], sc[j]);
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[m][j] = mfma_16x16x32(h ? a1[m] : a0[m], bb[j], acc[m][j]);
      }
    }
  };
  if constexpr (MTMAX == 2) {
    run(IntC<2>{});
  } else {
    if (mt_run <= 2)
      run(IntC<2>{});
    else if (mt_run == 4)
      run(IntC<4>{});
    else if (mt_run == 6)
      run(IntC<6>{});
    else
      run(IntC<8>{});
  }
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");  // every load landed, LDS free

  // the K-half-1 waves hand their sums to the K-half-0 waves through LDS
  // (lane-major: element (m, j, i) of lane l at ((m * 4 + j) * 4 + i) * 256 + 4 l
  // within the column group's AR x 256 B)
  float* red = reinterpret_cast<float*>(pool) + cg * (AR * 64);  // 4 x AR x 256 B of the pool
  const int mtr = min(m_tiles, MTMAX);
  if (kh == 1) {
#pragma unroll
    for (int m = 0; m < MTMAX; ++m) {
      if (m >= mtr) break;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[((m * 4 + j) * 4 + i) * 64 + lane] = acc[m][j][i];
    }
  }
  __syncthreads();
  if (kh == 1) return;
#pragma unroll
  for (int m = 0; m < MTMAX; ++m) {
    if (m >= mtr) break;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[m][j][i] += red[((m * 4 + j) * 4 + i) * 64 + lane];
  }

  const int n0w = n0 + cg * CW;
#pragma unroll
  for (int m = 0; m < MTMAX; ++m) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * m + 4 * grp + i;
      if (r < rows) {
        if constexpr (SWIGLU) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int n = n0w + 16 * jj + col;
            if (n < p.N)
              p.C[(int64_t)(m_begin + r) * p.ldc + n] =
                  f32_to_bf16(clamped_swiglu(acc[m][jj][i], acc[m][jj + 2][i], p.limit));
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

// Wide form of the pipelined kernel: 512 weight rows per block, eight waves
// of 64 weight rows each (32 gate + 32 up or 64 output columns), every wave
// taking the whole 128-wide K chunk (no K halves, no reduction).  The
// pipelined kernels are bound by issuing their global-to-LDS loads; here a
// block loads its tile's activation rows once per 512 weight rows instead of
// per 256, so the loads per unit of work drop by a fifth.  Two stages each
// (activations 32 KB, weight codes 32 KB, scales 2 KB per stage).
constexpr int kWideA = 2, kWideB = 2;
constexpr int kWideBStage = 512 * 64, kWideSStage = 512 * 4;
constexpr int kWideLoadsB = 4;  // 16-byte weight-code loads per wave per chunk (+ one 4-byte scale load)
constexpr bool kWideAFirst = kWideA <= kWideB;
constexpr int wide_wait(int la, int lb) {
  const int c = 64;
  const int ja = c - (kWideA - 1), jb = c - (kWideB - 1);
  const int oa = kWideAFirst ? 0 : 1, ob = 1 - oa;
  const bool a_later = ja > jb || (ja == jb && oa > ob);
  const int j_last = a_later ? ja : jb, o_last = a_later ? oa : ob;
  int n = 0;
  for (int j = j_last; j < c; ++j)
    for (int o = 0; o < 2; ++o)
      if (j > j_last || o > o_last) n += o == oa ? la : lb;
  return n;
}

template <bool SWIGLU>
__global__ __launch_bounds__(512, 1) void expert_gemm_wide_kernel(GemmParams p, int n_tiles, int col_blocks) {
  __shared__ __attribute__((aligned(16))) uint8_t pool[kWideA * kPipeAStage + kWideB * kWideBStage + kWideB * kWideSStage];
  __shared__ int32_t src_rows[128];
  auto a_lds = [&](int i) { return pool + i * kPipeAStage; };
  auto b_lds = [&](int i) { return pool + kWideA * kPipeAStage + i * kWideBStage; };
  auto s_lds = [&](int i) { return pool + kWideA * kPipeAStage + kWideB * kWideBStage + i * kWideSStage; };
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;

  const PipeBlock pb = pipe_block(col_blocks);
  if (pb.tile >= n_tiles) return;
  int e = 0, m_begin, m_end;
  if (p.tiles) {
    if (pb.tile >= *p.tile_count) return;
    const GemmTile tl = p.tiles[pb.tile];
    e = tl.e;
    m_begin = tl.m_begin;
    m_end = min(tl.m_end, tl.m_begin + 128);
  } else {
    m_begin = pb.tile * 128;
    m_end = min(m_begin + 128, p.M);
  }
  const int rows = m_end - m_begin;
  const int K = p.K, nchunks = K / 128;
  constexpr int CW = tiled_cols_per_wave<SWIGLU>();
  const int n0 = pb.cb * 8 * CW;
  for (int r = threadIdx.x; r < 128; r += 512) {
    int src = p.gather ? p.gather[m_begin + min(r, rows - 1)] / p.gather_div : m_begin + min(r, rows - 1);
    src_rows[r] = min(max(src, 0), p.a_rows - 1);
  }
  __syncthreads();

  // activation loads as in the 8-wave kernel (MT / 2 per wave)
  const int mt_run = min(2 * ((rows + 31) / 32), 8);
  const int a_rows_run = 16 * mt_run;
  const uint8_t* a_src[kPipe8LoadsA];
#pragma unroll
  for (int t = 0; t < kPipe8LoadsA; ++t) {
    const int row = 4 * (wave + 8 * t) + (lane >> 4);
    const int piece = (lane & 15) ^ (row & 15);
    a_src[t] = reinterpret_cast<const uint8_t*>(p.A + (int64_t)src_rows[row] * p.lda) + 16 * piece;
  }
  auto brow_col = [&](int brow) {
    int c;
    if constexpr (SWIGLU) {
      const int w = brow >> 6, j = (brow >> 4) & 3, n = brow & 15;
      const int gc = min(n0 + 32 * w + 16 * (j & 1) + n, p.N - 1);
      c = gc + (j >> 1) * p.b_row_second;
    } else {
      c = min(n0 + brow, p.N - 1);
    }
    return (int64_t)c;
  };
  const uint8_t* bq_e = p.bq + (int64_t)e * p.b_expert_rows * (K / 2);
  const uint8_t* bs_e = p.bs + (int64_t)e * p.b_expert_rows * (K / 32);
  // weight-code load t of wave w fills weight rows 16 (4 w + t) .. + 15
  const uint8_t* b_src[kWideLoadsB];
#pragma unroll
  for (int t = 0; t < kWideLoadsB; ++t) {
    const int brow = 16 * (4 * wave + t) + (lane >> 2);
    const int piece = (lane & 3) ^ ((brow >> 2) & 3);
    b_src[t] = bq_e + brow_col(brow) * (K / 2) + 16 * piece;
  }
  const uint8_t* s_src = bs_e + brow_col(64 * wave + lane) * (K / 32);

  auto issue_a = [&](int c) {
    const int cc = min(c, nchunks - 1);
    const uint32_t dst = lds_addr(a_lds(c % kWideA) + 1024 * wave);
#pragma unroll
    for (int t = 0; t < kPipe8LoadsA; ++t)
      if (4 * (wave + 8 * t) < a_rows_run) load_lds16(a_src[t] + 256 * cc, dst + 8192 * t);  // wave-uniform
  };
  auto issue_b = [&](int c) {
    const int cc = min(c, nchunks - 1);
    const uint32_t dst = lds_addr(b_lds(c % kWideB) + 4096 * wave);
#pragma unroll
    for (int t = 0; t < kWideLoadsB; ++t) load_lds16(b_src[t] + 64 * cc, dst + 1024 * t);
    load_lds4(s_src + 4 * cc, lds_addr(s_lds(c % kWideB) + 256 * wave));
  };

  f32x4_t acc[8][4];
#pragma unroll
  for (int m = 0; m < 8; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[m][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int c = 0; c < kWideB - 1; ++c) issue_b(c);
#pragma unroll
  for (int c = 0; c < kWideA - 1; ++c) issue_a(c);
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");

  auto run = [&](auto mt_tag) {
    constexpr int MT = decltype(mt_tag)::value;
    constexpr int kWait = wide_wait(MT / 2, kWideLoadsB + 1);
    for (int c = 0; c < nchunks; ++c) {
      if (c > 0) {
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(kWait) : "memory");
        asm volatile("s_barrier" ::: "memory");
      }
      const uint8_t* al = a_lds(c % kWideA);
      const uint8_t* bl = b_lds(c % kWideB);
      const uint8_t* sl = s_lds(c % kWideB);
      u32x4_t q[4];
      float sc[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int brow = 64 * wave + 16 * j + col;
        q[j] = *reinterpret_cast<const u32x4_t*>(bl + 64 * brow + 16 * (grp ^ ((brow >> 2) & 3)));
        sc[j] = e8m0_scale_operand(sl[4 * brow + grp]);
      }
      auto read_a = [&](bf16x8_t (&a)[MT], int s4) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
          a[m] = *reinterpret_cast<const bf16x8_t*>(al + 256 * (16 * m + col) + 16 * ((4 * grp + s4) ^ col));
      };
      bf16x8_t a0[MT], a1[MT];
      read_a(a0, 0);
      if constexpr (kWideAFirst) {
        issue_a(c + kWideA - 1);
        issue_b(c + kWideB - 1);
      } else {
        issue_b(c + kWideB - 1);
        issue_a(c + kWideA - 1);
      }
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        // the next K step's activations load while this one multiplies
        if (s4 < 3) read_a((s4 & 1) ? a0 : a1, s4 + 1);
        bf16x8_t bb[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) bb[j] = dequant_fp4x8(q[j][s4], sc[j]);
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[m][j] = mfma_16x16x32((s4 & 1) ? a1[m] : a0[m], bb[j], acc[m][j]);
      }
    }
  };
  if (mt_run <= 2)
    run(IntC<2>{});
  else if (mt_run == 4)
    run(IntC<4>{});
  else if (mt_run == 6)
    run(IntC<6>{});
  else
    run(IntC<8>{});
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");  // every load landed before the block ends

  const int n0w = n0 + wave * CW;
#pragma unroll
  for (int m = 0; m < 8; ++m) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * m + 4 * grp + i;
      if (r < rows) {
        if constexpr (SWIGLU) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int n = n0w + 16 * jj + col;
            if (n < p.N)
              p.C[(int64_t)(m_begin + r) * p.ldc + n] =
                  f32_to_bf16(clamped_swiglu(acc[m][jj][i], acc[m][jj + 2][i], p.limit));
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

// ---------------------------------------------------------------- dense bf16 pipelined kernel
// The shared expert at many tokens: a dense bf16 GEMM, rows [0, M) of A
// against one bf16 weight matrix.  Tiles of 128 rows x 256 weight rows (32
// gate + 32 up or 64 output columns per column group, four column groups),
// eight waves: column group w & 3, row half w >> 2 (64 rows, 4 x 4 MFMA
// tiles per wave).  Both operands reach LDS through the global-to-LDS loads
// in chunks of 32 K (64 bytes per row), DS stages ahead; every row of both
// stages keeps its 16-byte piece q in slot q ^ ((r >> 2) & 3), so the 16
// lanes reading one MFMA operand column hit 16 different bank groups.  Per
// chunk each wave issues one activation load (16 rows) and two weight loads
// (32 rows), whatever the tile's size (rows past M and columns past N re-read
// the last valid ones, results unused), so the waits are constants.
// F32: fp32 outputs in slices (blockIdx.y = z * k_slices + k-part): slice z
// multiplies the weight matrix bh + z * b_slice_stride over the k-part's range
// of K chunks and writes Cf + slice * c_slice_stride (the router's three-term
// split logits, summed later).
template <int DS>
constexpr int dense_pool_bytes() {
  return DS * (128 + 256) * 64;
}
template <bool SWIGLU, int DS, bool F32 = false>
__global__ __launch_bounds__(512, DS <= 3 ? 2 : 1) void expert_gemm_dense_kernel(GemmParams p, int n_tiles,
                                                                                  int col_blocks) {
  static_assert(!(F32 && SWIGLU), "fp32 slices are plain products");
  constexpr int MR = 4;             // 16-row MFMA tiles per wave
  constexpr int kRows = 32 * MR;    // block tile rows
  constexpr int kALoads = MR / 4;   // activation loads (16 rows each) per wave and chunk
  __shared__ __attribute__((aligned(16))) uint8_t pool[dense_pool_bytes<DS>()];
  auto a_lds = [&](int i) { return pool + i * (kRows * 64); };
  auto b_lds = [&](int i) { return pool + DS * (kRows * 64) + i * (256 * 64); };
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int cg = wave & 3, mh = wave >> 2;

  const PipeBlock pb = pipe_block(col_blocks);
  if (pb.tile >= n_tiles) return;
  const int m_begin = pb.tile * kRows;
  const int rows = min(kRows, p.M - m_begin);
  const int K = p.K;
  int c_lo = 0, nchunks = K / 32;
  const uint16_t* bh = p.bh;
  if constexpr (F32) {
    // the host sizes k_slices so that every k-part holds at least one chunk
    const int z = (int)blockIdx.y / p.k_slices, kp = (int)blockIdx.y % p.k_slices;
    const int per = (nchunks + p.k_slices - 1) / p.k_slices;
    c_lo = kp * per;
    nchunks = min(nchunks - c_lo, per);
    bh += z * p.b_slice_stride;
  }
  constexpr int CW = tiled_cols_per_wave<SWIGLU>();
  const int n0 = pb.cb * 4 * CW;

  // load sources: 16 rows x 64 bytes per instruction, lane l fills slot
  // l & 3 of row l >> 2 of its group
  const int lrow = lane >> 2;
  const uint8_t* a_src[kALoads];
#pragma unroll
  for (int t = 0; t < kALoads; ++t) {
    const int r = 16 * (wave + 8 * t) + lrow;
    const int q = (lane & 3) ^ ((r >> 2) & 3);
    const int src = min(m_begin + r, p.M - 1);
    a_src[t] = reinterpret_cast<const uint8_t*>(p.A + (int64_t)src * p.lda) + 64 * c_lo + 16 * q;
  }
  auto brow_col = [&](int brow) {
    int c;
    if constexpr (SWIGLU) {
      const int w = brow >> 6, j = (brow >> 4) & 3, n = brow & 15;
      const int gc = min(n0 + 32 * w + 16 * (j & 1) + n, p.N - 1);
      c = gc + (j >> 1) * p.b_row_second;
    } else {
      c = min(n0 + brow, p.N - 1);
    }
    return (int64_t)c;
  };
  const uint8_t* b_src[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int brow = 16 * (2 * wave + t) + lrow;
    const int q = (lane & 3) ^ ((brow >> 2) & 3);
    b_src[t] = reinterpret_cast<const uint8_t*>(bh + brow_col(brow) * K) + 64 * c_lo + 16 * q;
  }
  auto issue = [&](int c) {
    const int cc = min(c, nchunks - 1);
#pragma unroll
    for (int t = 0; t < kALoads; ++t) load_lds16(a_src[t] + 64 * cc, lds_addr(a_lds(c % DS) + 1024 * (wave + 8 * t)));
    const uint32_t dst = lds_addr(b_lds(c % DS) + 2048 * wave);
#pragma unroll
    for (int t = 0; t < 2; ++t) load_lds16(b_src[t] + 64 * cc, dst + 1024 * t);
  };

  f32x4_t acc[MR][4];
#pragma unroll
  for (int m = 0; m < MR; ++m)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[m][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // one chunk's MFMA operands: this wave's MR row tiles and 4 column tiles
  struct Frag {
    bf16x8_t a[MR], b[4];
  };
  auto read_frags = [&](int c, Frag& f) {
    const uint8_t* al = a_lds(c % DS);
    const uint8_t* bl = b_lds(c % DS);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int br = 64 * cg + 16 * j + col;
      f.b[j] = *reinterpret_cast<const bf16x8_t*>(bl + 64 * br + 16 * (grp ^ ((br >> 2) & 3)));
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      const int ar = 16 * MR * mh + 16 * m + col;
      f.a[m] = *reinterpret_cast<const bf16x8_t*>(al + 64 * ar + 16 * (grp ^ ((ar >> 2) & 3)));
    }
  };
  auto mfmas = [&](const Frag& f) {
#pragma unroll
    for (int m = 0; m < MR; ++m)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[m][j] = mfma_16x16x32(f.a[m], f.b[j], acc[m][j]);
  };

#pragma unroll
  for (int c = 0; c < DS - 1; ++c) issue(c);
  asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
  // at the top of iteration c, chunk c was issued DS - 1 iterations earlier;
  // the loads of the DS - 2 iterations since then may stay in flight
  constexpr int kWait = (DS - 2) * (kALoads + 2);
  for (int c = 0; c < nchunks; ++c) {
    if (c > 0) {
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(kWait) : "memory");
      asm volatile("s_barrier" ::: "memory");
    }
    Frag f;
    read_frags(c, f);
    issue(c + DS - 1);
    mfmas(f);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load may land in LDS after the block ends

  const int n0w = n0 + cg * CW;
#pragma unroll
  for (int m = 0; m < MR; ++m) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * MR * mh + 16 * m + 4 * grp + i;
      if (r < rows) {
        if constexpr (SWIGLU) {
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int n = n0w + 16 * jj + col;
            if (n < p.N)
              p.C[(int64_t)(m_begin + r) * p.ldc + n] =
                  f32_to_bf16(clamped_swiglu(acc[m][jj][i], acc[m][jj + 2][i], p.limit));
          }
        } else if constexpr (F32) {
          float* cf = p.Cf + (int64_t)blockIdx.y * p.c_slice_stride + (int64_t)(m_begin + r) * p.ldc;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int n = n0w + 16 * j + col;
            if (n < p.N) cf[n] = acc[m][j][i];
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
// ---------------------------------------------------------------- dense bf16, whole rounds
// The shared expert from a few thousand rows: block tiles of 256 rows x NT
// weight rows, one block per CU, eight waves.  The widths give whole rounds
// of blocks at the layer's shapes, where the 256-column tiles of the kernel
// above leave a partial last round (4096 rows: 288 or 320 tiles for 256 CUs):
// NT = 288 for SwiGLU (144 h columns: 9 gate MFMA tiles, then their 9 up
// tiles) makes 16 column blocks of I = 2304, NT = 320 makes 16 of H = 5120,
// so 4096 rows give 16 x 16 tiles, one round.
// Waves, SwiGLU: rows 64 (w & 3) .. + 63; waves 0-3 take h tiles 0..4
// (10 MFMA column tiles), waves 4-7 h tiles 5..8 (8), so each SIMD, running
// waves w and w + 4, does 18 column tiles.  Otherwise: rows 128 (w >> 2) ..
// + 127 against column tiles 5 (w & 3) .. + 4.
// Operands come in chunks of KC = 64 K (128 bytes per row: a probe moved
// 1.6x the bytes per CU with 128-byte row pieces as with 64-byte ones) or 32
// K, by global-to-LDS loads, DS stages, XOR-swizzled.  A chunk's load
// instructions (1 KB each: 8 rows x 128 bytes, or 16 x 64) are dealt to the
// waves round-robin: waves below the remainder issue one more, and each
// wave's wait counts its own loads.
// MODE: what the block tile's weight rows are and what the epilogue writes
constexpr int kNtPlain = 0;   // 320 output columns, bf16
constexpr int kNtSwiglu = 1;  // 144 h columns (9 gate, then 9 up MFMA tiles), clamped SwiGLU, bf16
constexpr int kNtRouter = 2;  // 96 experts x the three bf16 terms of W_r (term t of expert tile u is MFMA
                              // tile 6 t + u), the terms added in fp32, written as fp32 partial logits
template <int MODE>
constexpr int dense_nt_cols() {
  return MODE == kNtPlain ? 320 : 288;
}
// KC: K per chunk, 32 (64-byte row pieces) or 64 (128-byte pieces)
template <int MODE, int DS, int KC>
constexpr int dense_nt_pool_bytes() {
  return DS * (256 + dense_nt_cols<MODE>()) * 2 * KC;
}

// one wave's share: MRW row tiles from row r0 of the block tile, NJW column
// tiles (block tile columns 16 bt[j] ..), LW load instructions per chunk,
// chunks [c_lo, c_lo + nchunks) of K
template <int MODE, int DS, int KC, int MRW, int NJW, int LW>
__device__ __forceinline__ void dense_nt_wave(const GemmParams& p, uint8_t* pool, int m_begin, int rows, int n0,
                                              int r0, const int (&bt)[NJW], int wave, int c_lo, int nchunks,
                                              int slice) {
  constexpr int NT = dense_nt_cols<MODE>();
  constexpr int kRowB = 2 * KC;          // bytes of a row per chunk
  constexpr int kPieces = kRowB / 16;    // 16-byte pieces per row
  constexpr int kRpi = 64 / kPieces;     // rows per load instruction
  constexpr int kAInstr = 256 / kRpi;    // activation load instructions per chunk
  constexpr int kStage = (256 + NT) * kRowB;
  // piece q of row r sits in slot q ^ swz(r): the 16 lanes reading one MFMA
  // operand column (16 rows, one piece) hit 16 different bank groups
  auto swz = [](int r) { return kPieces == 4 ? (r >> 2) & 3 : (r >> 1) & 7; };
  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  const int lrow = lane / kPieces, lslot = lane % kPieces;
  const int K = p.K;
  const uint8_t* src[LW];
  int dst[LW];
#pragma unroll
  for (int t = 0; t < LW; ++t) {
    const int i = wave + 8 * t;  // load instruction: activation rows kRpi i.., or weight rows kRpi (i - kAInstr)..
    const int r = kRpi * (i < kAInstr ? i : i - kAInstr) + lrow;
    const int q = lslot ^ swz(r);
    if (i < kAInstr) {
      const int srow = min(m_begin + r, p.M - 1);
      src[t] = reinterpret_cast<const uint8_t*>(p.A + (int64_t)srow * p.lda) + kRowB * c_lo + 16 * q;
    } else {
      const int tj = r >> 4, n = r & 15;
      int64_t c;
      if constexpr (MODE == kNtSwiglu) {  // gate tiles 0..8, up tiles 9..17
        const int h = min(n0 + 16 * (tj < 9 ? tj : tj - 9) + n, p.N - 1);
        c = h + (tj < 9 ? 0 : p.b_row_second);
      } else if constexpr (MODE == kNtRouter) {  // term tj / 6 of expert n0 + 16 (tj % 6) + n
        c = (int64_t)(tj / 6) * p.N + min(n0 + 16 * (tj % 6) + n, p.N - 1);
      } else {
        c = min(n0 + r, p.N - 1);
      }
      src[t] = reinterpret_cast<const uint8_t*>(p.bh + c * K) + kRowB * c_lo + 16 * q;
    }
    dst[t] = 1024 * i;  // activation rows, then weight rows, kRowB bytes each
  }
  auto issue = [&](int c) {
    const int cc = min(c, nchunks - 1);
    uint8_t* st = pool + (c % DS) * kStage;
#pragma unroll
    for (int t = 0; t < LW; ++t) load_lds16(src[t] + kRowB * cc, lds_addr(st + dst[t]));
  };

  f32x4_t acc[MRW][NJW];
#pragma unroll
  for (int m = 0; m < MRW; ++m)
#pragma unroll
    for (int j = 0; j < NJW; ++j) acc[m][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int c = 0; c < DS - 1; ++c) issue(c);
  // at the top of iteration c, chunk c was issued DS - 1 iterations earlier;
  // the loads of the DS - 2 iterations since then may stay in flight
  constexpr int kWait = (DS - 2) * LW;
  for (int c = 0; c < nchunks; ++c) {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(kWait) : "memory");
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    issue(c + DS - 1);  // into the stage read in the previous iteration
    const uint8_t* al = pool + (c % DS) * kStage;
    const uint8_t* bl = al + 256 * kRowB;
#pragma unroll
    for (int s = 0; s < KC / 32; ++s) {  // MFMA K steps of 32
      bf16x8_t a[MRW], b[NJW];
#pragma unroll
      for (int m = 0; m < MRW; ++m) {
        const int ar = r0 + 16 * m + col;
        a[m] = *reinterpret_cast<const bf16x8_t*>(al + kRowB * ar + 16 * ((4 * s + grp) ^ swz(ar)));
      }
#pragma unroll
      for (int j = 0; j < NJW; ++j) {
        const int br = 16 * bt[j] + col;
        b[j] = *reinterpret_cast<const bf16x8_t*>(bl + kRowB * br + 16 * ((4 * s + grp) ^ swz(br)));
      }
#pragma unroll
      for (int j = 0; j < NJW; ++j)
#pragma unroll
        for (int m = 0; m < MRW; ++m) acc[m][j] = mfma_16x16x32(a[m], b[j], acc[m][j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // no load may land in LDS after the block ends

#pragma unroll
  for (int m = 0; m < MRW; ++m) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + 16 * m + 4 * grp + i;
      if (r < rows) {
        if constexpr (MODE == kNtSwiglu) {
          uint16_t* crow = p.C + (int64_t)(m_begin + r) * p.ldc;
#pragma unroll
          for (int j = 0; j < NJW / 2; ++j) {
            const int n = n0 + 16 * bt[j] + col;
            if (n < p.N) crow[n] = f32_to_bf16(clamped_swiglu(acc[m][j][i], acc[m][j + NJW / 2][i], p.limit));
          }
        } else if constexpr (MODE == kNtRouter) {
          float* crow = p.Cf + (int64_t)slice * p.c_slice_stride + (int64_t)(m_begin + r) * p.ldc;
#pragma unroll
          for (int j = 0; j < NJW / 3; ++j) {
            const int n = n0 + 16 * bt[j] + col;
            if (n < p.N) crow[n] = (acc[m][j][i] + acc[m][j + NJW / 3][i]) + acc[m][j + 2 * NJW / 3][i];
          }
        } else {
          uint16_t* crow = p.C + (int64_t)(m_begin + r) * p.ldc;
#pragma unroll
          for (int j = 0; j < NJW; ++j) {
            const int n = n0 + 16 * bt[j] + col;
            if (n < p.N) crow[n] = f32_to_bf16(acc[m][j][i]);
          }
        }
      }
    }
  }
}

// Router mode: blockIdx.y is the K range (p.k_slices of them), written to
// partial-logit slice blockIdx.y.
template <int MODE, int DS, int KC>
__global__ __launch_bounds__(512) void expert_gemm_dense_nt_kernel(GemmParams p, int n_tiles, int col_blocks) {
  constexpr int NT = dense_nt_cols<MODE>();
  constexpr int kInstr = (256 + NT) * 2 * KC / 1024;  // load instructions per chunk
  constexpr int kLo = kInstr / 8, kRem = kInstr % 8;
  static_assert(kRem <= 4, "waves 0 .. kRem - 1 issue one load more");
  __shared__ __attribute__((aligned(16))) uint8_t pool[dense_nt_pool_bytes<MODE, DS, KC>()];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const PipeBlock pb = pipe_block(col_blocks);
  if (pb.tile >= n_tiles) return;
  const int m_begin = pb.tile * 256;
  const int rows = min(256, p.M - m_begin);
  const int n0 = pb.cb * (MODE == kNtSwiglu ? NT / 2 : MODE == kNtRouter ? NT / 3 : NT);
  int c_lo = 0, nchunks = p.K / KC, slice = 0;
  if constexpr (MODE == kNtRouter) {
    // the host sizes k_slices so that every range holds at least one chunk
    slice = (int)blockIdx.y;
    const int per = (nchunks + p.k_slices - 1) / p.k_slices;
    c_lo = slice * per;
    nchunks = min(nchunks - c_lo, per);
  }
  if constexpr (MODE == kNtSwiglu || MODE == kNtRouter) {
    // rows 64 (w & 3) ..; waves 0-3 and 4-7 split the 18 column tiles so
    // that each SIMD (waves w and w + 4) does all 18: SwiGLU h tiles 0-4 /
    // 5-8 with their up tiles, router expert tiles 0-2 / 3-5 with all terms
    const int r0 = 64 * (wave & 3);
    if constexpr (MODE == kNtSwiglu) {
      if (wave < 4) {
        const int bt[10] = {0, 1, 2, 3, 4, 9, 10, 11, 12, 13};
        if (wave < kRem)
          dense_nt_wave<MODE, DS, KC, 4, 10, kLo + 1>(p, pool, m_begin, rows, n0, r0, bt, wave, c_lo, nchunks, 0);
        else
          dense_nt_wave<MODE, DS, KC, 4, 10, kLo>(p, pool, m_begin, rows, n0, r0, bt, wave, c_lo, nchunks, 0);
      } else {
        const int bt[8] = {5, 6, 7, 8, 14, 15, 16, 17};
        dense_nt_wave<MODE, DS, KC, 4, 8, kLo>(p, pool, m_begin, rows, n0, r0, bt, wave, c_lo, nchunks, 0);
      }
    } else {
      const int u0 = wave < 4 ? 0 : 3;
      const int bt[9] = {u0, u0 + 1, u0 + 2, u0 + 6, u0 + 7, u0 + 8, u0 + 12, u0 + 13, u0 + 14};
      if (wave < kRem)
        dense_nt_wave<MODE, DS, KC, 4, 9, kLo + 1>(p, pool, m_begin, rows, n0, r0, bt, wave, c_lo, nchunks, slice);
      else
        dense_nt_wave<MODE, DS, KC, 4, 9, kLo>(p, pool, m_begin, rows, n0, r0, bt, wave, c_lo, nchunks, slice);
    }
  } else {
    const int r0 = 128 * (wave >> 2), j0 = 5 * (wave & 3);
    const int bt[5] = {j0, j0 + 1, j0 + 2, j0 + 3, j0 + 4};
    if (wave < kRem)
      dense_nt_wave<MODE, DS, KC, 8, 5, kLo + 1>(p, pool, m_begin, rows, n0, r0, bt, wave, c_lo, nchunks, 0);
    else
      dense_nt_wave<MODE, DS, KC, 8, 5, kLo>(p, pool, m_begin, rows, n0, r0, bt, wave, c_lo, nchunks, 0);
  }
}

// three stages, two blocks per CU (measured against four stages, one block
// per CU: 274 -> 252 us for the gate/up projection at 4096 tokens)
constexpr int kDenseStages = 3;
// rows from which the shared expert takes the whole-round tiles (4096 rows:
// gate/up 253 -> 182 us, down 128 -> 100 us; 16384 rows, against 256-row tiles
// of the kernel above: 741 -> 686 us, 385 -> 375 us).  With K a multiple of
// 64 it takes 64-wide chunks, two stages (4096 rows: 176 -> 160 us, 98 -> 89
// us; 16384 rows: 676 -> 617 us, 370 -> 339 us), else 32-wide chunks, four.
constexpr int kDenseNtRows = 2048;
constexpr int kDenseNtStages = 4;
constexpr int kDenseNtStages64 = 2;

// MXFP4 weights with K a multiple of 128 at up to this many rows per expert
// on average: 32-row tiles for the pipelined kernel
constexpr int kPipeSmallMt = 2;
constexpr bool kPipeDownWholeScales = true;  // the 32-row down projection with whole scales (K <= 2560)
constexpr int64_t kPipeSmallAvgRows = 16;

int expert_gemm_mt(int64_t n_rows, int n_groups, WeightFormat fmt, bool k_pipelined) {
  const bool fp4 = fmt == kWMxfp4;
  const int kTiledRows = 16 * (fmt == kWBf16 ? tiled_m<kWBf16>() : fmt == kWMxfp8 ? tiled_m<kWMxfp8>()
                                                                                   : tiled_m<kWMxfp4>());
  // MXFP4 weights with every K a multiple of 128: the pipelined kernel at any
  // row count (it streams each expert's weights once per tile and measured
  // faster than 16-row tiles even at 1-5 rows per expert).  Otherwise rows
  // per group on average decides: 128-row tiles go to the LDS-tiled kernel,
  // which needs enough of them to fill the chip.
  const int64_t avg = n_groups > 0 ? (n_rows + n_groups - 1) / n_groups : n_rows;
  if (fp4 && k_pipelined) return avg <= kPipeSmallAvgRows ? kPipeSmallMt : kTiledRows / 16;
  const int64_t tiles = (n_rows + kTiledRows - 1) / kTiledRows;
  return (avg > 16 && tiles >= 16) ? kTiledRows / 16 : 1;
}

// the 512-row form of the pipelined kernel serves the down projection (measured
// faster there: 987 -> 827 us at 4096 tokens; the gate/up projection measured
// slower, 1713 -> 1800 us, and 770 -> 983 us at 64 tokens)
template <bool SWIGLU>
constexpr bool kPipeWide = !SWIGLU;

template <bool SWIGLU, int BF>
static void launch_t(const GemmParams& p, int mt, dim3 grid, hipStream_t stream) {
  constexpr bool FP4 = BF == kWMxfp4;
  if (mt == tiled_m<BF>()) {
    // 128- or 64-row tiles: the LDS-tiled kernel, 4 waves x tiled_cols_per_wave columns per block
    const int cols = 4 * tiled_cols_per_wave<SWIGLU>();
    const dim3 g(grid.x, (unsigned)((p.N + cols - 1) / cols));
    if constexpr (FP4) {
      if (p.K % 128 == 0) {  // MXFP4 weights: the pipelined kernel
        const int n_tiles = (int)grid.x;
        if constexpr (kPipeWide<SWIGLU>) {
          const int cols_wide = 8 * tiled_cols_per_wave<SWIGLU>();
          const int col_blocks = (p.N + cols_wide - 1) / cols_wide;
          const dim3 g1((unsigned)((n_tiles + 7) / 8 * 8 * col_blocks));
          hipLaunchKernelGGL((expert_gemm_wide_kernel<SWIGLU>), g1, dim3(512), 0, stream, p, n_tiles, col_blocks);
        } else {
          const int col_blocks = (int)g.y;
          const dim3 g1((unsigned)((n_tiles + 7) / 8 * 8 * col_blocks));
          if (p.K % 512 == 0)
            hipLaunchKernelGGL((expert_gemm_pipe8_kernel<SWIGLU, 128, 4>), g1, dim3(512), 0, stream, p, n_tiles,
                               col_blocks);
          else
            hipLaunchKernelGGL((expert_gemm_pipe8_kernel<SWIGLU, 128>), g1, dim3(512), 0, stream, p, n_tiles,
                               col_blocks);
        }
        return;
      }
    }
    if constexpr (BF == kWBf16) {
      if (!p.tiles && !p.gather) {  // one dense bf16 matrix (the shared expert): the pipelined dense kernel
        // from kDenseNtRows rows the whole-round tiles, below that 128-row tiles at two blocks per CU
        const int col_blocks = (int)g.y;
        if (p.M >= kDenseNtRows) {
          constexpr int MODE = SWIGLU ? kNtSwiglu : kNtPlain;
          const int n_tiles = (p.M + 255) / 256;
          const int cols_nt = SWIGLU ? dense_nt_cols<MODE>() / 2 : dense_nt_cols<MODE>();
          const int col_blocks_nt = (p.N + cols_nt - 1) / cols_nt;
          const dim3 g1((unsigned)((n_tiles + 7) / 8 * 8 * col_blocks_nt));
          if (p.K % 64 == 0)
            hipLaunchKernelGGL((expert_gemm_dense_nt_kernel<MODE, kDenseNtStages64, 64>), g1, dim3(512), 0, stream,
                               p, n_tiles, col_blocks_nt);
          else
            hipLaunchKernelGGL((expert_gemm_dense_nt_kernel<MODE, kDenseNtStages, 32>), g1, dim3(512), 0, stream,
                               p, n_tiles, col_blocks_nt);
        } else {
          const int n_tiles = (p.M + 127) / 128;
          const dim3 g1((unsigned)((n_tiles + 7) / 8 * 8 * col_blocks));
          hipLaunchKernelGGL((expert_gemm_dense_kernel<SWIGLU, kDenseStages>), g1, dim3(512), 0, stream, p,
                             n_tiles, col_blocks);
        }
        return;
      }
    }
    hipLaunchKernelGGL((expert_gemm_tiled_kernel<SWIGLU, BF>), g, dim3(256), 0, stream, p);
  } else if (FP4 && mt == kPipeSmallMt && p.K % 128 == 0) {
    // 32-row tiles: the 32-row pipelined kernel, two blocks per CU (one
    // block's start and end overlap the other's stream; down 382 -> 345 us at
    // 64 tokens).  Gate/up takes it with scale groups (673 -> 663 us); with
    // 4-byte scale words it measured slower (770 -> 850 us) and keeps the
    // 128-row kernel, one block per CU
    const int n_tiles = (int)grid.x;
    const int col_blocks = (p.N + 4 * tiled_cols_per_wave<SWIGLU>() - 1) / (4 * tiled_cols_per_wave<SWIGLU>());
    const dim3 g1((unsigned)((n_tiles + 7) / 8 * 8 * col_blocks));
    if constexpr (SWIGLU) {
      if (p.K % 512 == 0)
        hipLaunchKernelGGL((expert_gemm_pipe8_kernel<true, 32, 4>), g1, dim3(512), 0, stream, p, n_tiles,
                           col_blocks);
      else
        hipLaunchKernelGGL((expert_gemm_pipe8_kernel<true, 128>), g1, dim3(512), 0, stream, p, n_tiles, col_blocks);
    } else if (p.K / 32 * 256 <= kPipeWholeS && kPipeDownWholeScales) {
      hipLaunchKernelGGL((expert_gemm_pipe8_kernel<false, 32, 1>), g1, dim3(512), 0, stream, p, n_tiles, col_blocks);
    } else if (p.K % 384 == 0) {
      hipLaunchKernelGGL((expert_gemm_pipe8_kernel<false, 32, 3>), g1, dim3(512), 0, stream, p, n_tiles, col_blocks);
    } else {
      hipLaunchKernelGGL((expert_gemm_pipe8_kernel<false, 32>), g1, dim3(512), 0, stream, p, n_tiles, col_blocks);
    }
  } else {
    if constexpr (BF == kWBf16) {
      if (mt == 2) {  // 32-row tiles (the shared expert at 17..127 tokens)
        hipLaunchKernelGGL((expert_gemm_kernel<2, SWIGLU, BF>), grid, dim3(256), 0, stream, p);
        return;
      }
    }
    hipLaunchKernelGGL((expert_gemm_kernel<1, SWIGLU, BF>), grid, dim3(256), 0, stream, p);
  }
}

hipError_t launch_dense_f32(const GemmParams& p, int slices, hipStream_t stream) {
  const int n_tiles = (p.M + 127) / 128;
  const int col_blocks = (p.N + 255) / 256;
  const dim3 g((unsigned)((n_tiles + 7) / 8 * 8 * col_blocks), (unsigned)slices);
  hipLaunchKernelGGL((expert_gemm_dense_kernel<false, kDenseStages, true>), g, dim3(512), 0, stream, p, n_tiles,
                     col_blocks);
  return hipGetLastError();
}

// Router logits from the whole-round kernel: p.bh holds the three bf16 terms
// of W_r ([3][N][K]), p.k_slices K ranges, partial slice r = range r.
int dense_router_kslices(int M, int n_experts, int K) {
  const int tiles = (M + 255) / 256 * ((n_experts + 95) / 96);
  const int nch = K % 64 == 0 ? K / 64 : K / 32;
  int ks = (256 + tiles - 1) / tiles;
  ks = ks < 1 ? 1 : ks > 8 ? 8 : ks;
  if (ks > nch) ks = nch;
  const int per = (nch + ks - 1) / ks;
  return (nch + per - 1) / per;  // every K range non-empty
}

hipError_t launch_dense_router(const GemmParams& p, hipStream_t stream) {
  const int n_tiles = (p.M + 255) / 256;
  const int col_blocks = (p.N + 95) / 96;
  const dim3 g((unsigned)((n_tiles + 7) / 8 * 8 * col_blocks), (unsigned)p.k_slices);
  if (p.K % 64 == 0)
    hipLaunchKernelGGL((expert_gemm_dense_nt_kernel<kNtRouter, kDenseNtStages64, 64>), g, dim3(512), 0, stream, p,
                       n_tiles, col_blocks);
  else
    hipLaunchKernelGGL((expert_gemm_dense_nt_kernel<kNtRouter, kDenseNtStages, 32>), g, dim3(512), 0, stream, p,
                       n_tiles, col_blocks);
  return hipGetLastError();
}

// Sum of fp32 K slices in slice order, then clamp-SwiGLU of (gate column n,
// up column n + n_out) or the plain sum, rounded to bf16.
template <bool SWIGLU>
__global__ __launch_bounds__(256) void slice_sum_kernel(const float* __restrict__ part, int slices,
                                                        int64_t slice_stride, int rows, int n_out, int ld_part,
                                                        float limit, uint16_t* __restrict__ C, int64_t ldc) {
  const int64_t total = (int64_t)rows * n_out;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
    const int r = (int)(i / n_out), n = (int)(i % n_out);
    const float* src = part + (int64_t)r * ld_part + n;
    float g = 0.f, u = 0.f;
    for (int s = 0; s < slices; ++s) {
      g += src[s * slice_stride];
      if constexpr (SWIGLU) u += src[s * slice_stride + n_out];
    }
    C[(int64_t)r * ldc + n] = f32_to_bf16(SWIGLU ? clamped_swiglu(g, u, limit) : g);
  }
}

// ---------------------------------------------------------------- skinny bf16, few rows
// The shared expert below 512 tokens: fp32 partial products of up to 16 MT
// rows (row group blockIdx.z) against 64 weight rows per block over one K
// range (blockIdx.y of p.k_slices, in 128-wide chunks), summed and finished
// by slice_sum_kernel.  Four waves of 16 weight rows each: the weights stream
// from memory straight to registers, kSkPf chunks ahead, each weight byte
// read once by one wave; the rows' chunk goes global -> registers -> LDS
// (two stages) and all four waves read it there.  The 128-row kernels above
// computed at least 128 rows per tile, and their 32-row form re-read the
// weights for every row tile: 64 tokens took 52 + 28 us for 71 MB, against 28
// + 18 us here (with the partial sums).
constexpr int kSkPf = 4;            // weight chunks in flight per wave
constexpr int kSkMaxRows = 512;     // rows in up to four groups of 128
constexpr int kSkRowB = 256 + 16;   // LDS bytes per staged row: 128 bf16 + 16 (8 rows on 8 bank quads)
template <int MT>
__global__ __launch_bounds__(256) void skinny_bf16_kernel(GemmParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][16 * MT * kSkRowB];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int nch_all = p.K / 128;
  const int per = (nch_all + p.k_slices - 1) / p.k_slices;
  const int slice = (int)blockIdx.y, c_lo = slice * per;
  const int nch = min(per, nch_all - c_lo);  // >= 1: the host makes every range non-empty
  const int n = (int)blockIdx.x * 64 + 16 * wave + col;  // this lane's weight row (B operand column)
  const int r0 = 16 * MT * (int)blockIdx.z;              // this block's row group

  // weights: row n, 16 bytes at K offset 128 c + 32 s + 8 grp (s = MFMA K step)
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(p.bh, (uint32_t)((int64_t)p.N * p.K * 2));
  const uint32_t b_off = (uint32_t)min(n, p.N - 1) * (uint32_t)(p.K * 2) + 16u * grp;
  u32x4_t wb[kSkPf][4];
  // a chunk past the range reads zeros (per-lane offset kOob, which the
  // buffer range check turns into a zero), so its MFMAs add nothing
  auto load_w = [&](int c, u32x4_t (&d)[4]) {
    const int cc = c_lo + min(c, nch - 1);
    const bool in = c < nch;
#pragma unroll
    for (int s = 0; s < 4; ++s)
      d[s] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rb, (int)(in ? b_off + 64u * s : kOob), 256 * cc, 0));
  };
  // rows: piece q = tid + 256 i (row q / 16, 16-byte part q % 16) of the chunk
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, (uint32_t)((int64_t)p.a_rows * p.lda * 2));
  uint32_t a_off[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int q = (int)threadIdx.x + 256 * i, r = r0 + (q >> 4);
    a_off[i] = (uint32_t)((int64_t)min(r, p.M - 1) * p.lda * 2) + 16u * (q & 15);
  }
  // two chunks of rows in registers: each load has two iterations to land
  u32x4_t xr[2][MT];
  auto load_x = [&](int c, u32x4_t (&d)[MT]) {
    const int cc = c_lo + min(c, nch - 1);
#pragma unroll
    for (int i = 0; i < MT; ++i)
      d[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)a_off[i], 256 * cc, 0));
  };
  auto store_x = [&](int stage, const u32x4_t (&v)[MT]) {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int q = (int)threadIdx.x + 256 * i;
      *reinterpret_cast<u32x4_t*>(xs[stage] + (q >> 4) * kSkRowB + 16 * (q & 15)) = v[i];
    }
  };

  f32x4_t acc[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // the rows first: loads complete in issue order, so the wait for chunk 0's
  // rows would otherwise also wait for the weights
  load_x(0, xr[0]);
  load_x(1, xr[1]);
#pragma unroll
  for (int b = 0; b < kSkPf; ++b) load_w(b, wb[b]);
  store_x(0, xr[0]);
  load_x(2, xr[0]);
  __syncthreads();
  // iteration c: chunk c's rows are in stage c & 1, chunks c + 1 and c + 2's
  // in registers xr[(c + 1) & 1] and xr[c & 1]; chunk c's weights in wb[c % kSkPf]
  auto step = [&](int c, u32x4_t (&w)[4], u32x4_t (&xn)[MT]) {
    const uint8_t* st = xs[c & 1];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(st + (16 * m + col) * kSkRowB + 64 * s + 16 * grp);
        acc[m] = mfma_16x16x32(a, __builtin_bit_cast(bf16x8_t, w[s]), acc[m]);
      }
    }
    // issue order pinned (loads complete in that order, and the compiler's
    // waits count it): this step's weights, then the rows stored from the
    // registers loaded two steps ago, then the rows for two steps ahead
    __builtin_amdgcn_sched_barrier(0);
    load_w(c + kSkPf, w);
    __builtin_amdgcn_sched_barrier(0);
    store_x((c + 1) & 1, xn);  // stage (c + 1) & 1 was last read in iteration c - 1
    __builtin_amdgcn_sched_barrier(0);
    load_x(c + 3, xn);
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
  };
  // whole groups of kSkPf steps, those past the range on zero weights: with
  // a guard around each step the compiler's waits would have to hold for the
  // path that skips steps, and they drained the weight prefetch every step
  for (int c = 0; c < nch; c += kSkPf) {
#pragma unroll
    for (int u = 0; u < kSkPf; ++u) step(c + u, wb[u], xr[(u + 1) & 1]);
  }

  float* out = p.Cf + (int64_t)slice * p.c_slice_stride;
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = r0 + 16 * m + 4 * grp + i;
      if (r < p.M && n < p.N) out[(int64_t)r * p.ldc + n] = acc[m][i];
    }
}

int skinny_k_slices(int M, int n_rows, int K) {
  if (M < 1 || M > kSkMaxRows || K % 128 != 0) return 0;
  const int blocks = (n_rows + 63) / 64 * ((M + 127) / 128), nch = K / 128;
  // ~128 blocks of long streams (64 tokens: 2 ranges 28 + 18 us, 4 ranges 31 + 21 us; 1 range 47 + 26 us)
  int ks = (128 + blocks - 1) / blocks;
  ks = ks < 1 ? 1 : ks > 8 ? 8 : ks;
  if (ks > nch) ks = nch;
  const int per = (nch + ks - 1) / ks;
  return (nch + per - 1) / per;  // every K range non-empty
}

hipError_t launch_skinny_sliced(const GemmParams& p, bool swiglu, int k_slices, float* part, hipStream_t stream) {
  GemmParams q = p;
  q.N = swiglu ? 2 * p.N : p.N;  // weight rows: gate rows, then up rows (b_row_second == N)
  q.ldc = q.N;
  q.Cf = part;
  q.k_slices = k_slices;
  q.c_slice_stride = (int64_t)p.M * q.N;
  // rows in groups of up to 128 (blockIdx.z), each re-reading the weights from the caches
  const dim3 g((unsigned)((q.N + 63) / 64), (unsigned)k_slices, (unsigned)((p.M + 127) / 128));
  const int mt = (p.M < 128 ? p.M + 15 : 128) / 16;
  if (mt <= 2)
    hipLaunchKernelGGL(skinny_bf16_kernel<2>, g, dim3(256), 0, stream, q);
  else if (mt <= 4)
    hipLaunchKernelGGL(skinny_bf16_kernel<4>, g, dim3(256), 0, stream, q);
  else if (mt <= 6)
    hipLaunchKernelGGL(skinny_bf16_kernel<6>, g, dim3(256), 0, stream, q);
  else
    hipLaunchKernelGGL(skinny_bf16_kernel<8>, g, dim3(256), 0, stream, q);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t total = (int64_t)p.M * p.N;
  const int64_t blocks = (total + 255) / 256;
  const dim3 gs((unsigned)(blocks < 4096 ? blocks : 4096));
  if (swiglu)
    hipLaunchKernelGGL(slice_sum_kernel<true>, gs, dim3(256), 0, stream, part, k_slices, q.c_slice_stride, p.M, p.N,
                       q.N, p.limit, p.C, p.ldc);
  else
    hipLaunchKernelGGL(slice_sum_kernel<false>, gs, dim3(256), 0, stream, part, k_slices, q.c_slice_stride, p.M,
                       p.N, q.N, p.limit, p.C, p.ldc);
  return hipGetLastError();
}

int dense_k_slices(int M, int n_rows, int K) {
  const int64_t blocks = (int64_t)((M + 127) / 128) * ((n_rows + 255) / 256);
  const int nch = K / 32;
  int64_t ks = (640 + blocks - 1) / blocks;
  ks = ks < 1 ? 1 : ks > 16 ? 16 : ks;
  if (ks > nch) ks = nch;
  const int per = (int)((nch + ks - 1) / ks);
  return (nch + per - 1) / per;  // every K range non-empty
}

hipError_t launch_dense_sliced(const GemmParams& p, bool swiglu, int k_slices, float* part, hipStream_t stream) {
  GemmParams q = p;
  q.N = swiglu ? 2 * p.N : p.N;  // weight rows: gate rows, then up rows (b_row_second == N)
  q.ldc = q.N;
  q.Cf = part;
  q.k_slices = k_slices;
  q.b_slice_stride = 0;
  q.c_slice_stride = (int64_t)p.M * q.N;
  hipError_t err = launch_dense_f32(q, k_slices, stream);
  if (err != hipSuccess) return err;
  const int64_t total = (int64_t)p.M * p.N;
  const int64_t blocks = (total + 255) / 256;
  const dim3 g((unsigned)(blocks < 4096 ? blocks : 4096));
  if (swiglu)
    hipLaunchKernelGGL(slice_sum_kernel<true>, g, dim3(256), 0, stream, part, k_slices, q.c_slice_stride, p.M, p.N,
                       q.N, p.limit, p.C, p.ldc);
  else
    hipLaunchKernelGGL(slice_sum_kernel<false>, g, dim3(256), 0, stream, part, k_slices, q.c_slice_stride, p.M, p.N,
                       q.N, p.limit, p.C, p.ldc);
  return hipGetLastError();
}

hipError_t launch_expert_gemm(const GemmParams& p, bool swiglu, WeightFormat fmt, int mt, int64_t grid_tiles,
                              hipStream_t stream) {
  dim3 grid((unsigned)grid_tiles, (unsigned)(p.N / 16));
  switch (fmt) {
    case kWMxfp4: swiglu ? launch_t<true, kWMxfp4>(p, mt, grid, stream) : launch_t<false, kWMxfp4>(p, mt, grid, stream); break;
    case kWMxfp8: swiglu ? launch_t<true, kWMxfp8>(p, mt, grid, stream) : launch_t<false, kWMxfp8>(p, mt, grid, stream); break;
    default: swiglu ? launch_t<true, kWBf16>(p, mt, grid, stream) : launch_t<false, kWBf16>(p, mt, grid, stream); break;
  }
  return hipGetLastError();
}

}  // namespace moe
