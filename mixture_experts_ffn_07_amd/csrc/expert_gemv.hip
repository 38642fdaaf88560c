// Expert projections for few tokens (decode): weight streaming at HBM rate.
//
// With T <= 8 tokens an expert receives at most T rows (a token selects an
// expert at most once), so one tile per expert reads each weight byte
// exactly once, and the layer's cost is the weight bytes (MXFP4 routed
// experts, bf16 shared expert: Strata DEEPSEEK41 notes, opening paragraph
// and the "Where it goes" table).  Both kernels keep as many weight bytes in
// flight as the register file allows and spend little ALU time per byte:
//   * weights are read with raw buffer loads: a load past the end of the
//     expert's matrix returns zero without touching memory, so every load
//     is issued unconditionally and each wait covers exactly the batch
//     about to be used;
//   * each wave streams its weights in double-buffered batches.
//
// MXFP4 (routed experts, expert_gemv_mx_kernel): the E2M1 codes go straight
// into gfx950's block-scaled matrix instruction
// (v_mfma_scale_f32_16x16x128_f8f6f4) as the B operand with their E8M0
// scales, no dequantisation; activation rows are in two-term MXFP8 form
// (mx_device.h), two MFMAs (hi, lo) per 128-wide chunk.  MXFP8 weights
// (E4M3, one code a byte) go in the same way as the instruction's 8-bit B
// operand, 32 codes per lane and chunk in two 16-byte pieces, at the FP8
// rate.  A wave owns 16 output columns over all of K.  Scale bytes are
// fetched as whole words covering several chunks: per-chunk byte loads cost
// as much memory-pipe time as the code loads they accompany.
//
// bf16 (shared expert, expert_gemv_bf16_kernel): v_mfma_f32_16x16x32_bf16
// on bf16 rows; the 4 waves of a block split K and add their partial tiles
// in a fixed order through LDS.
//
// Rows >= T of the 16-row MFMA tile are zero and are never read or
// written; the epilogue applies the clamped SwiGLU (gate/up) or stores bf16
// (down).
#include "moe_device.h"
#include "moe_internal.h"
#include "mx_device.h"
#include "gemv_bf16_device.h"

namespace moe {

namespace {

// ============================================================== MXFP4 weights (routed experts)
// Weights of kMxChunks consecutive 128-wide chunks of this lane's row(s):
// E2M1 codes (32 per lane per chunk) and, per chunk, the dword holding the
// 4 block scales of the chunk (byte g for lane group g).  Two batches are in
// flight per wave.
constexpr int kMxChunks = 4;  // a multiple of 4
// W8: MXFP8 weights, 32 E4M3 codes per lane and chunk in two 16-byte pieces
// (q: K offsets [16 g, 16 g + 16) of the chunk, q2: [64 + 16 g, 80 + 16 g),
// the matrix instruction's 8-bit operand layout, as for the A rows)
template <int NB, bool W8 = false>
struct MxBatch {
  u32x4_t q[kMxChunks][NB];
  u32x4_t q2[W8 ? kMxChunks : 1][NB];
  uint32_t s[kMxChunks][NB];
};

// D += A(16x128, E4M3, E8M0 per 32) * B(128x16, E4M3, E8M0 per 32), fp32:
// the MXFP8-weight form of mfma_mx (B in the 8-bit layout of A).
__device__ __forceinline__ f32x4_t mfma_mx8(const i32x8_t& a, const u32x4_t& b0, const u32x4_t& b1, int sa, int sb,
                                            f32x4_t c) {
  const i32x8_t bw = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bw, c, 0, 0, 0, sa, 0, sb);
}

struct MxView {
  __amdgpu_buffer_rsrc_t q, s;
  uint32_t qrow[2], srow[2];  // byte offsets of this lane's row(s); kOob for columns past N
  int K, nchunks;
};

// SW = bytes per scale load: 16 (K % 512 == 0), 8 (K % 256 == 0), 4
// (K % 128 == 0) or 1 (one byte per lane and chunk, any K % 32 == 0).  The
// wider loads bring the scales of 4, 2 or 1 chunks for all 4 lane groups
// at once; the row offsets are then multiples of the load width.  SW = 0:
// the block staged all its rows' scales in LDS once (no scale loads here).
template <int NB, int SW, bool W8 = false>
__device__ __forceinline__ void mx_load(MxBatch<NB, W8>& b, const MxView& v, int c0, int grp) {
#pragma unroll
  for (int u = 0; u < kMxChunks; ++u) {
    const int c = c0 + u;
    const bool ok = c < v.nchunks && c * 128 + grp * 32 < v.K;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      if constexpr (W8) {
        const uint32_t qo = ok ? v.qrow[nb] + (uint32_t)(c * 128 + grp * 16) : kOob;
        const uint32_t qo2 = ok ? qo + 64u : kOob;
        b.q[u][nb] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(v.q, (int)qo, 0, 0));
        b.q2[u][nb] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(v.q, (int)qo2, 0, 0));
      } else {
        const uint32_t qo = ok ? v.qrow[nb] + (uint32_t)(c * 64 + grp * 16) : kOob;
        b.q[u][nb] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(v.q, (int)qo, 0, 0));
      }
    }
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if constexpr (SW == 0) {
      // scales staged in LDS by the block
    } else if constexpr (SW == 16) {
#pragma unroll
      for (int h = 0; h < kMxChunks / 4; ++h) {
        const int c = c0 + 4 * h;
        const uint32_t so = c < v.nchunks ? v.srow[nb] + (uint32_t)(4 * c) : kOob;
        const u32x4_t w = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(v.s, (int)so, 0, 0));
#pragma unroll
        for (int u = 0; u < 4; ++u) b.s[4 * h + u][nb] = w[u];
      }
    } else if constexpr (SW == 8) {
#pragma unroll
      for (int h = 0; h < kMxChunks / 2; ++h) {
        const int c = c0 + 2 * h;
        const uint32_t so = c < v.nchunks ? v.srow[nb] + (uint32_t)(4 * c) : kOob;
        const auto w = __builtin_amdgcn_raw_buffer_load_b64(v.s, (int)so, 0, 0);
        b.s[2 * h][nb] = w[0];
        b.s[2 * h + 1][nb] = w[1];
      }
    } else if constexpr (SW == 4) {
#pragma unroll
      for (int u = 0; u < kMxChunks; ++u) {
        const int c = c0 + u;
        const uint32_t so = c < v.nchunks ? v.srow[nb] + (uint32_t)(4 * c) : kOob;
        b.s[u][nb] = __builtin_amdgcn_raw_buffer_load_b32(v.s, (int)so, 0, 0);
      }
    } else {
#pragma unroll
      for (int u = 0; u < kMxChunks; ++u) {
        const int c = c0 + u;
        const bool ok = c < v.nchunks && c * 128 + grp * 32 < v.K;
        const uint32_t so = ok ? v.srow[nb] + (uint32_t)(4 * c + grp) : kOob;
        b.s[u][nb] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(v.s, (int)so, 0, 0) << (8 * grp);
      }
    }
  }
}

// Two block-scaled MFMAs (hi and lo activation terms) per chunk and row set.
// `row` is this lane's staged MX row (tile row `col`), r_ok = col < rows.
// srow_lds: this lane's row scales in LDS (SW = 0), per NB at stride sl_stride.
template <int NB, int SW, bool W8 = false>
__device__ __forceinline__ void mx_mma(const MxBatch<NB, W8>& b, f32x4_t (&acc)[NB], const uint8_t* row, bool r_ok,
                                       int c0, const MxView& v, int grp, const uint8_t* srow_lds, int sl_stride) {
  const int K = v.K;
#pragma unroll
  for (int u = 0; u < kMxChunks; ++u) {
    const int c = c0 + u;
    if (c >= v.nchunks) break;  // wave-uniform
    const int kb = c * 128;
    const bool h0 = r_ok && kb + 16 * grp < K, h1 = r_ok && kb + 64 + 16 * grp < K;
    const u32x4_t z = u32x4_t{0u, 0u, 0u, 0u};
    const u32x4_t a0 = h0 ? *reinterpret_cast<const u32x4_t*>(row + kb + 16 * grp) : z;
    const u32x4_t a1 = h1 ? *reinterpret_cast<const u32x4_t*>(row + kb + 64 + 16 * grp) : z;
    const u32x4_t l0 = h0 ? *reinterpret_cast<const u32x4_t*>(row + K + kb + 16 * grp) : z;
    const u32x4_t l1 = h1 ? *reinterpret_cast<const u32x4_t*>(row + K + kb + 64 + 16 * grp) : z;
    const int sa = (r_ok && kb + 32 * grp < K) ? (int)row[2 * K + kb / 32 + grp] : 127;
    const i32x8_t ahi = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    const i32x8_t alo = {(int)l0[0], (int)l0[1], (int)l0[2], (int)l0[3], (int)l1[0], (int)l1[1], (int)l1[2], (int)l1[3]};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int sb = SW == 0 ? (int)srow_lds[nb * sl_stride + kb / 32 + grp]
                             : (int)((b.s[u][nb] >> (8 * grp)) & 0xffu);
      if constexpr (W8) {
        acc[nb] = mfma_mx8(ahi, b.q[u][nb], b.q2[u][nb], sa, sb, acc[nb]);
        acc[nb] = mfma_mx8(alo, b.q[u][nb], b.q2[u][nb], sa, sb, acc[nb]);
      } else {
        acc[nb] = mfma_mx(ahi, b.q[u][nb], sa, sb, acc[nb]);
        acc[nb] = mfma_mx(alo, b.q[u][nb], sa, sb, acc[nb]);
      }
    }
  }
}

// MX staging of one tile row into LDS (row stride mx_row_bytes(K)), in passes.
// Copy mode (p.amx): 16-byte pieces of a pre-converted row, 3 per thread per
// pass.  Convert mode: one 32-value block of bf16 per thread per pass.  The
// source row `sr` is uniform, so no per-lane row lookup is needed.
struct MxStage {
  u32x4_t v[4];
};

template <bool AMX>
__device__ __forceinline__ int mx_row_passes(const GemvProblem& p) {
  return AMX ? (mx_row_bytes(p.K) / 16 + 767) / 768 : (p.K / 32 + 255) / 256;
}

template <bool AMX>
__device__ __forceinline__ void mx_row_issue(const GemvProblem& p, int sr, int pass, MxStage& s) {
  const int K = p.K, stride = mx_row_bytes(K);
  if constexpr (AMX) {
    const int pieces = stride / 16;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.amx, (uint32_t)((int64_t)p.a_rows * stride));
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int q = pass * 768 + (int)threadIdx.x + 256 * j;
      const uint32_t off = q < pieces ? (uint32_t)(sr * stride + 16 * q) : kOob;
      s.v[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)off, 0, 0));
    }
  } else {
    const int nblk = K / 32;
    const int b = pass * 256 + (int)threadIdx.x;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, (uint32_t)((int64_t)p.a_rows * p.lda * 2));
    const uint32_t off = b < nblk ? (uint32_t)(((int64_t)sr * p.lda + 32 * b) * 2) : kOob;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      s.v[q] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)off, 16 * q, 0));
  }
}

template <bool AMX>
__device__ __forceinline__ void mx_row_commit(const GemvProblem& p, int r, int pass, const MxStage& s,
                                              uint8_t* lds) {
  const int K = p.K, stride = mx_row_bytes(K);
  uint8_t* row = lds + r * stride;
  if constexpr (AMX) {
    const int pieces = stride / 16;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int q = pass * 768 + (int)threadIdx.x + 256 * j;
      if (q < pieces) *reinterpret_cast<u32x4_t*>(row + 16 * q) = s.v[j];
    }
  } else {
    const int b = pass * 256 + (int)threadIdx.x;
    if (b < K / 32) {
      float x[32];
      unpack_bf16x32(s.v, x);
      mx_convert_block(x, row + 32 * b, row + K + 32 * b, row + 2 * K + b);
    }
  }
}

}  // namespace

// ---------------------------------------------------------------- bf16 kernel
// 1-D grid: problem 1's blocks first, then problem 0's.
template <bool SWIGLU>
__global__ __launch_bounds__(256) void expert_gemv_bf16_kernel(GemvParams prm) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int first = prm.p[1].grid_tiles * prm.p[1].col_tiles;
  const int id = blockIdx.x;
  if (id < first)
    gemv_bf16_block<SWIGLU>(prm.p[1], id, prm.rows_cap, prm.limit, lds);
  else
    gemv_bf16_block<SWIGLU>(prm.p[0], id - first, prm.rows_cap, prm.limit, lds);
}

// ---------------------------------------------------------------- MXFP4 kernel
// Block = one tile x 64 output columns; wave w owns columns n0 + 16w .. +15
// over the whole of K, so there is no cross-wave reduction.  Prologue: the
// tile record and the count (scalar loads issued together), then the source
// row of each tile row (gathered positions: one more scalar round trip).
// The first staging pass is issued before the weight prefetch, so the
// staged rows are in LDS by the time the first weights arrive.
// AMX: the activation rows come pre-converted (p.amx), else bf16 rows (p.A)
// are converted while staging.
template <int NB, int SW, bool AMX, bool W8 = false>
__global__ __launch_bounds__(256) void expert_gemv_mx_kernel(GemvProblem p, int rows_cap, float limit) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int tile = blockIdx.x % p.grid_tiles;
  const int nblk0 = (blockIdx.x / p.grid_tiles) * 64;  // first output column of the block
  const int n0 = nblk0 + wave * 16;
  int e = 0, m_begin, rows;
  int src[kTileRows];
  if (p.tile_rows) {
    // every tile record is written (unused ones empty): record and rows are
    // independent scalar loads, no count needed
    const GemmTile tl = p.tiles[tile];
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) src[r] = p.tile_rows[tile * kTileRows + r];
    e = tl.e;
    m_begin = tl.m_begin;
    rows = min(tl.m_end, tl.m_begin + rows_cap) - m_begin;
  } else if (p.tiles) {
    const int tc = *p.tile_count;
    const GemmTile tl = p.tiles[tile];
    if (tile >= tc) return;
    e = tl.e;
    m_begin = tl.m_begin;
    rows = min(tl.m_end, tl.m_begin + rows_cap) - m_begin;
  } else {
    m_begin = tile * rows_cap;
    rows = min(rows_cap, p.M - m_begin);
  }
  if (rows <= 0) return;
  if (p.tile_rows) {
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) src[r] = min(max(src[r], 0), p.a_rows - 1);
  } else if (p.gather) {
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) src[r] = p.gather[min(max(m_begin + r, 0), p.gather_len - 1)];
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) src[r] = min(max(src[r] / p.gather_div, 0), p.a_rows - 1);
  } else {
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) src[r] = min(max(m_begin + r, 0), p.a_rows - 1);
  }

  const int K = p.K;
  MxView v;
  v.K = K;
  v.nchunks = (K + 127) / 128;
  const int row_q = W8 ? K : K / 2;  // code bytes per weight row
  const uint32_t qbytes = (uint32_t)(p.b_expert_rows * row_q);
  const uint32_t sbytes = (uint32_t)(p.b_expert_rows * (K / 32));
  v.q = make_rsrc(p.bq + (int64_t)e * qbytes, qbytes);
  v.s = make_rsrc(p.bs + (int64_t)e * sbytes, sbytes);
  const bool n_ok = n0 < p.N;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const uint32_t r = (uint32_t)(n0 + col + nb * p.b_row_second);
    v.qrow[nb] = n_ok ? r * (uint32_t)row_q : kOob;
    v.srow[nb] = n_ok ? r * (uint32_t)(K / 32) : kOob;
  }

  // staging loads (activation rows; with SW = 0 also the scales of the
  // block's 64 rows per gate/up half) go out before the weight prefetch
  const int a_bytes = rows_cap * mx_row_bytes(K);
  const int sl_stride = 64 * (K / 32);  // LDS bytes of one half's scales
  MxStage st;
  mx_row_issue<AMX>(p, src[0], 0, st);
  constexpr int kScalePieces = SW == 0 ? 5 * NB : 1;  // 16-byte pieces per thread (K <= 5120 with SW = 0)
  u32x4_t sv[kScalePieces];
  if constexpr (SW == 0) {
    const int pieces = sl_stride / 16;  // per half
#pragma unroll
    for (int j = 0; j < kScalePieces; ++j) {
      const int i = (int)threadIdx.x + 256 * j;
      const int nb = i / pieces, q = i - nb * pieces;
      const uint32_t off = (nb < NB && q < pieces)
                               ? (uint32_t)(nblk0 + nb * p.b_row_second) * (uint32_t)(K / 32) + 16u * q
                               : kOob;
      sv[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(v.s, (int)off, 0, 0));
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  MxBatch<NB, W8> b0, b1;
  mx_load<NB, SW, W8>(b0, v, 0, grp);
  mx_load<NB, SW, W8>(b1, v, kMxChunks, grp);
  __builtin_amdgcn_sched_barrier(0);
  mx_row_commit<AMX>(p, 0, 0, st, lds);
  if constexpr (SW == 0) {
    const int pieces = sl_stride / 16;
#pragma unroll
    for (int j = 0; j < kScalePieces; ++j) {
      const int i = (int)threadIdx.x + 256 * j;
      if (i < NB * pieces) *reinterpret_cast<u32x4_t*>(lds + a_bytes + 16 * i) = sv[j];
    }
  }
  const int passes = mx_row_passes<AMX>(p);
#pragma unroll
  for (int r = 0; r < kTileRows; ++r) {
    if (r >= rows) break;  // block-uniform
    for (int pass = r == 0 ? 1 : 0; pass < passes; ++pass) {
      mx_row_issue<AMX>(p, src[r], pass, st);
      mx_row_commit<AMX>(p, r, pass, st, lds);
    }
  }
  __syncthreads();

  f32x4_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const bool r_ok = col < rows;
  const uint8_t* row = lds + (r_ok ? col : 0) * mx_row_bytes(K);
  const uint8_t* srow_lds = lds + a_bytes + (wave * 16 + col) * (K / 32);
  constexpr int CB = kMxChunks;
  for (int c = 0; c < v.nchunks; c += 2 * CB) {
    mx_mma<NB, SW, W8>(b0, acc, row, r_ok, c, v, grp, srow_lds, sl_stride);
    if (c + CB >= v.nchunks) break;
    mx_load<NB, SW, W8>(b0, v, c + 2 * CB, grp);
    mx_mma<NB, SW, W8>(b1, acc, row, r_ok, c + CB, v, grp, srow_lds, sl_stride);
    mx_load<NB, SW, W8>(b1, v, c + 3 * CB, grp);
  }
  if (NB == 2 && p.cmx) {
    // two-term MXFP8 output rows (stride mx_row_bytes(N)): the block's 64
    // columns are two 32-value blocks per row, gathered through LDS
    __shared__ float hout[kTileRows][64];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * grp + i;
      if (r < rows && r < kTileRows) hout[r][wave * 16 + col] = clamped_swiglu(acc[0][i], acc[NB - 1][i], limit);
    }
    __syncthreads();
    const int t = threadIdx.x, r = t >> 1, c0 = nblk0 + 32 * (t & 1);
    if (t < 2 * kTileRows && r < rows && c0 < p.N) {
      float x[32];
#pragma unroll
      for (int j = 0; j < 32; ++j) x[j] = hout[r][32 * (t & 1) + j];
      uint8_t* dst = p.cmx + (int64_t)(m_begin + r) * mx_row_bytes(p.N);
      mx_convert_block(x, dst + c0, dst + p.N + c0, dst + 2 * p.N + c0 / 32);
    }
    return;
  }
  if (!n_ok) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * grp + i;
    if (r < rows) {
      const float o = NB == 2 ? clamped_swiglu(acc[0][i], acc[NB - 1][i], limit) : acc[0][i];
      p.C[(int64_t)(m_begin + r) * p.ldc + n0 + col] = f32_to_bf16(o);
    }
  }
}


// ---------------------------------------------------------------- MXFP4 split-K kernel
// Block = one tile x 16 output columns.  Its W waves split K into
// contiguous ranges of CPW 128-wide chunks and each wave issues all the
// weight loads of its range at once (CPW * NB 16-byte loads per lane).  The
// block stages the tile's activation rows and its weight rows' scales in
// LDS; the partial tiles of the waves are added in wave order through LDS.
// Many light blocks keep more memory requests in flight across the chip
// than a few deep ones: a streaming read of 75 MB takes ~20 us with 216
// four-wave blocks and ~14-15 us with 1000 or more.
template <int CPW>
__device__ __forceinline__ int splitk_waves(int K) {
  return ((K + 127) / 128 + CPW - 1) / CPW;
}

__device__ __forceinline__ size_t splitk_scale_bytes(int nb, int K) { return (size_t)nb * 16 * (K / 32); }

template <int NB, int CPW, bool AMX, bool W8 = false>
__global__ __launch_bounds__(512) void expert_gemv_splitk_kernel(GemvProblem p, int rows_cap, float limit) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nthreads = blockDim.x;
  const int col = lane & 15, grp = lane >> 4;
  const int tile = blockIdx.x % p.grid_tiles;
  const int n0 = (blockIdx.x / p.grid_tiles) * 16;
  int e = 0, m_begin, rows;
  int src[kTileRows];
  if (p.tile_rows) {
    const GemmTile tl = p.tiles[tile];
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) src[r] = p.tile_rows[tile * kTileRows + r];
    e = tl.e;
    m_begin = tl.m_begin;
    rows = min(tl.m_end, tl.m_begin + rows_cap) - m_begin;
  } else if (p.tiles) {
    const int tc = *p.tile_count;
    const GemmTile tl = p.tiles[tile];
    if (tile >= tc) return;
    e = tl.e;
    m_begin = tl.m_begin;
    rows = min(tl.m_end, tl.m_begin + rows_cap) - m_begin;
  } else {
    m_begin = tile * rows_cap;
    rows = min(rows_cap, p.M - m_begin);
  }
  if (rows <= 0) return;
  if (p.tile_rows) {
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) src[r] = min(max(src[r], 0), p.a_rows - 1);
  } else if (p.gather) {
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) src[r] = p.gather[min(max(m_begin + r, 0), p.gather_len - 1)];
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) src[r] = min(max(src[r] / p.gather_div, 0), p.a_rows - 1);
  } else {
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) src[r] = min(max(m_begin + r, 0), p.a_rows - 1);
  }

  const int K = p.K, nchunks = (K + 127) / 128, stride = mx_row_bytes(K), ks = K / 32;
  const int a_bytes = rows_cap * stride;
  const int s_bytes = (int)splitk_scale_bytes(NB, K);
  uint8_t* s_lds = lds + a_bytes;                                   // [NB][16 rows][ks]
  f32x4_t* red = reinterpret_cast<f32x4_t*>(lds + a_bytes + ((s_bytes + 15) & ~15));  // [W-1][NB][64]
  const int row_q = W8 ? K : K / 2;  // code bytes per weight row
  const uint32_t qbytes = (uint32_t)(p.b_expert_rows * row_q);
  const uint32_t sbytes = (uint32_t)(p.b_expert_rows * ks);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.bq + (int64_t)e * qbytes, qbytes);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.bs + (int64_t)e * sbytes, sbytes);

  // staging loads first: scales of the block's rows and the first pass of
  // activation row 0 (one 16-byte piece or one 32-value block per thread)
  const int s_pieces = s_bytes / 16;
  const int si = threadIdx.x;
  u32x4_t sv[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = si + nthreads * j;
    const int half = i / (s_pieces / NB), q = i - half * (s_pieces / NB);
    const uint32_t off = i < s_pieces ? (uint32_t)((n0 + half * p.b_row_second) * ks + 16 * q) : kOob;
    sv[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0));
  }
  // activation rows: AMX copies 16-byte pieces, else converts 32-value blocks
  const int units = AMX ? stride / 16 : ks;  // per row
  const __amdgpu_buffer_rsrc_t ra = AMX ? make_rsrc(p.amx, (uint32_t)((int64_t)p.a_rows * stride))
                                        : make_rsrc(p.A, (uint32_t)((int64_t)p.a_rows * p.lda * 2));
  u32x4_t av[4];
  auto a_issue_row = [&](int sr, int unit) {
    if constexpr (AMX) {
      const uint32_t off = unit < units ? (uint32_t)(sr * stride + 16 * unit) : kOob;
      av[0] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)off, 0, 0));
    } else {
      const uint32_t off = unit < units ? (uint32_t)(((int64_t)sr * p.lda + 32 * unit) * 2) : kOob;
#pragma unroll
      for (int qq = 0; qq < 4; ++qq)
        av[qq] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)off, 16 * qq, 0));
    }
  };
  auto a_commit = [&](int r, int unit) {
    if (unit >= units) return;
    uint8_t* row = lds + r * stride;
    if constexpr (AMX) {
      *reinterpret_cast<u32x4_t*>(row + 16 * unit) = av[0];
    } else {
      float x[32];
      unpack_bf16x32(av, x);
      mx_convert_block(x, row + 32 * unit, row + K + 32 * unit, row + 2 * K + unit);
    }
  };
  a_issue_row(src[0], threadIdx.x);
  __builtin_amdgcn_sched_barrier(0);

  // this wave's weights: chunks [c_begin, c_begin + CPW)
  const int c_begin = wave * CPW;
  u32x4_t q[CPW][NB];
  u32x4_t q2[W8 ? CPW : 1][NB];  // MXFP8: the second 16-byte piece of each lane's codes
#pragma unroll
  for (int u = 0; u < CPW; ++u) {
    const int c = c_begin + u;
    const bool ok = c < nchunks && c * 128 + grp * 32 < K;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint32_t rb = (uint32_t)(n0 + col + nb * p.b_row_second) * (uint32_t)row_q;
      if constexpr (W8) {
        const uint32_t qo = ok ? rb + (uint32_t)(c * 128 + grp * 16) : kOob;
        const uint32_t qo2 = ok ? qo + 64u : kOob;
        q[u][nb] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)qo, 0, 0));
        q2[u][nb] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)qo2, 0, 0));
      } else {
        const uint32_t qo = ok ? rb + (uint32_t)(c * 64 + grp * 16) : kOob;
        q[u][nb] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)qo, 0, 0));
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);

#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int i = si + nthreads * j;
    if (i < s_pieces) *reinterpret_cast<u32x4_t*>(s_lds + 16 * i) = sv[j];
  }
  a_commit(0, threadIdx.x);
  // remaining activation pieces (row 0 beyond the first pass, rows 1..)
#pragma unroll
  for (int r = 0; r < kTileRows; ++r) {
    if (r >= rows) break;  // block-uniform
    for (int unit = (r == 0 ? nthreads : 0) + (int)threadIdx.x; unit - (int)threadIdx.x < units; unit += nthreads) {
      a_issue_row(src[r], unit);
      a_commit(r, unit);
    }
  }
  __syncthreads();

  f32x4_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const bool r_ok = col < rows;
  const uint8_t* row = lds + (r_ok ? col : 0) * stride;
#pragma unroll
  for (int u = 0; u < CPW; ++u) {
    const int c = c_begin + u;
    if (c >= nchunks) break;  // wave-uniform
    const int kb = c * 128;
    const bool h0 = r_ok && kb + 16 * grp < K, h1 = r_ok && kb + 64 + 16 * grp < K;
    const u32x4_t z = u32x4_t{0u, 0u, 0u, 0u};
    const u32x4_t a0 = h0 ? *reinterpret_cast<const u32x4_t*>(row + kb + 16 * grp) : z;
    const u32x4_t a1 = h1 ? *reinterpret_cast<const u32x4_t*>(row + kb + 64 + 16 * grp) : z;
    const u32x4_t l0 = h0 ? *reinterpret_cast<const u32x4_t*>(row + K + kb + 16 * grp) : z;
    const u32x4_t l1 = h1 ? *reinterpret_cast<const u32x4_t*>(row + K + kb + 64 + 16 * grp) : z;
    const int sa = (r_ok && kb + 32 * grp < K) ? (int)row[2 * K + kb / 32 + grp] : 127;
    const i32x8_t ahi = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    const i32x8_t alo = {(int)l0[0], (int)l0[1], (int)l0[2], (int)l0[3], (int)l1[0], (int)l1[1], (int)l1[2], (int)l1[3]};
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const bool sok = kb + 32 * grp < K;
      const int sb = sok ? (int)s_lds[(nb * 16 + col) * ks + kb / 32 + grp] : 127;
      if constexpr (W8) {
        acc[nb] = mfma_mx8(ahi, q[u][nb], q2[u][nb], sa, sb, acc[nb]);
        acc[nb] = mfma_mx8(alo, q[u][nb], q2[u][nb], sa, sb, acc[nb]);
      } else {
        acc[nb] = mfma_mx(ahi, q[u][nb], sa, sb, acc[nb]);
        acc[nb] = mfma_mx(alo, q[u][nb], sa, sb, acc[nb]);
      }
    }
  }
  const int nwaves = nthreads >> 6;
  if (wave > 0) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) red[((wave - 1) * NB + nb) * 64 + lane] = acc[nb];
  }
  __syncthreads();
  if (wave != 0) return;
  for (int w = 1; w < nwaves; ++w) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) acc[nb] += red[((w - 1) * NB + nb) * 64 + lane];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * grp + i;
    if (r < rows) {
      const float o = NB == 2 ? clamped_swiglu(acc[0][i], acc[NB - 1][i], limit) : acc[0][i];
      p.C[(int64_t)(m_begin + r) * p.ldc + n0 + col] = f32_to_bf16(o);
    }
  }
}

// LDS of one tile: the staged rows, bf16 or two-term MXFP8.
size_t gemv_lds_bytes(int rows_cap, int k_max, bool fp4) {
  return fp4 ? (size_t)rows_cap * mx_row_bytes(k_max) : gemv_bf16_lds_bytes(rows_cap, k_max);
}

namespace {

// Scales staged in LDS (SW = 0): the block's 64 rows per half, up to K = 5120
// (5 16-byte pieces per thread per half), when rows and scales fit in 64 KB.
constexpr size_t kMxMaxLds = 64 * 1024;
size_t mx_scale_lds_bytes(int nb, int K) { return (size_t)nb * 64 * (K / 32); }

template <int NB, bool AMX>
hipError_t launch_mx(const GemvProblem& p, int rows_cap, float limit, hipStream_t stream) {
  const dim3 grid((unsigned)(p.grid_tiles * ((p.N + 63) / 64)));
  const size_t shm = gemv_lds_bytes(rows_cap, p.K, true);
  const size_t shm_s = shm + mx_scale_lds_bytes(NB, p.K);
  if (p.w8) {
    // MXFP8 weights: K a multiple of 128 (whole 32-code pieces per lane); the
    // MXFP8 output rows (cmx) exist for the MXFP4 form only
    if (p.K % 128 != 0 || p.cmx) return hipErrorInvalidValue;
    if (p.K <= 5120 && shm_s <= kMxMaxLds)
      hipLaunchKernelGGL((expert_gemv_mx_kernel<NB, 0, AMX, true>), grid, dim3(256), shm_s, stream, p, rows_cap,
                         limit);
    else if (p.K % 512 == 0)
      hipLaunchKernelGGL((expert_gemv_mx_kernel<NB, 16, AMX, true>), grid, dim3(256), shm, stream, p, rows_cap, limit);
    else
      hipLaunchKernelGGL((expert_gemv_mx_kernel<NB, 4, AMX, true>), grid, dim3(256), shm, stream, p, rows_cap, limit);
    return hipGetLastError();
  }
  if (p.K <= 5120 && p.K % 128 == 0 && shm_s <= kMxMaxLds)
    hipLaunchKernelGGL((expert_gemv_mx_kernel<NB, 0, AMX>), grid, dim3(256), shm_s, stream, p, rows_cap, limit);
  else if (p.K % 512 == 0)
    hipLaunchKernelGGL((expert_gemv_mx_kernel<NB, 16, AMX>), grid, dim3(256), shm, stream, p, rows_cap, limit);
  else if (p.K % 256 == 0)
    hipLaunchKernelGGL((expert_gemv_mx_kernel<NB, 8, AMX>), grid, dim3(256), shm, stream, p, rows_cap, limit);
  else if (p.K % 128 == 0)
    hipLaunchKernelGGL((expert_gemv_mx_kernel<NB, 4, AMX>), grid, dim3(256), shm, stream, p, rows_cap, limit);
  else
    hipLaunchKernelGGL((expert_gemv_mx_kernel<NB, 1, AMX>), grid, dim3(256), shm, stream, p, rows_cap, limit);
  return hipGetLastError();
}

template <int NB, int CPW, bool AMX>
hipError_t launch_splitk(const GemvProblem& p, int rows_cap, float limit, hipStream_t stream) {
  const int waves = ((p.K + 127) / 128 + CPW - 1) / CPW;
  const dim3 grid((unsigned)(p.grid_tiles * (p.N / 16)));
  const size_t s_bytes = ((size_t)NB * 16 * (p.K / 32) + 15) & ~size_t(15);
  const size_t shm = gemv_lds_bytes(rows_cap, p.K, true) + s_bytes + (size_t)(waves - 1) * NB * 64 * 16;
  if (p.w8) {
    if (p.K % 128 != 0) return hipErrorInvalidValue;
    hipLaunchKernelGGL((expert_gemv_splitk_kernel<NB, CPW, AMX, true>), grid, dim3(64 * waves), shm, stream, p,
                       rows_cap, limit);
  } else {
    hipLaunchKernelGGL((expert_gemv_splitk_kernel<NB, CPW, AMX>), grid, dim3(64 * waves), shm, stream, p, rows_cap,
                       limit);
  }
  return hipGetLastError();
}

}  // namespace

// Split-K few-token down projection (the gate/up projection measured faster
// on the 64-column kernel): usable when the rows of a tile, the block's scales
// and the wave partials fit in 64 KB and K needs at most 8 waves.
bool splitk_supported(int rows_cap, int K) {
  const int nb = 1, cpw = kSplitKChunksDown;
  const int waves = ((K + 127) / 128 + cpw - 1) / cpw;
  const size_t shm = gemv_lds_bytes(rows_cap, K, true) + (size_t)nb * 16 * (K / 32) + 16 + (size_t)(waves - 1) * nb * 1024;
  return rows_cap <= kTileRows && waves <= 8 && shm <= 64 * 1024;
}

hipError_t launch_expert_gemv_splitk(const GemvProblem& p, int rows_cap, hipStream_t stream) {
  if (p.grid_tiles == 0 || p.N == 0) return hipSuccess;
  return launch_splitk<1, kSplitKChunksDown, false>(p, rows_cap, 0.f, stream);
}

hipError_t launch_expert_gemv(const GemvParams& prm, bool swiglu, bool fp4, hipStream_t stream) {
  if (fp4) {
    // one problem per launch (p[1] unused)
    if (prm.p[0].grid_tiles == 0 || prm.p[0].N == 0) return hipSuccess;
    // pre-converted rows occur only for the gate/up projection
    if (swiglu)
      return prm.p[0].amx ? launch_mx<2, true>(prm.p[0], prm.rows_cap, prm.limit, stream)
                          : launch_mx<2, false>(prm.p[0], prm.rows_cap, prm.limit, stream);
    return launch_mx<1, false>(prm.p[0], prm.rows_cap, prm.limit, stream);
  }
  int k_max = prm.p[0].K;
  if (prm.p[1].grid_tiles > 0 && prm.p[1].K > k_max) k_max = prm.p[1].K;
  const size_t shm = gemv_lds_bytes(prm.rows_cap, k_max, false);
  dim3 grid((unsigned)(prm.p[0].grid_tiles * prm.p[0].col_tiles + prm.p[1].grid_tiles * prm.p[1].col_tiles));
  if (grid.x == 0) return hipSuccess;
  if (swiglu)
    hipLaunchKernelGGL((expert_gemv_bf16_kernel<true>), grid, dim3(256), shm, stream, prm);
  else
    hipLaunchKernelGGL((expert_gemv_bf16_kernel<false>), grid, dim3(256), shm, stream, prm);
  return hipGetLastError();
}

}  // namespace moe
