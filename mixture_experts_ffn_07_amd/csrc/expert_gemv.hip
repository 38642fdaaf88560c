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
// (mx_device.h), two MFMAs (hi, lo) per 128-wide chunk.  A wave owns 16
// output columns over all of K.  Scale bytes are fetched as whole words
// covering several chunks: per-chunk byte loads cost as much memory-pipe
// time as the code loads they accompany.
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
template <int NB>
struct MxBatch {
  u32x4_t q[kMxChunks][NB];
  uint32_t s[kMxChunks][NB];
};

struct MxView {
  __amdgpu_buffer_rsrc_t q, s;
  uint32_t qrow[2], srow[2];  // byte offsets of this lane's row(s); kOob for columns past N
  int K, nchunks;
};

// SW = bytes per scale load: 16 (K % 512 == 0), 8 (K % 256 == 0), 4
// (K % 128 == 0) or 1 (one byte per lane and chunk, any K % 32 == 0).  The
// wider loads bring the scales of 4, 2 or 1 chunks for all 4 lane groups
// at once; the row offsets are then multiples of the load width.
template <int NB, int SW>
__device__ __forceinline__ void mx_load(MxBatch<NB>& b, const MxView& v, int c0, int grp) {
#pragma unroll
  for (int u = 0; u < kMxChunks; ++u) {
    const int c = c0 + u;
    const bool ok = c < v.nchunks && c * 128 + grp * 32 < v.K;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const uint32_t qo = ok ? v.qrow[nb] + (uint32_t)(c * 64 + grp * 16) : kOob;
      b.q[u][nb] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(v.q, (int)qo, 0, 0));
    }
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    if constexpr (SW == 16) {
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
template <int NB>
__device__ __forceinline__ void mx_mma(const MxBatch<NB>& b, f32x4_t (&acc)[NB], const uint8_t* row, bool r_ok,
                                       int c0, const MxView& v, int grp) {
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
      const int sb = (int)((b.s[u][nb] >> (8 * grp)) & 0xffu);
      acc[nb] = mfma_mx(ahi, b.q[u][nb], sa, sb, acc[nb]);
      acc[nb] = mfma_mx(alo, b.q[u][nb], sa, sb, acc[nb]);
    }
  }
}

// MX staging of the tile's rows into LDS (row stride mx_row_bytes(K)).
// Copy mode (p.amx): 16-byte pieces of pre-converted rows, 3 per thread per
// pass.  Convert mode: one 32-value block of bf16 per thread per pass.
struct MxStage {
  u32x4_t v[4];
};

__device__ __forceinline__ void mx_stage_issue(const GemvProblem& p, const int (&src)[8], int rows, int pass,
                                               MxStage& s) {
  const int K = p.K, stride = mx_row_bytes(K);
  if (p.amx) {
    const int pieces = stride / 16, total = rows * pieces;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.amx, (uint32_t)((int64_t)p.a_rows * stride));
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int i = pass * 768 + (int)threadIdx.x + 256 * j;
      int r = 0;
#pragma unroll
      for (int rr = 1; rr < 8; ++rr) r += i >= rr * pieces;
      int sr = src[0];
#pragma unroll
      for (int rr = 1; rr < 8; ++rr) sr = rr == r ? src[rr] : sr;
      const uint32_t off = i < total ? (uint32_t)(sr * stride + 16 * (i - r * pieces)) : kOob;
      s.v[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)off, 0, 0));
    }
  } else {
    const int nblk = K / 32, total = rows * nblk;
    const int i = pass * 256 + (int)threadIdx.x;
    int r = 0;
#pragma unroll
    for (int rr = 1; rr < 8; ++rr) r += i >= rr * nblk;
    int sr = src[0];
#pragma unroll
    for (int rr = 1; rr < 8; ++rr) sr = rr == r ? src[rr] : sr;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, (uint32_t)((int64_t)p.a_rows * p.lda * 2));
    const uint32_t off = i < total ? (uint32_t)(((int64_t)sr * p.lda + 32 * (i - r * nblk)) * 2) : kOob;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      s.v[q] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)off, 16 * q, 0));
  }
}

__device__ __forceinline__ void mx_stage_commit(const GemvProblem& p, int rows, int pass, const MxStage& s,
                                                uint8_t* lds) {
  const int K = p.K, stride = mx_row_bytes(K);
  if (p.amx) {
    const int total = rows * (stride / 16);
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int i = pass * 768 + (int)threadIdx.x + 256 * j;
      if (i < total) *reinterpret_cast<u32x4_t*>(lds + 16 * i) = s.v[j];  // rows are contiguous
    }
  } else {
    const int nblk = K / 32, total = rows * nblk;
    const int i = pass * 256 + (int)threadIdx.x;
    if (i < total) {
      const int r = i / nblk, b = i - r * nblk;
      float x[32];
      unpack_bf16x32(s.v, x);
      uint8_t* row = lds + r * stride;
      mx_convert_block(x, row + 32 * b, row + K + 32 * b, row + 2 * K + b);
    }
  }
}

__device__ __forceinline__ int mx_stage_passes(const GemvProblem& p, int rows) {
  const int K = p.K;
  return p.amx ? (rows * (mx_row_bytes(K) / 16) + 767) / 768 : (rows * (K / 32) + 255) / 256;
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
template <int NB, int SW>
__global__ __launch_bounds__(256) void expert_gemv_mx_kernel(GemvProblem p, int rows_cap, float limit) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int tile = blockIdx.x % p.grid_tiles;
  const int n0 = (blockIdx.x / p.grid_tiles) * 64 + wave * 16;
  int e = 0, m_begin, rows;
  if (p.tiles) {
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
  int src[8];
  if (p.gather) {
#pragma unroll
    for (int r = 0; r < 8; ++r) src[r] = p.gather[min(max(m_begin + r, 0), p.gather_len - 1)];
#pragma unroll
    for (int r = 0; r < 8; ++r) src[r] = min(max(src[r] / p.gather_div, 0), p.a_rows - 1);
  } else {
#pragma unroll
    for (int r = 0; r < 8; ++r) src[r] = min(max(m_begin + r, 0), p.a_rows - 1);
  }

  const int K = p.K;
  MxView v;
  v.K = K;
  v.nchunks = (K + 127) / 128;
  const uint32_t qbytes = (uint32_t)(p.b_expert_rows * (K / 2));
  const uint32_t sbytes = (uint32_t)(p.b_expert_rows * (K / 32));
  v.q = make_rsrc(p.bq + (int64_t)e * qbytes, qbytes);
  v.s = make_rsrc(p.bs + (int64_t)e * sbytes, sbytes);
  const bool n_ok = n0 < p.N;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const uint32_t r = (uint32_t)(n0 + col + nb * p.b_row_second);
    v.qrow[nb] = n_ok ? r * (uint32_t)(K / 2) : kOob;
    v.srow[nb] = n_ok ? r * (uint32_t)(K / 32) : kOob;
  }

  MxStage st;
  mx_stage_issue(p, src, rows, 0, st);
  __builtin_amdgcn_sched_barrier(0);  // staging loads go out before the weight prefetch
  MxBatch<NB> b0, b1;
  mx_load<NB, SW>(b0, v, 0, grp);
  mx_load<NB, SW>(b1, v, kMxChunks, grp);
  __builtin_amdgcn_sched_barrier(0);
  mx_stage_commit(p, rows, 0, st, lds);
  const int passes = mx_stage_passes(p, rows);
  for (int pass = 1; pass < passes; ++pass) {
    mx_stage_issue(p, src, rows, pass, st);
    mx_stage_commit(p, rows, pass, st, lds);
  }
  __syncthreads();

  f32x4_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const bool r_ok = col < rows;
  const uint8_t* row = lds + (r_ok ? col : 0) * mx_row_bytes(K);
  constexpr int CB = kMxChunks;
  for (int c = 0; c < v.nchunks; c += 2 * CB) {
    mx_mma<NB>(b0, acc, row, r_ok, c, v, grp);
    if (c + CB >= v.nchunks) break;
    mx_load<NB, SW>(b0, v, c + 2 * CB, grp);
    mx_mma<NB>(b1, acc, row, r_ok, c + CB, v, grp);
    mx_load<NB, SW>(b1, v, c + 3 * CB, grp);
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

// LDS of one tile: the staged rows, bf16 or two-term MXFP8.
size_t gemv_lds_bytes(int rows_cap, int k_max, bool fp4) {
  return fp4 ? (size_t)rows_cap * mx_row_bytes(k_max) : gemv_bf16_lds_bytes(rows_cap, k_max);
}

namespace {

template <int NB>
hipError_t launch_mx(const GemvProblem& p, int rows_cap, float limit, hipStream_t stream) {
  const dim3 grid((unsigned)(p.grid_tiles * ((p.N + 63) / 64)));
  const size_t shm = gemv_lds_bytes(rows_cap, p.K, true);
  if (p.K % 512 == 0)
    hipLaunchKernelGGL((expert_gemv_mx_kernel<NB, 16>), grid, dim3(256), shm, stream, p, rows_cap, limit);
  else if (p.K % 256 == 0)
    hipLaunchKernelGGL((expert_gemv_mx_kernel<NB, 8>), grid, dim3(256), shm, stream, p, rows_cap, limit);
  else if (p.K % 128 == 0)
    hipLaunchKernelGGL((expert_gemv_mx_kernel<NB, 4>), grid, dim3(256), shm, stream, p, rows_cap, limit);
  else
    hipLaunchKernelGGL((expert_gemv_mx_kernel<NB, 1>), grid, dim3(256), shm, stream, p, rows_cap, limit);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_expert_gemv(const GemvParams& prm, bool swiglu, bool fp4, hipStream_t stream) {
  if (fp4) {
    // one problem per launch (p[1] unused)
    if (prm.p[0].grid_tiles == 0 || prm.p[0].N == 0) return hipSuccess;
    return swiglu ? launch_mx<2>(prm.p[0], prm.rows_cap, prm.limit, stream)
                  : launch_mx<1>(prm.p[0], prm.rows_cap, prm.limit, stream);
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
