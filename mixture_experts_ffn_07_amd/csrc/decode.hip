// Few-token (decode) kernels around the routed weight-streaming projection:
//   decode_front_kernel  -- the router GEMV (scores) beside the shared
//                           expert's gate/up projection;
//   decode_mid_kernel    -- the routing block beside the shared expert's
//                           down projection.  The routing block computes the
//                           two-term MXFP8 form of x for the routed gate/up,
//                           the top-k of every token from the scores, and
//                           (one wave) the stable permutation and tile table
//                           of the T*k <= 64 slots;
//   down_combine_kernel  -- T <= 8: routed down projection with the weighted
//                           combine folded in (token-major: one block per 16
//                           output columns visits every selected expert and
//                           accumulates w * (h W_d^T) per token), plus the
//                           shared expert's output.
// The layer's steps are the router with top-k and renormalised weights
// (score_func sqrtsoftplus, route_scale: checkpoint config.json on the
// "DeepSeek V4.1" atlas page), the gated-MLP experts and the combine.
#include "moe_device.h"
#include "moe_internal.h"
#include "mx_device.h"
#include "router_device.h"
#include "gemv_bf16_device.h"
#include "gemv_valu_device.h"

namespace moe {

// ---------------------------------------------------------------- routing
// x -> two-term MXFP8 rows (mx_device.h): one thread per block of 32 values,
// items i = first + k * stride (k = 0, 1, ...), loads first.
__device__ __forceinline__ void convert_x_mx(const uint16_t* x, uint8_t* xmx, int tokens, int hidden, int first,
                                             int stride) {
  const int nblk = hidden / 32, row_stride = mx_row_bytes(hidden);
  const int total = tokens * nblk;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)tokens * hidden * 2);
  for (int i = first; i < total; i += stride) {
    const int r = i / nblk, b = i - r * nblk;
    u32x4_t v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      v[q] = __builtin_bit_cast(u32x4_t,
                                __builtin_amdgcn_raw_buffer_load_b128(rx, (int)((r * hidden + 32 * b) * 2), 16 * q, 0));
    float xv[32];
    unpack_bf16x32(v, xv);
    uint8_t* row = xmx + (int64_t)r * row_stride;
    mx_convert_block(xv, row + 32 * b, row + hidden + 32 * b, row + 2 * hidden + b);
  }
}

template <int MPL>
__device__ __forceinline__ void route_small_block(const RouteSmallParams& p) {
  __shared__ int32_t idx_sh[64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = p.tokens * p.top_k;
  // the routing is a chain of dependent wave reductions on a CU shared with
  // streaming waves: highest issue priority for this block's waves
  __builtin_amdgcn_s_setprio(3);

  // x -> MXFP8 rows (when launch 1 has not made them); items are dealt from
  // the last thread down, so the first waves, which also run the top-k
  // below, get the least conversion work
  if (p.xmx) convert_x_mx(p.x, p.xmx, p.tokens, p.hidden, 255 - (int)threadIdx.x, 256);

  // top-k of each token from its scores (s at scores[t], s + bias at scores[T + t]);
  // past four tokens a wave takes tokens t and t + 4 together
  if (p.tokens <= 4) {
    for (int t = wave; t < p.tokens; t += 4)
      topk_token<MPL, true>(p.scores + (size_t)t * p.n_experts, 1, 0, nullptr, p.n_experts, p.top_k, p.route_scale,
                            p.idx + (size_t)t * p.top_k, p.w + (size_t)t * p.top_k, nullptr, idx_sh + t * p.top_k,
                            p.scores + (size_t)(p.tokens + t) * p.n_experts);
  } else {
    for (int t0 = wave; t0 < p.tokens; t0 += 8) {
      const bool two = t0 + 4 < p.tokens;
      const int t1 = two ? t0 + 4 : t0;
      const float* const s_row[2] = {p.scores + (size_t)t0 * p.n_experts, p.scores + (size_t)t1 * p.n_experts};
      const float* const u_row[2] = {p.scores + (size_t)(p.tokens + t0) * p.n_experts,
                                     p.scores + (size_t)(p.tokens + t1) * p.n_experts};
      int32_t* const idx_row[2] = {p.idx + (size_t)t0 * p.top_k, p.idx + (size_t)t1 * p.top_k};
      float* const w_row[2] = {p.w + (size_t)t0 * p.top_k, p.w + (size_t)t1 * p.top_k};
      int32_t* const idx_l[2] = {idx_sh + t0 * p.top_k, idx_sh + t1 * p.top_k};
      topk_token_pair<MPL>(s_row, u_row, two, p.n_experts, p.top_k, p.route_scale, idx_row, w_row, idx_l);
    }
  }
  __syncthreads();
  if (wave != 0) return;

  // permutation of the n <= 64 flat slots, one per lane: position = number of
  // slots with a smaller expert id, plus earlier slots with the same id
  const int e = lane < n ? idx_sh[lane] : 0x7fffffff;
  int pos = 0, dup_before = 0, count = 0;
  for (int j = 0; j < n; ++j) {
    const int ej = __builtin_amdgcn_readlane(e, j);
    pos += (ej < e) || (ej == e && j < lane);
    dup_before += (ej == e && j < lane);
    count += (ej == e);
  }
  const bool first = lane < n && dup_before == 0;  // first slot of its expert
  const uint64_t firsts = __ballot(first);
  int distinct_smaller = 0;
  for (int j = 0; j < n; ++j) {
    const int ej = __builtin_amdgcn_readlane(e, j);
    distinct_smaller += (((firsts >> j) & 1ull) && ej < e);
  }
  if (lane < n) {
    p.sorted_slots[pos] = lane;
    p.slot_pos[lane] = pos;
  }
  if (first && distinct_smaller < p.max_tiles) {
    GemmTile tl;
    tl.e = e;
    tl.m_begin = pos;
    tl.m_end = pos + count;
    tl.pad = 0;
    p.tiles[distinct_smaller] = tl;
  }
  // token of each tile row (row = rank of the slot among its expert's slots;
  // an expert has at most T <= 8 rows)
  if (p.tile_rows && lane < n && distinct_smaller < p.max_tiles && dup_before < kTileRows)
    p.tile_rows[distinct_smaller * kTileRows + dup_before] = lane / p.top_k;
  const int n_tiles = min((int)__popcll(firsts), p.max_tiles);
  if (lane == 0) *p.tile_count = n_tiles;
  // the remaining records are written empty, so readers need not load the count
  if (lane >= n_tiles && lane < p.max_tiles) p.tiles[lane] = GemmTile{0, 0, 0, 0};
}

// Launch 1 of the few-token layer: the shared expert's gate/up blocks
// (longest first), then the router GEMV, one expert per wave, then (with
// f.xmx) the blocks that put x in two-term MXFP8 form for the routed gate/up,
// off the routing block's critical path in launch 2.
__global__ __launch_bounds__(256) void decode_front_kernel(FrontParams f) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int shared_blocks = f.shared.grid_tiles * f.shared.col_tiles;
  if ((int)blockIdx.x < shared_blocks) {
    gemv_bf16_block<true>(f.shared, blockIdx.x, f.rows_cap, f.limit, lds);
    return;
  }
  const int router_blocks = (f.n_experts + 3) / 4;
  const int rb = (int)blockIdx.x - shared_blocks;
  if (rb < router_blocks) {
    router_gemv_wave(f.x, f.router_w, nullptr, f.tokens, f.n_experts, f.hidden, f.scores, f.bias,
                     rb * 4 + (int)(threadIdx.x >> 6));
    return;
  }
  const int cb = rb - router_blocks, conv_blocks = (int)gridDim.x - shared_blocks - router_blocks;
  convert_x_mx(f.x, f.xmx, f.tokens, f.hidden, cb * 256 + (int)threadIdx.x, conv_blocks * 256);
}

// Launch 2: the routing block (block 0), then the shared expert's down
// projection blocks.
template <int MPL>
__global__ __launch_bounds__(256) void decode_mid_kernel(RouteSmallParams p, GemvProblem shared_down, int rows_cap) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  if (blockIdx.x == 0) {
    route_small_block<MPL>(p);
    return;
  }
  gemv_bf16_block<false>(shared_down, (int)blockIdx.x - 1, rows_cap, 0.f, lds);
}

// T <= kValuMaxTokens, hidden and shared inter <= 5120: the same two launches
// with every weight row streamed by one wave on the vector ALUs.
// Launch 1: the shared gate/up row pairs (gate row n and up row I_s + n per
// wave, then the clamped SwiGLU), then the router rows (scores s and u).
__global__ __launch_bounds__(256) void decode_front_valu_kernel(FrontValuParams f) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // x rows [T][hidden] bf16
  uint16_t* x_lds = reinterpret_cast<uint16_t*>(lds);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int H = f.hidden, T = f.tokens, Is = f.shared_inter;
  const int shared_blocks = f.sh_gu ? (Is + 3) / 4 : 0;
  float out2[2][kValuMaxTokens];
  if ((int)blockIdx.x < shared_blocks) {
    const int nrow = (int)blockIdx.x * 4 + wave;  // gate/up pair
    const bool ok = nrow < Is;
    const __amdgpu_buffer_rsrc_t rw = make_rsrc(f.sh_gu, (uint32_t)((int64_t)2 * Is * H * 2));
    const uint32_t off[2] = {ok ? (uint32_t)nrow * (uint32_t)H * 2u : kOob,
                             ok ? (uint32_t)(Is + nrow) * (uint32_t)H * 2u : kOob};
    ValuRows<8, 10, 2> st;
    valu_issue<8, 10, 2>(st, rw, off, H);
    valu_stage_rows(f.x, H, T, H, x_lds);
    __syncthreads();
    valu_compute<8, 10, 2, kValuMaxTokens>(st, x_lds, H, T, H, out2);
    if (lane == 0 && ok)
      for (int t = 0; t < T; ++t)
        f.h_sh[(int64_t)t * Is + nrow] = f32_to_bf16(clamped_swiglu(out2[0][t], out2[1][t], f.limit));
    return;
  }
  const int e = ((int)blockIdx.x - shared_blocks) * 4 + wave;
  const bool ok = e < f.n_experts;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(f.router_w, (uint32_t)((int64_t)f.n_experts * H * 4));
  const uint32_t off[1] = {ok ? (uint32_t)e * (uint32_t)H * 4u : kOob};
  ValuRows<4, 20, 1> st;
  valu_issue<4, 20, 1>(st, rw, off, H);
  valu_stage_rows(f.x, H, T, H, x_lds);
  __syncthreads();
  float out1[1][kValuMaxTokens];
  valu_compute<4, 20, 1, kValuMaxTokens>(st, x_lds, H, T, H, out1);
  if (lane == 0 && ok) {
    const float b = f.bias ? f.bias[e] : 0.f;
    for (int t = 0; t < T; ++t) {
      const float s = sqrtsoftplus(out1[0][t]);
      f.scores[(int64_t)t * f.n_experts + e] = s;
      f.scores[(int64_t)(T + t) * f.n_experts + e] = s + b;
    }
  }
}

// Launch 2: the routing block (block 0), then the shared down rows (two per
// wave) from the SwiGLU rows of launch 1.
template <int MPL, int KVD>
__global__ __launch_bounds__(256) void decode_mid_valu_kernel(RouteSmallParams p, MidValuParams m) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // h_sh rows [T][shared_inter] bf16
  if (blockIdx.x == 0) {
    route_small_block<MPL>(p);
    return;
  }
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int H = m.hidden, Is = m.shared_inter, T = m.tokens;
  const int n = (((int)blockIdx.x - 1) * 4 + wave) * 2;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(m.sh_dn, (uint32_t)((int64_t)H * Is * 2));
  const uint32_t off[2] = {n < H ? (uint32_t)n * (uint32_t)Is * 2u : kOob,
                           n + 1 < H ? (uint32_t)(n + 1) * (uint32_t)Is * 2u : kOob};
  ValuRows<8, KVD, 2> st;
  valu_issue<8, KVD, 2>(st, rw, off, Is);
  uint16_t* h_lds = reinterpret_cast<uint16_t*>(lds);
  valu_stage_rows(m.h_sh, Is, T, Is, h_lds);
  __syncthreads();
  float out[2][kValuMaxTokens];
  valu_compute<8, KVD, 2, kValuMaxTokens>(st, h_lds, Is, T, Is, out);
  if (lane == 0)
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int r = 0; r < 2; ++r)
        if (n + r < H) m.y_sh[(int64_t)t * H + n + r] = f32_to_bf16(out[r][t]);
}

// Launch 2 of the streaming few-token layer (T <= kValuMaxTokens; launch 1 is
// the router GEMV writing the scores): block 0 routes, the other blocks
// compute the shared gate/up row pairs, so the routing latency hides behind
// the shared expert's weight stream.
template <int MPL>
__global__ __launch_bounds__(256) void decode_route_shared_gu_kernel(FrontValuParams f, RouteSmallParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // x rows [T][hidden] bf16
  if (blockIdx.x == 0) {
    route_small_block<MPL>(p);
    return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  shared_gate_up_pair(f.x, f.sh_gu, f.h_sh, f.tokens, f.hidden, f.shared_inter, f.limit,
                      ((int)blockIdx.x - 1) * 4 + wave, reinterpret_cast<uint16_t*>(lds));
}

bool decode_valu_supported(int tokens, int hidden, int shared_inter) {
  return tokens <= kValuMaxTokens && hidden <= 5120 && shared_inter <= 5120;
}

hipError_t launch_decode_front_valu(const FrontValuParams& f, hipStream_t stream) {
  const int shared_blocks = f.sh_gu ? (f.shared_inter + 3) / 4 : 0;
  const dim3 grid((unsigned)(shared_blocks + (f.n_experts + 3) / 4));
  hipLaunchKernelGGL(decode_front_valu_kernel, grid, dim3(256), (size_t)f.tokens * f.hidden * 2, stream, f);
  return hipGetLastError();
}

hipError_t launch_decode_mid_valu(const RouteSmallParams& p, const MidValuParams& m, hipStream_t stream) {
  const int nj = (p.n_experts + 63) / 64;
  const bool small = m.shared_inter <= 2560;  // 5 vectors of 8 per lane cover a row
  auto kern = nj <= 2   ? (small ? decode_mid_valu_kernel<2, 5> : decode_mid_valu_kernel<2, 10>)
              : nj <= 4 ? (small ? decode_mid_valu_kernel<4, 5> : decode_mid_valu_kernel<4, 10>)
              : nj <= 6 ? (small ? decode_mid_valu_kernel<6, 5> : decode_mid_valu_kernel<6, 10>)
              : nj <= 8 ? (small ? decode_mid_valu_kernel<8, 5> : decode_mid_valu_kernel<8, 10>)
                        : (small ? decode_mid_valu_kernel<16, 5> : decode_mid_valu_kernel<16, 10>);
  const int shared_blocks = m.sh_dn ? (m.hidden + 7) / 8 : 0;
  hipLaunchKernelGGL(kern, dim3((unsigned)(1 + shared_blocks)), dim3(256),
                     (size_t)m.tokens * (m.shared_inter > 0 ? m.shared_inter : 8) * 2, stream, p, m);
  return hipGetLastError();
}

hipError_t launch_decode_route_shared_gu(const FrontValuParams& f, const RouteSmallParams& p, hipStream_t stream) {
  const int nj = (p.n_experts + 63) / 64;
  auto kern = nj <= 2   ? decode_route_shared_gu_kernel<2>
              : nj <= 4 ? decode_route_shared_gu_kernel<4>
              : nj <= 6 ? decode_route_shared_gu_kernel<6>
              : nj <= 8 ? decode_route_shared_gu_kernel<8>
                        : decode_route_shared_gu_kernel<16>;
  const int shared_blocks = f.sh_gu ? (f.shared_inter + 3) / 4 : 0;
  hipLaunchKernelGGL(kern, dim3((unsigned)(1 + shared_blocks)), dim3(256), (size_t)f.tokens * f.hidden * 2, stream,
                     f, p);
  return hipGetLastError();
}

hipError_t launch_decode_front(const FrontParams& f, hipStream_t stream) {
  const int shared_blocks = f.shared.grid_tiles * f.shared.col_tiles;
  const int conv_blocks = f.xmx ? (f.tokens * (f.hidden / 32) + 255) / 256 : 0;
  const dim3 grid((unsigned)(shared_blocks + (f.n_experts + 3) / 4 + conv_blocks));
  const size_t shm = shared_blocks ? gemv_bf16_lds_bytes(f.rows_cap, f.shared.K) : 0;
  hipLaunchKernelGGL(decode_front_kernel, grid, dim3(256), shm, stream, f);
  return hipGetLastError();
}

hipError_t launch_decode_mid(const RouteSmallParams& p, const GemvProblem& shared_down, int rows_cap,
                             hipStream_t stream) {
  const int nj = (p.n_experts + 63) / 64;
  auto kern = nj <= 2 ? decode_mid_kernel<2>
              : nj <= 4 ? decode_mid_kernel<4>
              : nj <= 6 ? decode_mid_kernel<6>
              : nj <= 8 ? decode_mid_kernel<8>
                        : decode_mid_kernel<16>;
  const int shared_blocks = shared_down.grid_tiles * shared_down.col_tiles;
  const size_t shm = shared_blocks ? gemv_bf16_lds_bytes(rows_cap, shared_down.K) : 0;
  hipLaunchKernelGGL(kern, dim3((unsigned)(1 + shared_blocks)), dim3(256), shm, stream, p, shared_down, rows_cap);
  return hipGetLastError();
}

// ---------------------------------------------------------------- down + combine
namespace {

// Work unit = (tile, group of G consecutive 128-wide chunks of K); unit u of
// the block goes to wave u % 4.  A scale load of 4G bytes covers a group's
// scales.  kDcUnitRegs bounds the registers of the loads a wave keeps in
// flight, so one round covers 14 units at G = 2 (all 54 of a block at one
// token with inter 2304).
constexpr int kDcUnitRegs = 140;
template <int G>
struct DcShape {
  static constexpr int kUnits = kDcUnitRegs / (5 * G);  // units per wave per round
};

template <int G>
struct DcUnit {
  u32x4_t q[G];
  uint32_t s[G];
};

template <int G>
__device__ __forceinline__ void dc_load_unit(DcUnit<G>& b, const DownCombineParams& p, bool ok, int e, int g,
                                             int n0, int col, int grp) {
  const int nchunks = (p.inter + 127) / 128;
  const uint32_t qbytes = (uint32_t)p.hidden * (uint32_t)(p.inter / 2);
  const uint32_t sbytes = (uint32_t)p.hidden * (uint32_t)(p.inter / 32);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.dn_q + (int64_t)e * qbytes, qbytes);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.dn_s + (int64_t)e * sbytes, sbytes);
  const uint32_t row = (uint32_t)(n0 + col);
  const uint32_t qrow = row * (uint32_t)(p.inter / 2), srow = row * (uint32_t)(p.inter / 32);
  const int c0 = g * G;
#pragma unroll
  for (int u = 0; u < G; ++u) {
    const int c = c0 + u;
    const bool okc = ok && c < nchunks && c * 128 + grp * 32 < p.inter;
    const uint32_t qo = okc ? qrow + (uint32_t)(c * 64 + grp * 16) : kOob;
    b.q[u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)qo, 0, 0));
  }
  const uint32_t so = (ok && c0 < nchunks) ? srow + (uint32_t)(4 * c0) : kOob;
  if constexpr (G == 4) {
    const u32x4_t w = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)so, 0, 0));
#pragma unroll
    for (int u = 0; u < 4; ++u) b.s[u] = w[u];
  } else if constexpr (G == 2) {
    const auto w = __builtin_amdgcn_raw_buffer_load_b64(rs, (int)so, 0, 0);
    b.s[0] = w[0];
    b.s[1] = w[1];
  } else {
    const bool okb = ok && c0 < nchunks && c0 * 128 + grp * 32 < p.inter;
    const uint32_t sob = okb ? srow + (uint32_t)(4 * c0 + grp) : kOob;
    b.s[0] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rs, (int)sob, 0, 0) << (8 * grp);
  }
}

}  // namespace

// grid: hidden / 16 blocks of 256 threads (16 output columns each).  Each
// wave adds w * (partial product of its units) into per-token sums; the
// sums of the 4 lane groups and 4 waves are added in a fixed order at the
// end, then the shared expert's output.
template <int G>
__global__ __launch_bounds__(256) void down_combine_kernel(DownCombineParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // n MX rows of h
  __shared__ int32_t tile_e[64], tile_b[64], tile_r[64];
  __shared__ int32_t slot_tok[64];
  __shared__ float slot_w[64];
  __shared__ int32_t tile_n;
  __shared__ float red[4][4][kDownCombineMaxTokens][16];
  constexpr int U = DcShape<G>::kUnits;
  // the wave index and everything derived from it are wave-uniform: keep them scalar
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int n = p.tokens * p.top_k;
  const int K = p.inter, stride = mx_row_bytes(K), nchunks = (K + 127) / 128;
  const int ngroups = (nchunks + G - 1) / G;
  // tile table and slot table: every load issued before the first use
  if (threadIdx.x < 64) {
    const int t = threadIdx.x;
    const int tc = *p.tile_count;
    GemmTile tl = {0, 0, 0, 0};
    if (t < p.max_tiles) tl = p.tiles[t];
    const int f = t < n ? p.sorted_slots[t] : 0;  // flat slot at position t
    const int fc = min(max(f, 0), n - 1);
    const float w = t < n ? p.topk_w[fc] : 0.f;
    if (t == 0) tile_n = min(max(tc, 0), min(p.max_tiles, 64));
    tile_e[t] = min(max(tl.e, 0), p.n_experts - 1);
    tile_b[t] = min(max(tl.m_begin, 0), n);
    tile_r[t] = min(max(tl.m_end - tl.m_begin, 0), n - min(max(tl.m_begin, 0), n));
    slot_tok[t] = fc / p.top_k;
    slot_w[t] = w;
  }
  // the n MX rows of h (contiguous), first pass issued before the sync
  constexpr int kPiecesPerThread = 4;
  const int pieces = n * stride / 16;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.hmx, (uint32_t)(n * stride));
  u32x4_t hv[kPiecesPerThread];
  auto h_issue = [&](int base) {
#pragma unroll
    for (int j = 0; j < kPiecesPerThread; ++j) {
      const int i = base + (int)threadIdx.x + 256 * j;
      hv[j] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(
                                              ra, (int)(i < pieces ? (uint32_t)(16 * i) : kOob), 0, 0));
    }
  };
  auto h_commit = [&](int base) {
#pragma unroll
    for (int j = 0; j < kPiecesPerThread; ++j) {
      const int i = base + (int)threadIdx.x + 256 * j;
      if (i < pieces) *reinterpret_cast<u32x4_t*>(lds + 16 * i) = hv[j];
    }
  };
  h_issue(0);
  __syncthreads();
  const int tc = __builtin_amdgcn_readfirstlane(tile_n);
  const int n_units = tc * ngroups;

  float yp[kDownCombineMaxTokens];
#pragma unroll
  for (int t = 0; t < kDownCombineMaxTokens; ++t) yp[t] = 0.f;
  for (int base = 0; base < n_units; base += 4 * U) {
    DcUnit<G> b[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int u = base + wave + 4 * i;
      const int t = min(u / ngroups, 63);
      const int e = __builtin_amdgcn_readfirstlane(tile_e[t]);  // same for the whole wave
      dc_load_unit<G>(b[i], p, u < n_units, e, u - (u / ngroups) * ngroups, n0, col, grp);
    }
    if (base == 0) {  // block-uniform: the staged h is needed from here on
      h_commit(0);
      for (int hb = 256 * kPiecesPerThread; hb < pieces; hb += 256 * kPiecesPerThread) {
        h_issue(hb);
        h_commit(hb);
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int u = base + wave + 4 * i;
      if (u >= n_units) break;  // wave-uniform
      const int tt = u / ngroups, g = u - tt * ngroups;
      const int m_begin = __builtin_amdgcn_readfirstlane(tile_b[tt]);
      const int rows = __builtin_amdgcn_readfirstlane(tile_r[tt]);
      const bool r_ok = col < rows;
      const uint8_t* row = lds + (m_begin + (r_ok ? col : 0)) * stride;
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int uc = 0; uc < G; ++uc) {
        const int c = g * G + uc;
        if (c >= nchunks) break;
        const int kb = c * 128;
        const bool h0 = r_ok && kb + 16 * grp < K, h1 = r_ok && kb + 64 + 16 * grp < K;
        const u32x4_t z = u32x4_t{0u, 0u, 0u, 0u};
        const u32x4_t a0 = h0 ? *reinterpret_cast<const u32x4_t*>(row + kb + 16 * grp) : z;
        const u32x4_t a1 = h1 ? *reinterpret_cast<const u32x4_t*>(row + kb + 64 + 16 * grp) : z;
        const u32x4_t l0 = h0 ? *reinterpret_cast<const u32x4_t*>(row + K + kb + 16 * grp) : z;
        const u32x4_t l1 = h1 ? *reinterpret_cast<const u32x4_t*>(row + K + kb + 64 + 16 * grp) : z;
        const int sa = (r_ok && kb + 32 * grp < K) ? (int)row[2 * K + kb / 32 + grp] : 127;
        const int sb = (int)((b[i].s[uc] >> (8 * grp)) & 0xffu);
        const i32x8_t ahi = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                             (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
        const i32x8_t alo = {(int)l0[0], (int)l0[1], (int)l0[2], (int)l0[3],
                             (int)l1[0], (int)l1[1], (int)l1[2], (int)l1[3]};
        acc = mfma_mx(ahi, b[i].q[uc], sa, sb, acc);
        acc = mfma_mx(alo, b[i].q[uc], sa, sb, acc);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 4 * grp + q;
        if (r < rows) {
          const int pos = m_begin + r;
          const int tok = slot_tok[pos];
          const float contrib = slot_w[pos] * acc[q];
#pragma unroll
          for (int t2 = 0; t2 < kDownCombineMaxTokens; ++t2) yp[t2] += tok == t2 ? contrib : 0.f;
        }
      }
    }
  }
#pragma unroll
  for (int t2 = 0; t2 < kDownCombineMaxTokens; ++t2) red[wave][grp][t2][col] = yp[t2];
  __syncthreads();
  if (threadIdx.x < 16 * kDownCombineMaxTokens) {
    const int tok = threadIdx.x >> 4, c = threadIdx.x & 15;
    if (tok < p.tokens) {
      float s = 0.f;
      for (int w = 0; w < 4; ++w)
        for (int g = 0; g < 4; ++g) s += red[w][g][tok][c];
      if (p.y_shared) s += bf16_to_f32(p.y_shared[(int64_t)tok * p.hidden + n0 + c]);
      p.y[(int64_t)tok * p.hidden + n0 + c] = f32_to_bf16(s);
    }
  }
}

size_t down_combine_lds_bytes(int tokens, int top_k, int inter) {
  return (size_t)tokens * top_k * mx_row_bytes(inter);
}

hipError_t launch_down_combine(const DownCombineParams& p, hipStream_t stream) {
  const size_t shm = down_combine_lds_bytes(p.tokens, p.top_k, p.inter);
  const dim3 grid(p.hidden / 16);
  if (p.inter % 512 == 0)
    hipLaunchKernelGGL((down_combine_kernel<4>), grid, dim3(256), shm, stream, p);
  else if (p.inter % 256 == 0)
    hipLaunchKernelGGL((down_combine_kernel<2>), grid, dim3(256), shm, stream, p);
  else
    hipLaunchKernelGGL((down_combine_kernel<1>), grid, dim3(256), shm, stream, p);
  return hipGetLastError();
}

}  // namespace moe
