// Few-token (decode) kernels that sit around the weight-streaming projections:
//   route_small_kernel   -- one block: two-term MXFP8 form of x for the
//                           routed gate/up, top-k of every token from the
//                           scores the router GEMV computed, and (one wave)
//                           the stable permutation and tile table of the
//                           T*k <= 64 slots;
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
#include "topk_device.h"

namespace moe {

// ---------------------------------------------------------------- routing
template <int MPL>
__global__ __launch_bounds__(256) void route_small_kernel(RouteSmallParams p) {
  __shared__ int32_t idx_sh[64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = p.tokens * p.top_k;

  // x -> MXFP8 rows: one thread per block of 32 values, loads first
  if (p.xmx) {
    const int nblk = p.hidden / 32, stride = mx_row_bytes(p.hidden);
    const int total = p.tokens * nblk;
    const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x, (uint32_t)p.tokens * p.hidden * 2);
    // items are dealt from the last thread down, so the first waves, which
    // also run the top-k below, get the least conversion work
    for (int i = 255 - (int)threadIdx.x; i < total; i += 256) {
      const int r = i / nblk, b = i - r * nblk;
      u32x4_t v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        v[q] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)((r * p.hidden + 32 * b) * 2), 16 * q, 0));
      float xv[32];
      unpack_bf16x32(v, xv);
      uint8_t* row = p.xmx + (int64_t)r * stride;
      mx_convert_block(xv, row + 32 * b, row + p.hidden + 32 * b, row + 2 * p.hidden + b);
    }
  }

  // top-k of each token from its scores (s at scores[t], s + bias at scores[T + t])
  for (int t = wave; t < p.tokens; t += 4)
    topk_token<MPL, true>(p.scores + (size_t)t * p.n_experts, 1, 0, nullptr, p.n_experts, p.top_k, p.route_scale,
                          p.idx + (size_t)t * p.top_k, p.w + (size_t)t * p.top_k, nullptr, idx_sh + t * p.top_k,
                          p.scores + (size_t)(p.tokens + t) * p.n_experts);
  __syncthreads();
  if (wave != 0) return;

  // permutation of the n <= 64 flat slots, one per lane: position = number of
  // slots with a smaller expert id, plus earlier slots with the same id
  const int e = lane < n ? idx_sh[lane] : 0x7fffffff;
  int pos = 0, dup_before = 0, count = 0;
  for (int j = 0; j < n; ++j) {
    const int ej = __shfl(e, j, 64);
    pos += (ej < e) || (ej == e && j < lane);
    dup_before += (ej == e && j < lane);
    count += (ej == e);
  }
  const bool first = lane < n && dup_before == 0;  // first slot of its expert
  int distinct_smaller = 0;
  for (int j = 0; j < n; ++j) {
    const int ej = __shfl(e, j, 64);
    const bool fj = __shfl((int)first, j, 64) != 0;
    distinct_smaller += (fj && ej < e);
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
  const uint64_t firsts = __ballot(first);
  if (lane == 0) *p.tile_count = min((int)__popcll(firsts), p.max_tiles);
}

hipError_t launch_route_small(const RouteSmallParams& p, hipStream_t stream) {
  const int nj = (p.n_experts + 63) / 64;
  auto kern = nj <= 2 ? route_small_kernel<2>
              : nj <= 4 ? route_small_kernel<4>
              : nj <= 8 ? route_small_kernel<8>
                        : route_small_kernel<16>;
  hipLaunchKernelGGL(kern, dim3(1), dim3(256), 0, stream, p);
  return hipGetLastError();
}

// ---------------------------------------------------------------- down + combine
namespace {

constexpr int kDcChunks = 5;  // 128-wide chunks per wave per expert (inter <= 2560)

struct DcBatch {
  u32x4_t q[kDcChunks];
  uint32_t s[kDcChunks];
};

__device__ __forceinline__ void dc_load(DcBatch& b, const DownCombineParams& p, int tile, int tc, int n0, int col,
                                        int wave, int grp, const int32_t* tile_e) {
  const int nchunks = (p.inter + 127) / 128;
  const bool tile_ok = tile < tc;
  const int e = tile_ok ? tile_e[tile] : 0;
  const uint32_t qbytes = (uint32_t)p.hidden * (uint32_t)(p.inter / 2);
  const uint32_t sbytes = (uint32_t)p.hidden * (uint32_t)(p.inter / 32);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.dn_q + (int64_t)e * qbytes, qbytes);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.dn_s + (int64_t)e * sbytes, sbytes);
  const uint32_t row = (uint32_t)(n0 + col);
#pragma unroll
  for (int u = 0; u < kDcChunks; ++u) {
    const int c = wave + 4 * u;
    const int k0 = c * 128 + grp * 32;
    const bool ok = tile_ok && c < nchunks && k0 < p.inter;
    const uint32_t qo = ok ? row * (uint32_t)(p.inter / 2) + (uint32_t)(k0 / 2) : kOob;
    const uint32_t so = ok ? row * (uint32_t)(p.inter / 32) + (uint32_t)(k0 / 32) : kOob;
    b.q[u] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)qo, 0, 0));
    b.s[u] = __builtin_amdgcn_raw_buffer_load_b8(rs, (int)so, 0, 0);
  }
}

}  // namespace

// grid: hidden / 16 blocks of 256 threads.  The 4 waves split the inter
// dimension; each wave keeps per-token partial sums of w * o for its 16
// columns, added over the experts in tile (expert id) order; the partials
// of the 4 lane groups and 4 waves are added in a fixed order at the end,
// then the shared expert's output.
__global__ __launch_bounds__(256) void down_combine_kernel(DownCombineParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // n staged MXFP8 rows of h
  __shared__ int32_t tile_e[64], tile_b[64], tile_r[64];
  __shared__ int32_t slot_tok[64];
  __shared__ float slot_w[64];
  __shared__ float red[4][4][kDownCombineMaxTokens][16];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int n = p.tokens * p.top_k;
  const int tc = min(*p.tile_count, 64);
  if (threadIdx.x < 64) {
    const int t = threadIdx.x;
    if (t < tc) {
      const GemmTile tl = p.tiles[t];
      tile_e[t] = min(max(tl.e, 0), p.n_experts - 1);
      tile_b[t] = min(max(tl.m_begin, 0), n);
      tile_r[t] = min(max(tl.m_end - tl.m_begin, 0), n - tile_b[t]);
    }
    if (t < n) {
      const int f = min(max(p.sorted_slots[t], 0), n - 1);  // flat slot at position t
      slot_tok[t] = f / p.top_k;
      slot_w[t] = p.topk_w[f];
    }
  }
  __syncthreads();
  DcBatch b0, b1;
  dc_load(b0, p, 0, tc, n0, col, wave, grp, tile_e);
  dc_load(b1, p, 1, tc, n0, col, wave, grp, tile_e);
  // stage h (n rows) as two-term MXFP8
  {
    const int nblk = p.inter / 32, stride = mx_row_bytes(p.inter);
    const int total = n * nblk;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.h, (uint32_t)n * p.inter * 2);
    for (int i = threadIdx.x; i < total; i += 256) {
      const int r = i / nblk, b = i - r * nblk;
      u32x4_t v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        v[q] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)((r * p.inter + 32 * b) * 2), 16 * q, 0));
      float xv[32];
      unpack_bf16x32(v, xv);
      uint8_t* row = lds + r * stride;
      mx_convert_block(xv, row + 32 * b, row + p.inter + 32 * b, row + 2 * p.inter + b);
    }
  }
  __syncthreads();

  const int nchunks = (p.inter + 127) / 128;
  const int stride = mx_row_bytes(p.inter);
  float yp[kDownCombineMaxTokens];
#pragma unroll
  for (int t = 0; t < kDownCombineMaxTokens; ++t) yp[t] = 0.f;
  for (int t = 0; t < tc; t += 2) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int tt = t + half;
      if (tt >= tc) break;
      const DcBatch& b = half ? b1 : b0;
      const int m_begin = tile_b[tt], rows = tile_r[tt];
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int u = 0; u < kDcChunks; ++u) {
        const int c = wave + 4 * u;
        if (c >= nchunks) break;
        const int kb = c * 128;
        const bool r_ok = col < rows;
        const uint8_t* row = lds + (m_begin + (r_ok ? col : 0)) * stride;
        const bool h0 = r_ok && kb + 16 * grp < p.inter, h1 = r_ok && kb + 64 + 16 * grp < p.inter;
        const u32x4_t z = u32x4_t{0u, 0u, 0u, 0u};
        const u32x4_t a0 = h0 ? *reinterpret_cast<const u32x4_t*>(row + kb + 16 * grp) : z;
        const u32x4_t a1 = h1 ? *reinterpret_cast<const u32x4_t*>(row + kb + 64 + 16 * grp) : z;
        const u32x4_t l0 = h0 ? *reinterpret_cast<const u32x4_t*>(row + p.inter + kb + 16 * grp) : z;
        const u32x4_t l1 = h1 ? *reinterpret_cast<const u32x4_t*>(row + p.inter + kb + 64 + 16 * grp) : z;
        const int sa = (r_ok && kb + 32 * grp < p.inter) ? (int)row[2 * p.inter + kb / 32 + grp] : 127;
        const i32x8_t ahi = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3], (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
        const i32x8_t alo = {(int)l0[0], (int)l0[1], (int)l0[2], (int)l0[3], (int)l1[0], (int)l1[1], (int)l1[2], (int)l1[3]};
        acc = mfma_mx(ahi, b.q[u], sa, (int)b.s[u], acc);
        acc = mfma_mx(alo, b.q[u], sa, (int)b.s[u], acc);
      }
      // refill this buffer two tiles ahead (loads past the last tile read zero)
      if (half) dc_load(b1, p, tt + 2, tc, n0, col, wave, grp, tile_e);
      else dc_load(b0, p, tt + 2, tc, n0, col, wave, grp, tile_e);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * grp + i;
        if (r < rows) {
          const int pos = m_begin + r;
          const int tok = slot_tok[pos];
          const float contrib = slot_w[pos] * acc[i];
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
  hipLaunchKernelGGL(down_combine_kernel, dim3(p.hidden / 16), dim3(256),
                     down_combine_lds_bytes(p.tokens, p.top_k, p.inter), stream, p);
  return hipGetLastError();
}

}  // namespace moe
