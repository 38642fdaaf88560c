// Router of the MoE FFN layer: fp32 logits, sqrtsoftplus scores, top-k with
// lowest-index tie-break, renormalised weights times the route scale.
//
// Score function "sqrtsoftplus" and route_scale: checkpoint config.json on the
// "DeepSeek V4.1" atlas page (score_func, route_scale, n_activated_experts);
// routed_scaling_factor / num_experts_per_tok: DeepseekV41Config in the
// max.pipelines.architectures.deepseekV41 API reference.
//
// Logits.  l = x W_r^T with bf16 x and fp32 W_r, accumulated in fp32.  On
// gfx950 this runs on the bf16 matrix cores: each fp32 weight is split
// exactly into three bf16 terms (hi + mid + lo carry its 24 significand
// bits), every bf16 x bf16 product is exact in fp32, so three MFMAs per
// K-step give an fp32-accumulated dot product of the exact products.
#include "moe_device.h"
#include "moe_internal.h"
#include "mx_device.h"
#include "permute_device.h"
#include "norm_device.h"
#include "router_device.h"

#include <math.h>

namespace moe {

// K-chunk of 128: lane group g = lane/16 covers K offsets [32g, 32g+32) of the
// chunk; MFMA step s (0..3) takes its eight elements 8s..8s+7.  The same
// permutation of K on both operands leaves the dot product unchanged and
// gives each lane contiguous 64-byte (x) and 128-byte (W_r) loads.
template <int MT>
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ wr, float* __restrict__ part,
                                                            int tokens, int n_experts, int hidden,
                                                            int chunks_per_split) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int e = blockIdx.y * 64 + wave * 16 + col;
  const int t0 = blockIdx.x * 16 * MT;
  const int z = blockIdx.z;
  const int nchunks = (hidden + 127) / 128;
  const int c_begin = z * chunks_per_split;
  const int c_end = min(nchunks, c_begin + chunks_per_split);
  const bool e_ok = e < n_experts;
  const float* wrow = wr + (size_t)(e_ok ? e : 0) * hidden;

  f32x4_t acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (int c = c_begin; c < c_end; ++c) {
    const int k0 = c * 128 + grp * 32;
    const bool k_ok = k0 < hidden;  // hidden % 32 == 0: a lane group is all in or all out
    float wv[32];
    if (e_ok && k_ok) {
      const float4* src = reinterpret_cast<const float4*>(wrow + k0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float4 v = src[i];
        wv[4 * i + 0] = v.x;
        wv[4 * i + 1] = v.y;
        wv[4 * i + 2] = v.z;
        wv[4 * i + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) wv[i] = 0.f;
    }
    bf16x8_t bh[4], bm[4], bl[4];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint16_t h = f32_to_bf16(wv[i]);
      const float r1 = wv[i] - bf16_to_f32(h);
      const uint16_t m = f32_to_bf16(r1);
      const float r2 = r1 - bf16_to_f32(m);
      const uint16_t l = f32_to_bf16(r2);
      bh[i / 8][i % 8] = bits_to_bf16(h);
      bm[i / 8][i % 8] = bits_to_bf16(m);
      bl[i / 8][i % 8] = bits_to_bf16(l);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const int t = t0 + 16 * mt + col;
      bf16x8_t a[4];
      if (t < tokens && k_ok) {
        const bf16x8_t* src = reinterpret_cast<const bf16x8_t*>(x + (size_t)t * hidden + k0);
#pragma unroll
        for (int s = 0; s < 4; ++s) a[s] = src[s];
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s) a[s] = zero_bf16x8();
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        acc[mt] = mfma_16x16x32(a[s], bh[s], acc[mt]);
        acc[mt] = mfma_16x16x32(a[s], bm[s], acc[mt]);
        acc[mt] = mfma_16x16x32(a[s], bl[s], acc[mt]);
      }
    }
  }
  if (!e_ok) return;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = t0 + 16 * mt + 4 * grp + i;
      if (t < tokens) part[((size_t)z * tokens + t) * n_experts + e] = acc[mt][i];
    }
  }
}

// One wave per token.
template <int MPL>
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ part, int ksplit,
                                                          const float* __restrict__ bias, int tokens,
                                                          int n_experts, int top_k, float route_scale,
                                                          int32_t* __restrict__ idx_out,
                                                          float* __restrict__ w_out, float* __restrict__ gap_out) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= tokens) return;
  constexpr int G = MPL <= 4 ? 8 : MPL <= 8 ? 4 : 2;
  topk_token<MPL, false, G>(part + (size_t)t * n_experts, ksplit, (int64_t)tokens * n_experts, bias, n_experts,
                            top_k, route_scale, idx_out + (size_t)t * top_k, w_out + (size_t)t * top_k,
                            gap_out ? gap_out + t : nullptr, nullptr);
}

// Few tokens (T*k <= 1024): top-k of every token, then the permutation and
// the grouped-GEMM tile table, in one block of 1024 threads.
template <int MPL>
__global__ __launch_bounds__(1024) void route_permute_small_kernel(
    const float* __restrict__ part, int ksplit, const float* __restrict__ bias, int tokens, int n_experts, int top_k,
    float route_scale, int32_t* __restrict__ idx_out, float* __restrict__ w_out, float* __restrict__ gap_out,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slots, int32_t* __restrict__ slot_pos, int bm,
    int max_tiles, GemmTile* __restrict__ tiles, int32_t* __restrict__ tile_count) {
  extern __shared__ uint16_t cnt[];
  __shared__ int32_t idx_sh[1024];
  const int wave = threadIdx.x >> 6;
  for (int t = wave; t < tokens; t += 16)
    topk_token<MPL>(part + (size_t)t * n_experts, ksplit, (int64_t)tokens * n_experts, bias, n_experts, top_k,
                    route_scale, idx_out + (size_t)t * top_k, w_out + (size_t)t * top_k,
                    gap_out ? gap_out + t : nullptr, idx_sh + t * top_k);
  __syncthreads();
  permute_block(idx_sh, tokens * top_k, n_experts, cnt, offsets, sorted_slots, slot_pos, bm, max_tiles, tiles,
                tile_count);
}

// W_r [E][H] fp32 -> three bf16 matrices [3][E][H] with hi + mid + lo == w
// exactly (the same split as router_logits_kernel's registers).
__global__ __launch_bounds__(256) void router_split3_kernel(const float* __restrict__ wr, uint16_t* __restrict__ w3,
                                                            int64_t n) {
  for (int64_t i = blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float v = wr[i];
    const uint16_t h = f32_to_bf16(v);
    const float r1 = v - bf16_to_f32(h);
    const uint16_t m = f32_to_bf16(r1);
    const float r2 = r1 - bf16_to_f32(m);
    w3[i] = h;
    w3[n + i] = m;
    w3[2 * n + i] = f32_to_bf16(r2);
  }
}

// From this many tokens the split weights go through the dense pipelined
// GEMM with 128-token tiles (4096 tokens: logits 180 -> 81 us, the top-k over
// twelve partials 19 -> 37 us; 16384 tokens: 269 + 18 -> 140 + 23 us).
constexpr int64_t kDenseRouterMinTokens = 1024;
// From this many tokens the whole-round dense kernel, the three terms added
// in its registers: ksplit = the K ranges alone.
constexpr int64_t kDenseRouterNtTokens = 2048;

size_t router_w3_bytes(const RouterPlan& plan, int n_experts, int hidden) {
  return plan.dense_kslices > 0 ? sizeof(uint16_t) * 3 * (size_t)n_experts * hidden : 0;
}

RouterPlan router_plan(int64_t tokens, int n_experts, int hidden) {
  RouterPlan p;
  p.dense_kslices = 0;
  p.whole_round = false;
  if (tokens >= kDenseRouterNtTokens) {
    p.dense_kslices = dense_router_kslices((int)tokens, n_experts, hidden);
    p.ksplit = p.dense_kslices;
    p.whole_round = true;
    p.mt = 4;
    p.chunks_per_split = 0;
    return p;
  }
  if (tokens >= kDenseRouterMinTokens) {
    // three weight slices x K ranges: aim for ~768 blocks of 128 tokens x 256 experts
    const int64_t per_slice = (tokens + 127) / 128 * ((n_experts + 255) / 256);
    const int nch = hidden / 32;
    int64_t ks = (768 + 3 * per_slice - 1) / (3 * per_slice);
    ks = ks < 1 ? 1 : ks > 8 ? 8 : ks;
    if (ks > nch) ks = nch;
    const int per = (int)((nch + ks - 1) / ks);
    p.dense_kslices = (nch + per - 1) / per;  // every K range non-empty
    p.ksplit = 3 * p.dense_kslices;
    p.mt = 4;
    p.chunks_per_split = 0;
    return p;
  }
  // 64-token tiles from 256 tokens; below that 16-token tiles give more
  // blocks (64 tokens: 32 -> 24 us)
  p.mt = tokens >= 256 ? 4 : 1;
  const int64_t etiles = (n_experts + 63) / 64;
  const int64_t ttiles = tokens > 0 ? (tokens + 16 * p.mt - 1) / (16 * p.mt) : 1;
  const int nchunks = (hidden + 127) / 128;
  // aim for ~2048 blocks, at most 16 K ranges (the top-k adds the partials;
  // 64 tokens: 512 blocks and 8 ranges 24 + 11 us, this 19 + 13 us)
  int64_t want = (2048 + etiles * ttiles - 1) / (etiles * ttiles);
  if (want < 1) want = 1;
  if (want > 16) want = 16;
  if (want > nchunks) want = nchunks;
  p.chunks_per_split = (int)((nchunks + want - 1) / want);
  p.ksplit = (nchunks + p.chunks_per_split - 1) / p.chunks_per_split;
  return p;
}

hipError_t launch_router_logits(const RouterPlan& plan, const uint16_t* x, const float* router_w, float* part,
                                int tokens, int n_experts, int hidden, uint16_t* w3, hipStream_t stream) {
  if (plan.dense_kslices > 0) {
    const int64_t n = (int64_t)n_experts * hidden;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(router_split3_kernel, dim3((unsigned)(blocks < 2048 ? blocks : 2048)), dim3(256), 0, stream,
                       router_w, w3, n);
    GemmParams q{};
    q.M = tokens;
    q.A = x;
    q.lda = hidden;
    q.a_rows = tokens;
    q.K = hidden;
    q.bh = w3;
    q.N = n_experts;
    q.ldc = n_experts;
    q.Cf = part;
    q.k_slices = plan.dense_kslices;
    q.b_slice_stride = n;
    q.c_slice_stride = (int64_t)tokens * n_experts;
    if (plan.whole_round) return launch_dense_router(q, stream);
    return launch_dense_f32(q, 3 * plan.dense_kslices, stream);
  }
  dim3 grid((tokens + 16 * plan.mt - 1) / (16 * plan.mt), (n_experts + 63) / 64, plan.ksplit);
  if (plan.mt == 4)
    hipLaunchKernelGGL(router_logits_kernel<4>, grid, dim3(256), 0, stream, x, router_w, part, tokens, n_experts,
                       hidden, plan.chunks_per_split);
  else
    hipLaunchKernelGGL(router_logits_kernel<1>, grid, dim3(256), 0, stream, x, router_w, part, tokens, n_experts,
                       hidden, plan.chunks_per_split);
  return hipGetLastError();
}

// One wave (block) per expert.
__global__ __launch_bounds__(64) void router_gemv_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ wr, float* __restrict__ logits,
                                                          int tokens, int n_experts, int hidden,
                                                          float* __restrict__ scores,
                                                          const float* __restrict__ bias) {
  router_gemv_wave(x, wr, logits, tokens, n_experts, hidden, scores, bias, blockIdx.x);
}

hipError_t launch_router_gemv(const uint16_t* x, const float* router_w, float* logits, int tokens, int n_experts,
                              int hidden, float* scores, const float* bias, hipStream_t stream) {
  hipLaunchKernelGGL(router_gemv_kernel, dim3(n_experts), dim3(64), 0, stream, x, router_w, logits, tokens,
                     n_experts, hidden, scores, bias);
  return hipGetLastError();
}

// The router GEMV with the pre-FFN RMSNorm in front (T <= TM tokens, hidden
// <= 256 * NX).  A block of four waves serves four experts.  Its 256 threads
// first normalise the rows together (each a quarter of what one wave would
// do): x and the gain are loaded before the router rows, so the waits for
// them leave the rows' loads in flight and the normalisation runs under that
// stream; the squares are summed per wave, the four wave sums added in a
// fixed order, so every block derives the same scale and the same bits.  The
// normalised rows go to LDS, where each wave reads them for its dot product
// as router_gemv_wave does from x.  Block 0 also writes them to x_norm [T][H]
// for the launches that follow.  Barriers are bare s_barrier after an LDS
// wait: a workgroup fence would also wait for the router rows.
template <int NX, int TM>
__global__ __launch_bounds__(256) void router_norm_gemv_kernel(const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ gamma, double eps,
                                                               uint16_t* __restrict__ x_norm,
                                                               const float* __restrict__ wr, int tokens,
                                                               int n_experts, int hidden, float* __restrict__ scores,
                                                               const float* __restrict__ bias) {
  constexpr int NB = (NX + 3) / 4;  // 4-element vectors per thread in the block's share of a row
  __shared__ __attribute__((aligned(16))) uint32_t xs[TM][128 * NX];  // bf16 pairs
  __shared__ double part[TM][4];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: the row's buffer stays scalar
  const int e = blockIdx.x * 4 + wv;
  const int nv = hidden / 4;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(x, (uint32_t)tokens * hidden * 2);
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(gamma, (uint32_t)hidden * 2);
  const __amdgpu_buffer_rsrc_t rw =
      make_rsrc(wr + (size_t)(e < n_experts ? e : 0) * hidden, e < n_experts ? (uint32_t)hidden * 4 : 0u);
  uint32_t xv[TM][NB][2], gv[NB][2];
#pragma unroll
  for (int tt = 0; tt < TM; ++tt) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int v = 256 * i + tid;
      const uint32_t off = v < nv && tt < tokens ? ((uint32_t)tt * hidden + 4u * v) * 2u : kOob;
      const auto d = __builtin_amdgcn_raw_buffer_load_b64(rx, (int)off, 0, 0);
      xv[tt][i][0] = d[0];
      xv[tt][i][1] = d[1];
    }
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int v = 256 * i + tid;
    const auto d = __builtin_amdgcn_raw_buffer_load_b64(rg, (int)(v < nv ? 8u * v : kOob), 0, 0);
    gv[i][0] = d[0];
    gv[i][1] = d[1];
  }
  f32x4_t w[NX];
#pragma unroll
  for (int i = 0; i < NX; ++i) {
    const int v = 64 * i + lane;
    w[i] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)(v < nv ? 16u * v : kOob), 0, 0));
  }
  __builtin_amdgcn_sched_barrier(0);  // every load issued before the first wait
#pragma unroll
  for (int tt = 0; tt < TM; ++tt) {
    double acc = 0.0;
#pragma unroll
    for (int i = 0; i < NB; ++i) acc = add_squares4(xv[tt][i][0], xv[tt][i][1], acc);
    acc = wave_sum_f64(acc);
    if (lane == 0) part[tt][wv] = acc;
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int tt = 0; tt < TM; ++tt) {
    const double r = rms_recip(((part[tt][0] + part[tt][1]) + part[tt][2]) + part[tt][3], hidden, eps);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int v = 256 * i + tid;
      if (v < nv) {
        const uint32_t a = norm_pair(xv[tt][i][0], gv[i][0], r);
        const uint32_t b = norm_pair(xv[tt][i][1], gv[i][1], r);
        *reinterpret_cast<uint2*>(&xs[tt][2 * v]) = make_uint2(a, b);
        if (x_norm && blockIdx.x == 0 && tt < tokens)
          *reinterpret_cast<uint2*>(x_norm + (size_t)tt * hidden + 4 * v) = make_uint2(a, b);
      }
    }
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  if (e >= n_experts) return;
  float acc[TM];
#pragma unroll
  for (int tt = 0; tt < TM; ++tt) {
    acc[tt] = 0.f;
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int v = 64 * i + lane;
      if (v < nv) {  // rows of x past hidden hold nothing; their weights read zero
        const uint2 q = *reinterpret_cast<const uint2*>(&xs[tt][2 * v]);
        acc[tt] = fmaf(__uint_as_float(q.x << 16), w[i][0], acc[tt]);
        acc[tt] = fmaf(__uint_as_float(q.x & 0xffff0000u), w[i][1], acc[tt]);
        acc[tt] = fmaf(__uint_as_float(q.y << 16), w[i][2], acc[tt]);
        acc[tt] = fmaf(__uint_as_float(q.y & 0xffff0000u), w[i][3], acc[tt]);
      }
    }
  }
#pragma unroll
  for (int tt = 0; tt < TM; ++tt) {
    const float v = wave_sum_f32(acc[tt]);
    if (lane == 0 && tt < tokens) {
      const float s = sqrtsoftplus(v);
      scores[(size_t)tt * n_experts + e] = s;
      scores[(size_t)(tokens + tt) * n_experts + e] = s + (bias ? bias[e] : 0.f);
    }
  }
}

bool router_norm_gemv_supported(int tokens, int hidden) {
  return tokens >= 1 && tokens <= 2 && hidden <= 256 * 20;
}

hipError_t launch_router_norm_gemv(const uint16_t* x, const uint16_t* gamma, double eps, uint16_t* x_norm,
                                   const float* router_w, int tokens, int n_experts, int hidden, float* scores,
                                   const float* bias, hipStream_t stream) {
  if (!router_norm_gemv_supported(tokens, hidden)) return hipErrorInvalidValue;
  const bool two = tokens == 2;
  auto kern = hidden <= 256 * 8 ? (two ? router_norm_gemv_kernel<8, 2> : router_norm_gemv_kernel<8, 1>)
                                : (two ? router_norm_gemv_kernel<20, 2> : router_norm_gemv_kernel<20, 1>);
  hipLaunchKernelGGL(kern, dim3((n_experts + 3) / 4), dim3(256), 0, stream, x, gamma, eps, x_norm, router_w, tokens,
                     n_experts, hidden, scores, bias);
  return hipGetLastError();
}

hipError_t launch_route_permute_small(const float* part, int ksplit, const float* bias, int tokens, int n_experts,
                                      int top_k, float route_scale, int32_t* idx, float* w, float* gap,
                                      int32_t* offsets, int32_t* sorted_slots, int32_t* slot_pos, int bm,
                                      int max_tiles, GemmTile* tiles, int32_t* tile_count, hipStream_t stream) {
  const int nj = (n_experts + 63) / 64;
  auto kern = nj <= 2 ? route_permute_small_kernel<2>
              : nj <= 4 ? route_permute_small_kernel<4>
              : nj <= 6 ? route_permute_small_kernel<6>
              : nj <= 8 ? route_permute_small_kernel<8>
                        : route_permute_small_kernel<16>;
  hipLaunchKernelGGL(kern, dim3(1), dim3(1024), permute_block_lds_bytes(n_experts), stream, part, ksplit, bias, tokens,
                     n_experts, top_k, route_scale, idx, w, gap, offsets, sorted_slots, slot_pos, bm, max_tiles, tiles,
                     tile_count);
  return hipGetLastError();
}

hipError_t launch_router_topk(const float* part, int ksplit, const float* bias, int tokens, int n_experts,
                              int top_k, float route_scale, int32_t* idx, float* w, float* gap,
                              hipStream_t stream) {
  dim3 grid((tokens + 3) / 4);
  const int nj = (n_experts + 63) / 64;
  auto kern = nj <= 2 ? router_topk_kernel<2>
              : nj <= 4 ? router_topk_kernel<4>
              : nj <= 6 ? router_topk_kernel<6>
              : nj <= 8 ? router_topk_kernel<8>
                        : router_topk_kernel<16>;
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, part, ksplit, bias, tokens, n_experts, top_k, route_scale, idx,
                     w, gap);
  return hipGetLastError();
}

}  // namespace moe
