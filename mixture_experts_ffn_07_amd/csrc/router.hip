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
#include "permute_device.h"
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
  topk_token<MPL>(part + (size_t)t * n_experts, ksplit, (int64_t)tokens * n_experts, bias, n_experts, top_k,
                  route_scale, idx_out + (size_t)t * top_k, w_out + (size_t)t * top_k,
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

RouterPlan router_plan(int64_t tokens, int n_experts, int hidden) {
  RouterPlan p;
  p.mt = tokens >= 64 ? 4 : 1;
  const int64_t etiles = (n_experts + 63) / 64;
  const int64_t ttiles = tokens > 0 ? (tokens + 16 * p.mt - 1) / (16 * p.mt) : 1;
  const int nchunks = (hidden + 127) / 128;
  int64_t want = (512 + etiles * ttiles - 1) / (etiles * ttiles);  // aim for ~512 blocks
  if (want < 1) want = 1;
  if (want > 8) want = 8;  // the top-k adds the partials; keep that short
  if (want > nchunks) want = nchunks;
  p.chunks_per_split = (int)((nchunks + want - 1) / want);
  p.ksplit = (nchunks + p.chunks_per_split - 1) / p.chunks_per_split;
  return p;
}

hipError_t launch_router_logits(const RouterPlan& plan, const uint16_t* x, const float* router_w, float* part,
                                int tokens, int n_experts, int hidden, hipStream_t stream) {
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
