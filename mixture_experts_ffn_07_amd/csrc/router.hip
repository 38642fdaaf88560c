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

// (u, e) ranks above (bu, be): larger u, or equal u and lower index.
__device__ __forceinline__ bool ranks_above(float u, int e, float bu, int be) {
  return u > bu || (u == bu && e < be);
}

// One wave per token.  Lane l holds experts l, l+64, ... (at most 16 each).
// Top-k by k rounds of a wave-wide arg-max under ranks_above; round k+1
// gives the next score for the tie gap.  NaN scores rank as -inf, so the
// selection is always k distinct valid experts.
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ part, int ksplit,
                                                          const float* __restrict__ bias, int tokens,
                                                          int n_experts, int top_k, float route_scale,
                                                          int32_t* __restrict__ idx_out,
                                                          float* __restrict__ w_out, float* __restrict__ gap_out) {
  constexpr int kMaxPerLane = 16;  // n_experts <= 1024
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= tokens) return;
  float s[kMaxPerLane], u[kMaxPerLane];
  uint32_t valid = 0;
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) {
    const int e = lane + 64 * j;
    s[j] = 0.f;
    u[j] = -INFINITY;
    if (e < n_experts) {
      float l = 0.f;
      for (int zz = 0; zz < ksplit; ++zz) l += part[((size_t)zz * tokens + t) * n_experts + e];
      const float sp = fmaxf(l, 0.f) + log1pf(expf(-fabsf(l)));
      s[j] = sqrtf(sp);
      float uu = s[j] + (bias ? bias[e] : 0.f);
      u[j] = (uu != uu) ? -INFINITY : uu;
      valid |= 1u << j;
    }
  }
  float sel_s[16];
  int sel_e[16];
  float u_kth = 0.f, gap = INFINITY;
  const int rounds = top_k < n_experts ? top_k + 1 : top_k;
  for (int r = 0; r < rounds; ++r) {
    float bu = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
      if ((valid >> j) & 1u) {
        const int e = lane + 64 * j;
        if (ranks_above(u[j], e, bu, be)) {
          bu = u[j];
          be = e;
        }
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float ou = __shfl_xor(bu, off, 64);
      const int oe = __shfl_xor(be, off, 64);
      if (ranks_above(ou, oe, bu, be)) {
        bu = ou;
        be = oe;
      }
    }
    if (r == top_k) {
      gap = u_kth - bu;
      break;
    }
    // winner's unbiased score, broadcast from its owner lane
    const int jw = be >> 6;
    float mine = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) mine = (j == jw) ? s[j] : mine;
    const float sw = __shfl(mine, be & 63, 64);
    if (lane == (be & 63)) valid &= ~(1u << jw);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      if (q == r) {
        sel_s[q] = sw;
        sel_e[q] = be;
      }
    }
    u_kth = bu;
  }
  if (lane != 0) return;
  float total = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (r < top_k) total += sel_s[r];
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    if (r < top_k) {
      idx_out[(size_t)t * top_k + r] = sel_e[r];
      w_out[(size_t)t * top_k + r] = total > 0.f ? route_scale * sel_s[r] / total : route_scale / (float)top_k;
    }
  }
  if (gap_out) gap_out[t] = gap;
}

RouterPlan router_plan(int64_t tokens, int n_experts, int hidden) {
  RouterPlan p;
  p.mt = tokens >= 64 ? 4 : 1;
  const int64_t etiles = (n_experts + 63) / 64;
  const int64_t ttiles = tokens > 0 ? (tokens + 16 * p.mt - 1) / (16 * p.mt) : 1;
  const int nchunks = (hidden + 127) / 128;
  int64_t want = (512 + etiles * ttiles - 1) / (etiles * ttiles);  // aim for ~512 blocks
  if (want < 1) want = 1;
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

hipError_t launch_router_topk(const float* part, int ksplit, const float* bias, int tokens, int n_experts,
                              int top_k, float route_scale, int32_t* idx, float* w, float* gap,
                              hipStream_t stream) {
  dim3 grid((tokens + 3) / 4);
  hipLaunchKernelGGL(router_topk_kernel, grid, dim3(256), 0, stream, part, ksplit, bias, tokens, n_experts, top_k,
                     route_scale, idx, w, gap);
  return hipGetLastError();
}

}  // namespace moe
