// Router device code shared by the router kernels and the fused few-token
// kernels: the weight-streaming logit GEMV (one wave per expert) and the
// per-token top-k (one wave per token).
//
// Score s = sqrtsoftplus(l); selection score u = s + bias (bias only
// chooses, the weights use s); the k experts of largest u, ties to the lower
// index; weights route_scale * s / sum of the selected s (checkpoint
// config.json on the "DeepSeek V4.1" atlas page: score_func, route_scale).
#pragma once

#include <math.h>

#include "moe_device.h"

namespace moe {

// sqrtsoftplus(l) = sqrt(log(1 + e^l)), written as sqrt(max(l, 0) + log1p(e^-|l|)).
__device__ __forceinline__ float sqrtsoftplus(float l) { return sqrtf(fmaxf(l, 0.f) + log1pf(expf(-fabsf(l)))); }

// (u, e) ranks above (bu, be): larger u, or equal u and lower index.
__device__ __forceinline__ bool ranks_above(float u, int e, float bu, int be) {
  return u > bu || (u == bu && e < be);
}

// The selection of topk_token, from each lane's scores: u (selection) and s
// (weights) of experts lane, lane + 64, ... (valid bits mark the ones that
// exist).  Each lane sorts its slots once by (u desc, index asc) with an
// odd-even transposition network (taken and unused slots rank last); a round
// then takes the wave's best list head (max score, then lowest index among
// the lanes holding it, with DPP reductions) and only the owner lane advances
// its list.  Lane r < k ends with selection r (expert my_e, score my_s);
// every lane gets gap = u(k) - u(k+1) (+inf when k == n_experts, or when
// want_gap is false and the extra round is skipped).
template <int kMaxPerLane>
__device__ __forceinline__ void topk_select(const float (&u)[kMaxPerLane], const float (&s)[kMaxPerLane],
                                            uint32_t valid, int n_experts, int top_k, int& my_e_out,
                                            float& my_s_out, float& gap_out, bool want_gap = true) {
  const int lane = threadIdx.x & 63;
  float su[kMaxPerLane], ss[kMaxPerLane];
  int se[kMaxPerLane];
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) {
    const bool v = (valid >> j) & 1u;
    su[j] = v ? u[j] : -INFINITY;
    se[j] = v ? lane + 64 * j : 0x7fffffff;
    ss[j] = s[j];
  }
#pragma unroll
  for (int pass = 0; pass < kMaxPerLane; ++pass) {
#pragma unroll
    for (int i = pass & 1; i + 1 < kMaxPerLane; i += 2) {
      const bool sw = (su[i + 1] > su[i]) | ((su[i + 1] == su[i]) & (se[i + 1] < se[i]));
      const float tu = su[i], ts = ss[i];
      const int te = se[i];
      su[i] = sw ? su[i + 1] : su[i];
      se[i] = sw ? se[i + 1] : se[i];
      ss[i] = sw ? ss[i + 1] : ss[i];
      su[i + 1] = sw ? tu : su[i + 1];
      se[i + 1] = sw ? te : se[i + 1];
      ss[i + 1] = sw ? ts : ss[i + 1];
    }
  }
  float hu = su[0], hs = ss[0];
  int he = se[0], ptr = 0;
  float my_s = 0.f;
  int my_e = 0;
  float u_kth = 0.f, gap = INFINITY;
  const int rounds = want_gap && top_k < n_experts ? top_k + 1 : top_k;
  for (int r = 0; r < rounds; ++r) {
    const float M = wave_max_f32(hu);
    const int ew = wave_min_i32(hu == M ? he : 0x7fffffff);
    if (r == top_k) {
      gap = u_kth - M;
      break;
    }
    const int owner = ew & 63;  // expert e lives in lane e % 64
    const float sw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hs), owner));
    if (lane == owner) {
      ++ptr;
      float nu = -INFINITY, ns = 0.f;
      int ne = 0x7fffffff;
#pragma unroll
      for (int j = 1; j < kMaxPerLane; ++j) {
        nu = (j == ptr) ? su[j] : nu;
        ne = (j == ptr) ? se[j] : ne;
        ns = (j == ptr) ? ss[j] : ns;
      }
      hu = nu;
      he = ne;
      hs = ns;
    }
    if (lane == r) {
      my_s = sw;
      my_e = ew;
    }
    u_kth = M;
  }
  my_e_out = my_e;
  my_s_out = my_s;
  gap_out = gap;
}

// Top-k of one token by one wave.  Lane l holds experts l, l+64, ... (at
// most 16 each); logit e is the sum of `ksplit` partials at
// part[z * part_stride + e], added in z order.  Top-k is k rounds of a
// wave-wide arg-max under ranks_above; round k+1 gives the next score for
// the tie gap.  NaN scores rank as -inf, so the selection is always k
// distinct valid experts.  Lane r < k writes selection r to idx_row/w_row
// (and idx_lds when non-null); lane 0 writes *gap_out when non-null.
// With FROM_SCORES, `part` holds the scores s and `sel` the selection scores
// u of this token (computed by the router kernel) and ksplit/bias are unused.
// G: partials whose loads issue together (1 where registers are short).
template <int kMaxPerLane, bool FROM_SCORES = false, int G = 1>  // ceil(n_experts / 64) rounded up; at most 16
__device__ __forceinline__ void topk_token(const float* __restrict__ part, int ksplit, int64_t part_stride,
                                           const float* __restrict__ bias, int n_experts, int top_k,
                                           float route_scale, int32_t* __restrict__ idx_row,
                                           float* __restrict__ w_row, float* __restrict__ gap_out,
                                           int32_t* idx_lds, const float* __restrict__ sel = nullptr) {
  const int lane = threadIdx.x & 63;
  float s[kMaxPerLane], u[kMaxPerLane];
  uint32_t valid = 0;
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) {
    s[j] = 0.f;
    if (lane + 64 * j < n_experts) valid |= 1u << j;
  }
  if constexpr (FROM_SCORES) {
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
      const int e = min(lane + 64 * j, n_experts - 1);
      s[j] = part[e];
      const float uu = sel[e];
      u[j] = ((valid >> j) & 1u) && uu == uu ? uu : -INFINITY;
    }
  } else {
  // Partial sums, z in order.  The loads of G partials at a time (expert
  // index clamped into range; unused slots are dropped below) all issue
  // before the first wait: the partials were just written, often through
  // another XCD's L2, and one round trip per partial would dominate.
  const int nj = (n_experts + 63) / 64;
  for (int z0 = 0; z0 < ksplit; z0 += G) {
    float v[G][kMaxPerLane];
#pragma unroll
    for (int dz = 0; dz < G; ++dz)
#pragma unroll
      for (int j = 0; j < kMaxPerLane; ++j)
        v[dz][j] = (z0 + dz < ksplit && j < nj) ? part[(z0 + dz) * part_stride + min(lane + 64 * j, n_experts - 1)]
                                                : 0.f;
#pragma unroll
    for (int dz = 0; dz < G; ++dz)
#pragma unroll
      for (int j = 0; j < kMaxPerLane; ++j)
        if (z0 + dz < ksplit) s[j] += v[dz][j];
  }
  // u holds the bias until the scores are known
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) u[j] = (bias && j < nj) ? bias[min(lane + 64 * j, n_experts - 1)] : 0.f;
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) {
    if ((valid >> j) & 1u) {
      s[j] = sqrtsoftplus(s[j]);
      const float uu = s[j] + u[j];
      u[j] = (uu != uu) ? -INFINITY : uu;
    } else {
      u[j] = -INFINITY;
    }
  }
  }
  int my_e;
  float my_s, gap;
  topk_select<kMaxPerLane>(u, s, valid, n_experts, top_k, my_e, my_s, gap);
  // sum of the selected scores in selection order, then each lane r < k writes selection r
  float total = 0.f;
  for (int r = 0; r < top_k; ++r) total += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), r));
  if (lane < top_k) {
    idx_row[lane] = my_e;
    if (idx_lds) idx_lds[lane] = my_e;
    w_row[lane] = total > 0.f ? route_scale * my_s / total : route_scale / (float)top_k;
  }
  if (gap_out && lane == 0) *gap_out = gap;
}

// topk_token<MPL, true> for two tokens at once (scores s at s_row[i], selection
// scores u at u_row[i], i = 0, 1): the same per-token selection, with the two
// tokens' loads issued together and their reduction chains interleaved, so
// the pair takes about the latency of one.  Outputs as topk_token (no tie
// gap); the second token is skipped when `two` is false (wave-uniform).
template <int kMaxPerLane>
__device__ __forceinline__ void topk_token_pair(const float* const (&s_row)[2], const float* const (&u_row)[2],
                                                bool two, int n_experts, int top_k, float route_scale,
                                                int32_t* const (&idx_row)[2], float* const (&w_row)[2],
                                                int32_t* const (&idx_lds)[2]) {
  const int lane = threadIdx.x & 63;
  const int nt = two ? 2 : 1;
  uint32_t valid = 0;
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j)
    if (lane + 64 * j < n_experts) valid |= 1u << j;
  float su[2][kMaxPerLane], ss[2][kMaxPerLane];
  int se[2][kMaxPerLane];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int t = tt < nt ? tt : 0;  // a missing second token repeats the first (results dropped)
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
      const int e = min(lane + 64 * j, n_experts - 1);
      const bool v = (valid >> j) & 1u;
      const float uu = u_row[t][e];
      ss[tt][j] = s_row[t][e];
      su[tt][j] = v && uu == uu ? uu : -INFINITY;
      se[tt][j] = v ? lane + 64 * j : 0x7fffffff;
    }
  }
  // each lane's list sorted by (u desc, index asc): odd-even transposition
#pragma unroll
  for (int pass = 0; pass < kMaxPerLane; ++pass) {
#pragma unroll
    for (int i = pass & 1; i + 1 < kMaxPerLane; i += 2) {
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        const bool sw = (su[tt][i + 1] > su[tt][i]) | ((su[tt][i + 1] == su[tt][i]) & (se[tt][i + 1] < se[tt][i]));
        const float tu = su[tt][i], ts = ss[tt][i];
        const int te = se[tt][i];
        su[tt][i] = sw ? su[tt][i + 1] : su[tt][i];
        se[tt][i] = sw ? se[tt][i + 1] : se[tt][i];
        ss[tt][i] = sw ? ss[tt][i + 1] : ss[tt][i];
        su[tt][i + 1] = sw ? tu : su[tt][i + 1];
        se[tt][i + 1] = sw ? te : se[tt][i + 1];
        ss[tt][i + 1] = sw ? ts : ss[tt][i + 1];
      }
    }
  }
  float hu[2], hs[2], my_s[2];
  int he[2], ptr[2], my_e[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    hu[tt] = su[tt][0];
    hs[tt] = ss[tt][0];
    he[tt] = se[tt][0];
    ptr[tt] = 0;
    my_s[tt] = 0.f;
    my_e[tt] = 0;
  }
  for (int r = 0; r < top_k; ++r) {
    float M[2];
    int ew[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) M[tt] = wave_max_f32(hu[tt]);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) ew[tt] = wave_min_i32(hu[tt] == M[tt] ? he[tt] : 0x7fffffff);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int owner = ew[tt] & 63;  // expert e lives in lane e % 64
      const float sw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(hs[tt]), owner));
      if (lane == owner) {
        ++ptr[tt];
        float nu = -INFINITY, ns = 0.f;
        int ne = 0x7fffffff;
#pragma unroll
        for (int j = 1; j < kMaxPerLane; ++j) {
          nu = (j == ptr[tt]) ? su[tt][j] : nu;
          ne = (j == ptr[tt]) ? se[tt][j] : ne;
          ns = (j == ptr[tt]) ? ss[tt][j] : ns;
        }
        hu[tt] = nu;
        he[tt] = ne;
        hs[tt] = ns;
      }
      if (lane == r) {
        my_s[tt] = sw;
        my_e[tt] = ew[tt];
      }
    }
  }
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    if (tt >= nt) break;  // wave-uniform
    float total = 0.f;
    for (int r = 0; r < top_k; ++r) total += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s[tt]), r));
    if (lane < top_k) {
      idx_row[tt][lane] = my_e[tt];
      idx_lds[tt][lane] = my_e[tt];
      w_row[tt][lane] = total > 0.f ? route_scale * my_s[tt] / total : route_scale / (float)top_k;
    }
  }
}

// Routing of T <= 2 tokens (T * k <= 64) by the calling wave from the
// router's scores (s at scores[t][e], selection scores u at scores[T + t][e]),
// kept in registers.  Every wave that calls it gets the same values: the
// same selection as topk_token, weights rho * s / sum s (rho / k for a zero
// sum), and the stable permutation of the flat slots f = t * k + j by
// expert.  Lane f < T * k holds slot f (expert e, weight w, position pos);
// lane d < n_tiles holds the d-th distinct expert in ascending order (tile):
// its expert, first position, rows, and the tokens of its rows (first |
// second << 16; an expert has at most one row per token).
struct WaveRoute {
  int e, pos;
  float w;
  int t_e, t_m, t_r, t_src;
  int n_tiles;
};

template <int kMaxPerLane>
__device__ __forceinline__ WaveRoute route_wave_small(const float* __restrict__ scores, int tokens, int n_experts,
                                                      int top_k, float route_scale) {
  const int lane = threadIdx.x & 63;
  const int n = tokens * top_k;
  uint32_t valid = 0;
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j)
    if (lane + 64 * j < n_experts) valid |= 1u << j;
  int sel_e[2] = {0, 0};
  float sel_w[2] = {0.f, 0.f};
  // both tokens' score loads issue before the first selection
  float s[2][kMaxPerLane], u[2][kMaxPerLane];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int tt = t < tokens ? t : 0;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
      const int e = min(lane + 64 * j, n_experts - 1);
      s[t][j] = scores[(size_t)tt * n_experts + e];
      const float uu = scores[(size_t)(tokens + tt) * n_experts + e];
      u[t][j] = ((valid >> j) & 1u) && uu == uu ? uu : -INFINITY;
    }
  }
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (t >= tokens) break;  // wave-uniform
    float my_s, gap;
    topk_select<kMaxPerLane>(u[t], s[t], valid, n_experts, top_k, sel_e[t], my_s, gap, false);
    float total = 0.f;
    for (int r = 0; r < top_k; ++r) total += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_s), r));
    sel_w[t] = total > 0.f ? route_scale * my_s / total : route_scale / (float)top_k;
  }
  WaveRoute out;
  // slot f = lane: token 0's selections are in lanes 0..k-1 already, token 1's move up by k
  const int src = max(lane - top_k, 0);
  const int e1 = __shfl(sel_e[1], src);
  const float w1 = __shfl(sel_w[1], src);
  const int e = lane < top_k ? sel_e[0] : e1;
  out.w = lane < top_k ? sel_w[0] : w1;
  const int ee = lane < n ? e : 0x7fffffff;
  out.e = ee;
  // position = slots with a smaller expert, plus earlier slots of the same one
  int pos = 0, dup_before = 0, count = 0;
  for (int j = 0; j < n; ++j) {
    const int ej = __builtin_amdgcn_readlane(ee, j);
    pos += (ej < ee) || (ej == ee && j < lane);
    dup_before += (ej == ee && j < lane);
    count += (ej == ee);
  }
  out.pos = pos;
  const bool first = lane < n && dup_before == 0;
  const uint64_t firsts = __ballot(first);
  int distinct_smaller = 0;
  for (int j = 0; j < n; ++j) {
    const int ej = __builtin_amdgcn_readlane(ee, j);
    distinct_smaller += (((firsts >> j) & 1ull) && ej < ee);
  }
  out.n_tiles = __popcll(firsts);
  // tile records to lane distinct_smaller (the other lanes fill the rest, a bijection)
  const int rank_other = lane - __popcll(firsts & ((1ull << lane) - 1ull));
  const int dst = 4 * (first ? distinct_smaller : out.n_tiles + rank_other);
  const int r0 = lane < n ? lane / top_k : 0, r1 = count > 1 ? 1 : r0;
  out.t_e = __builtin_amdgcn_ds_permute(dst, first ? ee : 0);
  out.t_m = __builtin_amdgcn_ds_permute(dst, pos);
  out.t_r = __builtin_amdgcn_ds_permute(dst, first ? count : 0);
  out.t_src = __builtin_amdgcn_ds_permute(dst, r0 | (r1 << 16));
  return out;
}

// Few tokens: logits as a weight-streaming GEMV on the vector ALUs.  One
// wave per expert reads its fp32 router row once (1 KB per load
// instruction across the wave, all loads of a 5120-wide row in flight) and
// accumulates x . w for every token in fp32, lane partials added by a fixed
// butterfly.  Equal router rows give bit-equal logits.
// With `scores` non-null it also writes s = sqrtsoftplus(l) to scores[t][e]
// and the selection score s + bias[e] to scores[T + t][e] (bias optional),
// so that the top-k that follows only compares.
// The calling wave computes expert e (wave-uniform; nothing for e >= n_experts).
template <int KV = 20>  // 4-float loads per lane held in registers per pass
__device__ __forceinline__ void router_gemv_wave(const uint16_t* __restrict__ x, const float* __restrict__ wr,
                                                 float* __restrict__ logits, int tokens, int n_experts, int hidden,
                                                 float* __restrict__ scores, const float* __restrict__ bias, int e) {
  const int lane = threadIdx.x & 63;
  if (e >= n_experts) return;
  // raw buffer loads: a vector past the end of the row reads zero, so every
  // load issues unconditionally
  const uint32_t row_bytes = (uint32_t)hidden * 4;
  const __amdgpu_buffer_rsrc_t rw =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(wr + (size_t)e * hidden), (short)0, (int)row_bytes,
                                        0x00020000);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x), (short)0, (int)((uint32_t)tokens * hidden * 2), 0x00020000);
  const int nv = hidden / 4;  // 4-float vectors per row
  for (int t = 0; t < tokens; t += 4) {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    for (int v0 = 0; v0 < nv; v0 += 64 * KV) {
      f32x4_t w[KV];
#pragma unroll
      for (int i = 0; i < KV; ++i) {
        const int v = v0 + 64 * i + lane;
        const uint32_t off = v < nv ? (uint32_t)v * 16u : 0x7ffffff0u;
        w[i] = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rw, (int)off, 0, 0));
      }
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        if (t + tt >= tokens) break;  // wave-uniform
        uint32_t xv[KV][2];
#pragma unroll
        for (int i = 0; i < KV; ++i) {
          const int v = v0 + 64 * i + lane;
          const uint32_t off = v < nv ? ((uint32_t)(t + tt) * hidden + 4u * v) * 2u : 0x7ffffff0u;
          const auto d = __builtin_amdgcn_raw_buffer_load_b64(rx, (int)off, 0, 0);
          xv[i][0] = d[0];
          xv[i][1] = d[1];
        }
#pragma unroll
        for (int i = 0; i < KV; ++i) {
          acc[tt] = fmaf(bf16_to_f32((uint16_t)(xv[i][0] & 0xffffu)), w[i][0], acc[tt]);
          acc[tt] = fmaf(bf16_to_f32((uint16_t)(xv[i][0] >> 16)), w[i][1], acc[tt]);
          acc[tt] = fmaf(bf16_to_f32((uint16_t)(xv[i][1] & 0xffffu)), w[i][2], acc[tt]);
          acc[tt] = fmaf(bf16_to_f32((uint16_t)(xv[i][1] >> 16)), w[i][3], acc[tt]);
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const float v = wave_sum_f32(acc[tt]);
      if (lane == 0 && t + tt < tokens) {
        if (logits) logits[(size_t)(t + tt) * n_experts + e] = v;
        if (scores) {
          const float s = sqrtsoftplus(v);
          scores[(size_t)(t + tt) * n_experts + e] = s;
          scores[(size_t)(tokens + t + tt) * n_experts + e] = s + (bias ? bias[e] : 0.f);
        }
      }
    }
  }
}

}  // namespace moe
