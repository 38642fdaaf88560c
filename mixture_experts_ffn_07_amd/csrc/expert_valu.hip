// Routed expert projections for one or two tokens on the vector ALUs.
//
// At T <= 2 the routed experts are pure MXFP4 weight streaming (the layer's
// cost is the weight bytes: Strata DEEPSEEK41 notes, opening paragraph and
// the "Where it goes" table).  Here each wave owns CPW output columns and
// issues every weight load of them at once: a 16-byte vector of E2M1 codes
// is exactly one 32-element E8M0 block, so lane l takes vectors l, l + 64,
// ... of the column's rows laid end to end, with one scale byte each.  Many
// light waves keep more requests in flight than a few long streams (a 75 MB
// streaming read: ~20 us from 864 long waves, ~14 us from a few thousand
// light ones).  Each vector is dequantised to bf16 pairs and multiplied with
// the activations staged in LDS by v_dot2 (mx4_dot32); lanes' partial sums
// are added in a fixed order.
//
//   gate/up: work = (selected expert, column j): rows j (gate) and I + j (up)
//            of W_gu[e] against the expert's token rows of x; writes
//            h[pos] = SwiGLU_clamped(gate, up) in bf16.
//   down:    work = output column n: row n of W_dn[e_s] for every slot s
//            (token t, choice j) against h of that slot; the weighted sum
//            over the slots plus the shared expert's output is y[t][n]
//            (the combine folded in: DeepSeek-V4 report, MoE section, the
//            gate-weighted sum of the routed outputs plus the shared one).
#include "gemv_valu_device.h"
#include "moe_device.h"
#include "moe_internal.h"
#include "mx_device.h"

namespace moe {

namespace {

constexpr int kValuBlock = 256;  // threads per block (4 waves)

// 16-byte h pieces each thread of the down kernel stages (n * I / 8 in all)
constexpr int down_staging_pieces(int jm) { return jm >= 14 ? 16 : 8; }

// gate/up: grid (ceil(I / (4 * CPW)), max_tiles).  JM >= ceil(2 * (H/32) / 64).
template <int JM, int CPW>
__global__ __launch_bounds__(kValuBlock) void gate_up_valu_kernel(GateUpValuParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // x rows of the tile [rows][H] bf16
  uint16_t* x_lds = reinterpret_cast<uint16_t*>(lds);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tile = blockIdx.y;
  const GemmTile tl = p.tiles[tile];
  int src[kValuMaxTokens];
#pragma unroll
  for (int r = 0; r < kValuMaxTokens; ++r) src[r] = p.tile_rows[tile * kTileRows + r];
  const int rows = min(tl.m_end - tl.m_begin, p.tokens);
  if (rows <= 0) return;  // unused tile record
  const int H = p.hidden, I = p.inter, VR = H / 32;

  // activation staging loads first: they return before the weights
  constexpr int kXs = 8;  // 16-byte pieces per thread: T <= 2, H <= 8192
  const int per_row = H / 8, pieces = rows * per_row;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x, (uint32_t)(p.tokens * H * 2));
  u32x4_t xs[kXs];
#pragma unroll
  for (int i = 0; i < kXs; ++i) {
    const int q = (int)threadIdx.x + kValuBlock * i;
    const int r = q >= per_row ? 1 : 0, c = q - r * per_row;
    const int sr = min(max(r ? src[1] : src[0], 0), p.tokens - 1);
    const uint32_t off = q < pieces ? (uint32_t)((sr * H + 8 * c) * 2) : kOob;
    xs[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rx, (int)off, 0, 0));
  }

  // weight loads: column j's gate row then up row, 2 * VR vectors
  const int e = tl.e;
  const uint32_t qbytes = (uint32_t)(2 * I * (H / 2)), sbytes = (uint32_t)(2 * I * VR);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.gu_q + (int64_t)e * qbytes, qbytes);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(p.gu_s + (int64_t)e * sbytes, sbytes);
  const int j0 = ((int)blockIdx.x * (kValuBlock / 64) + wave) * CPW;
  u32x4_t q[CPW][JM];
  uint32_t sc[CPW][JM];
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    const int j = j0 + c;
#pragma unroll
    for (int jj = 0; jj < JM; ++jj) {
      const int v = lane + 64 * jj;
      const bool up = v >= VR;
      const int b = v - (up ? VR : 0);
      const bool ok = j < I && v < 2 * VR;
      const uint32_t row = (uint32_t)(j + (up ? I : 0));
      q[c][jj] = __builtin_bit_cast(
          u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)(ok ? row * (uint32_t)(H / 2) + 16u * b : kOob), 0, 0));
      sc[c][jj] = __builtin_amdgcn_raw_buffer_load_b8(rs, (int)(ok ? row * (uint32_t)VR + b : kOob), 0, 0);
    }
  }
#pragma unroll
  for (int i = 0; i < kXs; ++i) {
    const int qq = (int)threadIdx.x + kValuBlock * i;
    if (qq < pieces) *reinterpret_cast<u32x4_t*>(x_lds + 8 * qq) = xs[i];
  }
  __syncthreads();

#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    float g[kValuMaxTokens], u[kValuMaxTokens];
#pragma unroll
    for (int r = 0; r < kValuMaxTokens; ++r) g[r] = u[r] = 0.f;
#pragma unroll
    for (int jj = 0; jj < JM; ++jj) {
      const int v = lane + 64 * jj;
      const bool up = v >= VR;
      const int b = min(v - (up ? VR : 0), VR - 1);  // past the pair the codes are zero
      const float scale = e8m0_scale_operand(sc[c][jj]);
#pragma unroll
      for (int r = 0; r < kValuMaxTokens; ++r) {
        if (r >= rows) break;  // block-uniform
        const float d = mx4_dot32(q[c][jj], scale, x_lds + r * H + 32 * b, 0.f);
        g[r] += up ? 0.f : d;
        u[r] += up ? d : 0.f;
      }
    }
    const int j = j0 + c;
#pragma unroll
    for (int r = 0; r < kValuMaxTokens; ++r) {
      if (r >= rows) break;
      const float gs = wave_sum_f32(g[r]), us = wave_sum_f32(u[r]);
      if (lane == 0 && j < I) p.h[(int64_t)(tl.m_begin + r) * I + j] = f32_to_bf16(clamped_swiglu(gs, us, p.limit));
    }
  }
}

// down + combine: grid ceil(H / (4 * CPW)).  JM >= ceil(n * (I/32) / 64).
template <int JM, int CPW>
__global__ __launch_bounds__(kValuBlock) void down_combine_valu_kernel(DownValuParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // h of every slot [n][I] bf16
  uint16_t* h_lds = reinterpret_cast<uint16_t*>(lds);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int T = p.tokens, k = p.top_k, n = T * k;
  const int H = p.hidden, I = p.inter, VR = I / 32;
  // lane s < n holds slot s: expert, position of its h row, weight
  const int ls = min(lane, n - 1);
  const int my_e = p.idx[ls];
  const int my_p = p.slot_pos[ls];
  const float my_w = p.topk_w[ls];
  const int n0 = ((int)blockIdx.x * (kValuBlock / 64) + wave) * CPW;

  // the shared expert's outputs of this wave's columns: lane t < T, column c
  float ysh[CPW];
#pragma unroll
  for (int c = 0; c < CPW; ++c)
    ysh[c] = (p.y_shared && lane < T && n0 + c < H) ? bf16_to_f32(p.y_shared[(int64_t)lane * H + n0 + c]) : 0.f;

  // h staging loads (slot order), before the weights
  constexpr int kHs = down_staging_pieces(JM);
  const int per_row = I / 8, pieces = n * per_row;
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(p.h, (uint32_t)(n * I * 2));
  u32x4_t hs[kHs];
#pragma unroll
  for (int i = 0; i < kHs; ++i) {
    const int qq = (int)threadIdx.x + kValuBlock * i;
    const int s = min(qq / per_row, n - 1), c = qq - s * per_row;
    const int pos = __shfl(my_p, s);
    const uint32_t off = qq < pieces ? (uint32_t)((pos * I + 8 * c) * 2) : kOob;
    hs[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rh, (int)off, 0, 0));
  }

  // weights: vector v = lane + 64 jj is block b of slot s's row n
  int vs[JM], vb[JM];
  const uint8_t* qrow[JM];
  const uint8_t* srow[JM];
#pragma unroll
  for (int jj = 0; jj < JM; ++jj) {
    const int v = lane + 64 * jj;
    const int s = min(v / VR, n - 1);
    vs[jj] = v < n * VR ? s : -1;  // -1: past the last slot (its load repeats a valid address)
    vb[jj] = v - s * VR < VR ? v - s * VR : VR - 1;
    const int64_t er = (int64_t)__shfl(my_e, s) * H;
    qrow[jj] = p.dn_q + er * (I / 2) + 16 * vb[jj];
    srow[jj] = p.dn_s + er * VR + vb[jj];
  }
  u32x4_t q[CPW][JM];
  uint32_t sc[CPW][JM];
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    const int64_t nc = min(n0 + c, H - 1);
#pragma unroll
    for (int jj = 0; jj < JM; ++jj) {
      q[c][jj] = *reinterpret_cast<const u32x4_t*>(qrow[jj] + nc * (I / 2));
      sc[c][jj] = srow[jj][nc * VR];
    }
  }
#pragma unroll
  for (int i = 0; i < kHs; ++i) {
    const int qq = (int)threadIdx.x + kValuBlock * i;
    if (qq < pieces) *reinterpret_cast<u32x4_t*>(h_lds + 8 * qq) = hs[i];
  }
  __syncthreads();

  float wsl[JM];
#pragma unroll
  for (int jj = 0; jj < JM; ++jj) wsl[jj] = __shfl(my_w, max(vs[jj], 0));
#pragma unroll
  for (int c = 0; c < CPW; ++c) {
    float acc[kValuMaxTokens];
#pragma unroll
    for (int t = 0; t < kValuMaxTokens; ++t) acc[t] = 0.f;
#pragma unroll
    for (int jj = 0; jj < JM; ++jj) {
      const int s = max(vs[jj], 0);
      const float d = mx4_dot32(q[c][jj], e8m0_scale_operand(sc[c][jj]), h_lds + s * I + 32 * vb[jj], 0.f);
      const float wd = vs[jj] >= 0 ? wsl[jj] * d : 0.f;
      const int t = s / k;
#pragma unroll
      for (int tt = 0; tt < kValuMaxTokens; ++tt) acc[tt] += t == tt ? wd : 0.f;
    }
    float r = 0.f;
#pragma unroll
    for (int t = 0; t < kValuMaxTokens; ++t) {
      const float st = wave_sum_f32(acc[t]);
      r = lane == t ? st : r;
    }
    if (lane < T && n0 + c < H) p.y[(int64_t)lane * H + n0 + c] = f32_to_bf16(r + ysh[c]);
  }
}

// instantiated vector counts per lane; the smallest >= the need is used
constexpr int kGateUpJm[] = {2, 4, 5, 7, 8};
constexpr int kDownJm[] = {2, 4, 7, 9, 14};
constexpr int kGateUpCpw = 2;
constexpr int kDownCpw = 1;

int gate_up_jm(int hidden) {
  const int need = (2 * (hidden / 32) + 63) / 64;
  for (int j : kGateUpJm)
    if (j >= need) return j;
  return 0;
}

int down_jm(int slots, int inter) {
  const int need = (slots * (inter / 32) + 63) / 64;
  for (int j : kDownJm)
    if (j >= need) return j;
  return 0;
}

}  // namespace

bool gate_up_valu_supported(int tokens, int hidden) {
  return tokens >= 1 && tokens <= kValuMaxTokens && hidden % 32 == 0 && hidden <= 8192 && gate_up_jm(hidden) > 0;
}

bool down_valu_supported(int tokens, int top_k, int inter) {
  const int n = tokens * top_k;
  if (tokens < 1 || tokens > kValuMaxTokens || inter % 32 != 0 || (int64_t)n * inter * 2 > 64 * 1024) return false;
  const int jm = down_jm(n, inter);
  return jm > 0 && (int64_t)n * (inter / 8) <= (int64_t)down_staging_pieces(jm) * kValuBlock;
}

hipError_t launch_gate_up_valu(const GateUpValuParams& p, int max_tiles, hipStream_t stream) {
  constexpr int cols = (kValuBlock / 64) * kGateUpCpw;
  const dim3 grid((p.inter + cols - 1) / cols, max_tiles);
  const size_t lds = (size_t)p.tokens * p.hidden * 2;
  switch (gate_up_jm(p.hidden)) {
    case 2: hipLaunchKernelGGL((gate_up_valu_kernel<2, kGateUpCpw>), grid, dim3(kValuBlock), lds, stream, p); break;
    case 4: hipLaunchKernelGGL((gate_up_valu_kernel<4, kGateUpCpw>), grid, dim3(kValuBlock), lds, stream, p); break;
    case 5: hipLaunchKernelGGL((gate_up_valu_kernel<5, kGateUpCpw>), grid, dim3(kValuBlock), lds, stream, p); break;
    case 7: hipLaunchKernelGGL((gate_up_valu_kernel<7, kGateUpCpw>), grid, dim3(kValuBlock), lds, stream, p); break;
    case 8: hipLaunchKernelGGL((gate_up_valu_kernel<8, kGateUpCpw>), grid, dim3(kValuBlock), lds, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_down_combine_valu(const DownValuParams& p, hipStream_t stream) {
  constexpr int cols = (kValuBlock / 64) * kDownCpw;
  const dim3 grid((p.hidden + cols - 1) / cols);
  const int n = p.tokens * p.top_k;
  const size_t lds = (size_t)n * p.inter * 2;
  switch (down_jm(n, p.inter)) {
    case 2: hipLaunchKernelGGL((down_combine_valu_kernel<2, kDownCpw>), grid, dim3(kValuBlock), lds, stream, p); break;
    case 4: hipLaunchKernelGGL((down_combine_valu_kernel<4, kDownCpw>), grid, dim3(kValuBlock), lds, stream, p); break;
    case 7: hipLaunchKernelGGL((down_combine_valu_kernel<7, kDownCpw>), grid, dim3(kValuBlock), lds, stream, p); break;
    case 9: hipLaunchKernelGGL((down_combine_valu_kernel<9, kDownCpw>), grid, dim3(kValuBlock), lds, stream, p); break;
    case 14: hipLaunchKernelGGL((down_combine_valu_kernel<14, kDownCpw>), grid, dim3(kValuBlock), lds, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace moe
