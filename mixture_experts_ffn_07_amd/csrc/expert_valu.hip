// Routed expert projections for one or two tokens on the vector ALUs.
//
// At T <= 2 the routed experts are pure MXFP4 weight streaming (the layer's
// cost is the weight bytes: Strata DEEPSEEK41 notes, opening paragraph and
// the "Where it goes" table).  A 16-byte vector of E2M1 codes is exactly one
// 32-element E8M0 block (of E4M3 codes, with MXFP8 weights, half a block), so
// a wave reads one output column's weight rows laid end to end: lane l takes
// vectors l, l + 64, ... with the scale byte of each, all issued at once.  Each vector is dequantised to bf16 pairs and
// multiplied with the activations staged in LDS by v_dot2 (mx4_dot32); the
// lanes' partial sums are added in a fixed order.
//
// Grid-stride loop: a block stages the activations once, then each wave
// walks columns wave_id, wave_id + W, ... (W = waves in the grid) with two
// register buffers: the next column's loads are in flight while the current
// one is multiplied, so the memory pipe does not idle behind the arithmetic
// and the last columns do not wait for a second round of waves.  Loads for a
// column past the end use out-of-range offsets or repeat a valid address,
// so the loop body has no branches around loads and its waits stay exact.
//
//   gate/up: column (tile, j): rows j (gate) and I + j (up) of W_gu[e]
//            against the tile's token rows of x; h[pos] = SwiGLU_clamped.
//   down:    column n: row n of W_dn[e_s] for every slot s (token t, choice
//            j) against h of that slot; the weighted sum over the slots plus
//            the shared expert's output is y[t][n] (the combine folded in:
//            DeepSeek-V4 report, MoE section, the gate-weighted sum of the
//            routed outputs plus the shared one).
#include "gemv_valu_device.h"
#include "moe_device.h"
#include "moe_internal.h"
#include "mx_device.h"
#include "router_device.h"

namespace moe {

namespace {

constexpr int kValuBlock = 256;  // threads per block (4 waves)
constexpr int kValuWaves = kValuBlock / 64;
constexpr int kMaxLiveTiles = 64;  // tile records of the one-block routing (T * k <= 64), one per lane

template <int JM>
struct ColBuf {
  u32x4_t q[JM];
  uint32_t s[JM];
  uint32_t ysh;  // down: lane t < T holds the shared expert's y[t][col] (bf16 bits)
};

// ---------------------------------------------------------------- gate/up
// A column: live tile `tile` (-1 past the end), its record and column j.
struct GuItem {
  int4 rec;  // {expert, first position, rows, src0 | src1 << 16}
  int tile, j;
};

// elements per 16-byte code vector: 32 (MXFP4) or 16 (MXFP8)
template <bool FP8>
constexpr int kVecElems = FP8 ? 16 : 32;

template <int JM, bool FP8>
__device__ __forceinline__ void gu_issue(ColBuf<JM>& b, const uint8_t* gu_q, const uint8_t* gu_s, const GuItem& it,
                                         int H, int I, int lane) {
  const int VR = H / kVecElems<FP8>, row_bytes = FP8 ? H : H / 2;
  const uint32_t qbytes = (uint32_t)(2 * I * row_bytes), sbytes = (uint32_t)(2 * I * (H / 32));
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(gu_q + (int64_t)it.rec.x * qbytes, qbytes);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(gu_s + (int64_t)it.rec.x * sbytes, sbytes);
#pragma unroll
  for (int jj = 0; jj < JM; ++jj) {
    const int v = lane + 64 * jj;
    const bool up = v >= VR;
    const int bb = v - (up ? VR : 0);
    const bool ok = it.tile >= 0 && v < 2 * VR;
    const uint32_t row = (uint32_t)(it.j + (up ? I : 0));
    const uint32_t qo = row * (uint32_t)row_bytes + 16u * (uint32_t)bb;
    const uint32_t so = row * (uint32_t)(H / 32) + (uint32_t)(FP8 ? bb >> 1 : bb);
    b.q[jj] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)(ok ? qo : kOob), 0, 0));
    b.s[jj] = __builtin_amdgcn_raw_buffer_load_b8(rs, (int)(ok ? so : kOob), 0, 0);
  }
}

// blocks blk of nblk run the gate/up loop; lds holds x rows [T][H] bf16.
// MPL = 0: the tiles come from the one-block routing's records (tiles,
// tile_rows); MPL > 0: every wave routes for itself from the scores
// (route_wave_small, MPL = experts per lane), and wave 0 of block 0 writes
// the routing for the launches that follow.
template <int JM, int TM, bool FP8, int MPL = 0>
__device__ __forceinline__ void gate_up_valu_blocks(const GateUpValuParams& p, int max_tiles, int blk, int nblk,
                                                    uint8_t* lds) {
  uint16_t* x_lds = reinterpret_cast<uint16_t*>(lds);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int T = p.tokens, H = p.hidden, I = p.inter, VR = H / kVecElems<FP8>;

  // x staging loads go out first (they need no routing)
  const int x_pieces = T * (H / 8);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(p.x, (uint32_t)(T * H * 2));
  auto x_off = [&](int q) {
    const int t = q / (H / 8), c = q - t * (H / 8);
    return (uint32_t)((t * H + 8 * c) * 2);
  };
  StageBatch<4> xb;
  int c_e, c_m, c_r, c_s, n_live;
  if constexpr (MPL > 0) {
    stage_issue<4>(xb, rx, x_pieces, 0, x_off);
    const WaveRoute rt = route_wave_small<MPL>(p.scores, T, p.n_experts, p.top_k, p.route_scale);
    c_e = min(max(rt.t_e, 0), p.n_experts - 1);
    c_m = rt.t_m;
    c_r = min(rt.t_r, T);
    c_s = rt.t_src;
    n_live = rt.n_tiles;
    if (blk == 0 && wave == 0 && lane < T * p.top_k) {
      p.idx[lane] = rt.e;
      p.w[lane] = rt.w;
      p.slot_pos[lane] = rt.pos;
      p.sorted_slots[rt.pos] = lane;
    }
  } else {
    // tile records: lane t < max_tiles loads record t and its first two token
    // rows (one round trip, every wave for itself); the live ones are moved to
    // the lowest lanes in order, so lane i holds live tile i
    const bool in = lane < max_tiles;
    const GemmTile tl = in ? p.tiles[lane] : GemmTile{0, 0, 0, 0};
    const int r0 = in ? p.tile_rows[lane * kTileRows] : 0, r1 = in ? p.tile_rows[lane * kTileRows + 1] : 0;
    // x staging loads go out together with the records
    stage_issue<4>(xb, rx, x_pieces, 0, x_off);
    const int rows = min(tl.m_end - tl.m_begin, T);
    const bool live = in && rows > 0;
    const uint64_t live_mask = __ballot(live);
    n_live = __popcll(live_mask);
    const int rank = __popcll(live_mask & ((1ull << lane) - 1ull));
    const int dst = 4 * (live ? rank : n_live + (lane - rank));
    c_e = __builtin_amdgcn_ds_permute(dst, tl.e);
    c_m = __builtin_amdgcn_ds_permute(dst, tl.m_begin);
    c_r = __builtin_amdgcn_ds_permute(dst, rows);
    c_s = __builtin_amdgcn_ds_permute(dst, min(max(r0, 0), T - 1) | (min(max(r1, 0), T - 1) << 16));
  }
  const int total = n_live * I;
  const int W = nblk * kValuWaves;
  const int wg = blk * kValuWaves + wave;

  auto item = [&](int it) {
    GuItem g;
    const bool ok = it < total;
    const int ti = ok ? it / I : 0;
    g.tile = ok ? ti : -1;
    g.j = ok ? it - ti * I : 0;
    g.rec.x = __builtin_amdgcn_readlane(c_e, ti);
    g.rec.y = __builtin_amdgcn_readlane(c_m, ti);
    g.rec.z = __builtin_amdgcn_readlane(c_r, ti);
    g.rec.w = __builtin_amdgcn_readlane(c_s, ti);
    return g;
  };
  ColBuf<JM> b0, b1;
  GuItem g0 = item(wg);
  gu_issue<JM, FP8>(b0, p.gu_q, p.gu_s, g0, H, I, lane);

  stage_commit<4>(xb, x_pieces, 0, lds);
  stage_pieces<4>(rx, x_pieces, lds, x_off, 4 * kValuBlock);  // T = 2 rows beyond the first batch
  __syncthreads();
  if (wg >= total) return;

  auto compute = [&](const ColBuf<JM>& b, const GuItem& g) {
    float gs[TM], us[TM];
#pragma unroll
    for (int r = 0; r < TM; ++r) gs[r] = us[r] = 0.f;
#pragma unroll
    for (int jj = 0; jj < JM; ++jj) {
      // one vector at a time: hoisting every vector's LDS reads ahead of the
      // arithmetic would double the registers and halve the waves per SIMD
      __builtin_amdgcn_sched_barrier(0);
      const int v = lane + 64 * jj;
      const bool up = v >= VR;
      const int bb = min(v - (up ? VR : 0), VR - 1);  // past the pair the codes are zero
      const float scale = e8m0_scale_operand(b.s[jj]);
#pragma unroll
      for (int r = 0; r < TM; ++r) {
        if (r >= g.rec.z) break;  // wave-uniform
        const int src = r ? (g.rec.w >> 16) : (g.rec.w & 0xffff);
        const float d = mx_dot_vec<FP8>(b.q[jj], scale, x_lds + src * H + kVecElems<FP8> * bb, 0.f);
        gs[r] += up ? 0.f : d;
        us[r] += up ? d : 0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < TM; ++r) {
      if (r >= g.rec.z) break;
      const float gsum = wave_sum_f32(gs[r]), usum = wave_sum_f32(us[r]);
      if (lane == 0) p.h[(int64_t)(g.rec.y + r) * I + g.j] = f32_to_bf16(clamped_swiglu(gsum, usum, p.limit));
    }
  };

  for (int it = wg; it < total; it += 2 * W) {
    const GuItem g1 = item(it + W);
    gu_issue<JM, FP8>(b1, p.gu_q, p.gu_s, g1, H, I, lane);
    compute(b0, g0);
    g0 = item(it + 2 * W);
    gu_issue<JM, FP8>(b0, p.gu_q, p.gu_s, g0, H, I, lane);
    if (g1.tile >= 0) compute(b1, g1);
  }
}

template <int JM, int TM, bool FP8>
__global__ __launch_bounds__(kValuBlock) void gate_up_valu_kernel(GateUpValuParams p, int max_tiles) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  gate_up_valu_blocks<JM, TM, FP8>(p, max_tiles, (int)blockIdx.x, (int)gridDim.x, lds);
}

// ---------------------------------------------------------------- shared expert down
// Rows n of W_sd (bf16 [H][I_s]) against h_sh (T rows staged in LDS):
// y_sh[t][n], one row per wave at a time, grid-stride with two buffers.
template <int KVD, int TM>
__device__ __forceinline__ void shared_down_blocks(const MidValuParams& m, int blk, int nblk, uint8_t* lds) {
  uint16_t* h_lds = reinterpret_cast<uint16_t*>(lds);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int H = m.hidden, Is = m.shared_inter, T = m.tokens;
  const int W = nblk * kValuWaves, wg = blk * kValuWaves + wave;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(m.sh_dn, (uint32_t)((int64_t)H * Is * 2));
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(m.h_sh, (uint32_t)(T * Is * 2));
  const int pieces = T * (Is / 8);
  auto h_off = [&](int q) {
    const int t = q / (Is / 8), c = q - t * (Is / 8);
    return (uint32_t)((t * Is + 8 * c) * 2);
  };
  StageBatch<4> hb;
  stage_issue<4>(hb, rh, pieces, 0, h_off);
  auto issue = [&](ValuRows<8, KVD, 1>& b, int n) {
    const uint32_t off[1] = {n < H ? (uint32_t)n * (uint32_t)Is * 2u : kOob};
    valu_issue<8, KVD, 1>(b, rw, off, Is);
  };
  auto compute = [&](const ValuRows<8, KVD, 1>& b, int n) {
    float out[1][TM];
    valu_compute<8, KVD, 1, TM>(b, h_lds, Is, T, Is, out);
    if (lane == 0)
#pragma unroll
      for (int t = 0; t < TM; ++t)
        if (t < T) m.y_sh[(int64_t)t * H + n] = f32_to_bf16(out[0][t]);
  };
  ValuRows<8, KVD, 1> b0, b1;
  issue(b0, wg);
  stage_commit<4>(hb, pieces, 0, lds);
  stage_pieces<4>(rh, pieces, lds, h_off, 4 * kValuBlock);
  __syncthreads();
  for (int n = wg; n < H; n += 2 * W) {
    issue(b1, n + W);
    compute(b0, n);
    issue(b0, n + 2 * W);
    if (n + W < H) compute(b1, n + W);
  }
}

// Blocks [0, gu_blocks) run the routed gate/up loop, the rest the shared
// expert's down loop; the two are independent and stream together.  MPL > 0:
// the gate/up waves route for themselves from the router's scores (no
// routing launch between the router and the routed weights).
template <int JM, int TM, int KVD, bool FP8, int MPL = 0>
__global__ __launch_bounds__(kValuBlock) void gate_up_shared_down_kernel(GateUpValuParams p, int max_tiles,
                                                                         MidValuParams m, int gu_blocks) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int b = (int)blockIdx.x;
  if (b < gu_blocks)
    gate_up_valu_blocks<JM, TM, FP8, MPL>(p, MPL > 0 ? kMaxLiveTiles : max_tiles, b, gu_blocks, lds);
  else
    shared_down_blocks<KVD, TM>(m, b - gu_blocks, (int)gridDim.x - gu_blocks, lds);
}

// Launch 2 of the three-launch streaming layer: blocks [0, gu_blocks) run the
// routed gate/up loop, each wave routing for itself from the router's scores
// (so no routing launch sits between the router and the routed weights), the
// rest stream the shared expert's gate/up row pairs, one pair per wave.
template <int JM, int TM, bool FP8, int MPL>
__global__ __launch_bounds__(kValuBlock) void route_gate_up_shared_gu_kernel(GateUpValuParams p, FrontValuParams f,
                                                                             int gu_blocks) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int b = (int)blockIdx.x;
  if (b < gu_blocks) {
    gate_up_valu_blocks<JM, TM, FP8, MPL>(p, kMaxLiveTiles, b, gu_blocks, lds);
  } else {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    shared_gate_up_pair(f.x, f.sh_gu, f.h_sh, f.tokens, f.hidden, f.shared_inter, f.limit, (b - gu_blocks) * 4 + wave,
                        reinterpret_cast<uint16_t*>(lds));
  }
}

// ---------------------------------------------------------------- down + combine
// KVS > 0: the shared expert's down projection is folded in: column n also
// reads row n of sh_dn (KVS 16-byte vectors of bf16 per lane) against h_sh
// staged after the slots' h rows, and its product is added in fp32 to every
// token's sum before the one rounding to bf16.
template <int JM, int TM, bool FP8, int KVS = 0>
__global__ __launch_bounds__(kValuBlock) void down_combine_valu_kernel(DownValuParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];  // h of every slot [n][I] bf16, then h_sh [T][I_s]
  uint16_t* h_lds = reinterpret_cast<uint16_t*>(lds);
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int T = p.tokens, k = p.top_k, n = T * k;
  const int H = p.hidden, I = p.inter, VR = I / kVecElems<FP8>, row_bytes = FP8 ? I : I / 2;
  const int Is = KVS > 0 ? p.shared_inter : 0;
  uint16_t* hs_lds = h_lds + n * I;
  // lane s < n holds slot s: expert, position of its h row, weight
  const int ls = min(lane, n - 1);
  const int my_e = p.idx[ls];
  const int my_p = p.slot_pos[ls];
  const float my_w = p.topk_w[ls];

  // vector v = lane + 64 jj is block vb of slot vs's row (vs = -1: past the
  // last slot, its load repeats a valid address and its product is dropped)
  int vs[JM], vb[JM];
  float vw[JM];
  const uint8_t* qrow[JM];
  const uint8_t* srow[JM];
#pragma unroll
  for (int jj = 0; jj < JM; ++jj) {
    const int v = lane + 64 * jj;
    const int s = min(v / VR, n - 1);
    vs[jj] = v < n * VR ? s : -1;
    vb[jj] = v - s * VR < VR ? v - s * VR : VR - 1;
    vw[jj] = __shfl(my_w, s);
    const int64_t er = (int64_t)__shfl(my_e, s) * H;
    qrow[jj] = p.dn_q + er * row_bytes + 16 * vb[jj];
    srow[jj] = p.dn_s + er * (I / 32) + (FP8 ? vb[jj] >> 1 : vb[jj]);
  }
  const int W = (int)gridDim.x * kValuWaves;
  const int wg = (int)blockIdx.x * kValuWaves + wave;
  // a column past the end re-reads column H - 1 (cached) and is not stored
  const __amdgpu_buffer_rsrc_t rsh = make_rsrc(p.y_shared, p.y_shared ? (uint32_t)(T * H * 2) : 0u);
  const __amdgpu_buffer_rsrc_t rsd = make_rsrc(p.sh_dn, KVS > 0 ? (uint32_t)((int64_t)H * Is * 2) : 0u);
  constexpr int KVS1 = KVS > 0 ? KVS : 1;
  ValuRows<8, KVS1, 1> sd0, sd1;  // the shared row of each column buffer
  auto issue = [&](ColBuf<JM>& b, ValuRows<8, KVS1, 1>& sd, int col) {
    const int64_t c = min(col, H - 1);
#pragma unroll
    for (int jj = 0; jj < JM; ++jj) {
      b.q[jj] = *reinterpret_cast<const u32x4_t*>(qrow[jj] + c * row_bytes);
      b.s[jj] = srow[jj][c * (I / 32)];
    }
    if constexpr (KVS > 0) {
      const uint32_t off[1] = {(uint32_t)c * (uint32_t)Is * 2u};
      valu_issue<8, KVS1, 1>(sd, rsd, off, Is);
    } else {
      b.ysh =
          __builtin_amdgcn_raw_buffer_load_b16(rsh, (int)(lane < T ? (uint32_t)((lane * H + c) * 2) : kOob), 0, 0);
    }
  };

  // h staging (slot order): the first batch goes out before the first
  // column's weights and is stored while they are in flight
  const int per_row = I / 8, h_pieces = n * per_row;
  const __amdgpu_buffer_rsrc_t rh = make_rsrc(p.h, (uint32_t)(n * I * 2));
  auto h_off = [&](int q) {
    const int s = q / per_row, c = q - s * per_row;
    return (uint32_t)((__shfl(my_p, s) * I + 8 * c) * 2);
  };
  StageBatch<8> hb;
  stage_issue<8>(hb, rh, h_pieces, 0, h_off);
  ColBuf<JM> b0, b1;
  issue(b0, sd0, wg);
  stage_commit<8>(hb, h_pieces, 0, lds);
  stage_pieces<8>(rh, h_pieces, lds, h_off, 8 * kValuBlock);
  if constexpr (KVS > 0) valu_stage_rows(p.h_sh, Is, T, Is, hs_lds);
  __syncthreads();
  if (wg >= H) return;

  auto compute = [&](const ColBuf<JM>& b, const ValuRows<8, KVS1, 1>& sd, int col) {
    float acc[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t) acc[t] = 0.f;
    if constexpr (KVS > 0) {
      float sh[1][TM];
#pragma unroll
      for (int t = 0; t < TM; ++t) sh[0][t] = 0.f;
      valu_accumulate<8, KVS1, 1, TM>(sd, hs_lds, Is, T, Is, sh);
#pragma unroll
      for (int t = 0; t < TM; ++t) acc[t] = sh[0][t];
    }
#pragma unroll
    for (int jj = 0; jj < JM; ++jj) {
      __builtin_amdgcn_sched_barrier(0);  // one vector at a time (registers)
      const int s = max(vs[jj], 0);
      const float d = mx_dot_vec<FP8>(b.q[jj], e8m0_scale_operand(b.s[jj]), h_lds + s * I + kVecElems<FP8> * vb[jj],
                                      0.f);
      const float wd = vs[jj] >= 0 ? vw[jj] * d : 0.f;
      const int t = s / k;
#pragma unroll
      for (int tt = 0; tt < TM; ++tt) acc[tt] += t == tt ? wd : 0.f;
    }
    float r = 0.f;
#pragma unroll
    for (int t = 0; t < TM; ++t) {
      const float st = wave_sum_f32(acc[t]);
      r = lane == t ? st : r;
    }
    if (lane < T) p.y[(int64_t)lane * H + col] = f32_to_bf16(KVS > 0 ? r : r + bf16_to_f32((uint16_t)b.ysh));
  };

  for (int col = wg; col < H; col += 2 * W) {
    issue(b1, sd1, col + W);
    compute(b0, sd0, col);
    issue(b0, sd0, col + 2 * W);
    if (col + W < H) compute(b1, sd1, col + W);
  }
}

// instantiated vector counts per lane; the smallest >= the need is used
constexpr int kGateUpJm[] = {2, 4, 5, 7, 8};
constexpr int kDownJm[] = {2, 4, 7, 9, 14};
constexpr int kGateUpJm8[] = {2, 4, 10, 14};  // MXFP8: twice the vectors of a row
constexpr int kDownJm8[] = {2, 4, 7, 14};
// blocks per CU of the grid-stride loops (all resident at once)
constexpr int kGateUpBlocksPerCu = 2;
constexpr int kDownBlocksPerCu = 2;
constexpr int kSharedDownBlocksPerCu = 1;

template <size_t N>
int first_at_least(const int (&js)[N], int need) {
  for (int j : js)
    if (j >= need) return j;
  return 0;
}

int gate_up_jm(int hidden, bool fp8) {
  const int need = (2 * (hidden / (fp8 ? 16 : 32)) + 63) / 64;
  return fp8 ? first_at_least(kGateUpJm8, need) : first_at_least(kGateUpJm, need);
}

int down_jm(int slots, int inter, bool fp8) {
  const int need = (slots * (inter / (fp8 ? 16 : 32)) + 63) / 64;
  return fp8 ? first_at_least(kDownJm8, need) : first_at_least(kDownJm, need);
}

using GateUpKernel = void (*)(GateUpValuParams, int);
using GateUpSdKernel = void (*)(GateUpValuParams, int, MidValuParams, int);
using DownKernel = void (*)(DownValuParams);
using GateUpSdKernel2 = void (*)(GateUpValuParams, FrontValuParams, int);

template <int TM, int KVD, bool FP8, int MPL>
GateUpSdKernel pick_gate_up_sd_t(int jm) {
  if constexpr (FP8) {
    switch (jm) {
      case 2: return gate_up_shared_down_kernel<2, TM, KVD, true, MPL>;
      case 4: return gate_up_shared_down_kernel<4, TM, KVD, true, MPL>;
      case 10: return gate_up_shared_down_kernel<10, TM, KVD, true, MPL>;
      case 14: return gate_up_shared_down_kernel<14, TM, KVD, true, MPL>;
      default: return nullptr;
    }
  } else {
    switch (jm) {
      case 2: return gate_up_shared_down_kernel<2, TM, KVD, false, MPL>;
      case 4: return gate_up_shared_down_kernel<4, TM, KVD, false, MPL>;
      case 5: return gate_up_shared_down_kernel<5, TM, KVD, false, MPL>;
      case 7: return gate_up_shared_down_kernel<7, TM, KVD, false, MPL>;
      case 8: return gate_up_shared_down_kernel<8, TM, KVD, false, MPL>;
      default: return nullptr;
    }
  }
}
template <bool FP8, int MPL>
GateUpSdKernel pick_gate_up_sd_f(int jm, int tokens, int kvd) {
  if (kvd == 5) return tokens == 1 ? pick_gate_up_sd_t<1, 5, FP8, MPL>(jm) : pick_gate_up_sd_t<2, 5, FP8, MPL>(jm);
  if (kvd == 10) return tokens == 1 ? pick_gate_up_sd_t<1, 10, FP8, MPL>(jm) : pick_gate_up_sd_t<2, 10, FP8, MPL>(jm);
  return nullptr;
}
template <int MPL>
GateUpSdKernel pick_gate_up_sd_m(int jm, int tokens, int kvd, bool fp8) {
  return fp8 ? pick_gate_up_sd_f<true, MPL>(jm, tokens, kvd) : pick_gate_up_sd_f<false, MPL>(jm, tokens, kvd);
}
// mpl = 0: tiles from the routing launch; 2, 6, 16: in-wave routing (route_mpl)
GateUpSdKernel pick_gate_up_sd(int jm, int tokens, int kvd, bool fp8, int mpl = 0) {
  switch (mpl) {
    case 0: return pick_gate_up_sd_m<0>(jm, tokens, kvd, fp8);
    case 2: return pick_gate_up_sd_m<2>(jm, tokens, kvd, fp8);
    case 6: return pick_gate_up_sd_m<6>(jm, tokens, kvd, fp8);
    case 16: return pick_gate_up_sd_m<16>(jm, tokens, kvd, fp8);
    default: return nullptr;
  }
}

template <int TM, bool FP8>
GateUpKernel pick_gate_up_t(int jm) {
  if constexpr (FP8) {
    switch (jm) {
      case 2: return gate_up_valu_kernel<2, TM, true>;
      case 4: return gate_up_valu_kernel<4, TM, true>;
      case 10: return gate_up_valu_kernel<10, TM, true>;
      case 14: return gate_up_valu_kernel<14, TM, true>;
      default: return nullptr;
    }
  } else {
    switch (jm) {
      case 2: return gate_up_valu_kernel<2, TM, false>;
      case 4: return gate_up_valu_kernel<4, TM, false>;
      case 5: return gate_up_valu_kernel<5, TM, false>;
      case 7: return gate_up_valu_kernel<7, TM, false>;
      case 8: return gate_up_valu_kernel<8, TM, false>;
      default: return nullptr;
    }
  }
}
GateUpKernel pick_gate_up(int jm, int tokens, bool fp8) {
  if (fp8) return tokens == 1 ? pick_gate_up_t<1, true>(jm) : pick_gate_up_t<2, true>(jm);
  return tokens == 1 ? pick_gate_up_t<1, false>(jm) : pick_gate_up_t<2, false>(jm);
}

template <int TM, bool FP8>
DownKernel pick_down_t(int jm) {
  if constexpr (FP8) {
    switch (jm) {
      case 2: return down_combine_valu_kernel<2, TM, true>;
      case 4: return down_combine_valu_kernel<4, TM, true>;
      case 7: return down_combine_valu_kernel<7, TM, true>;
      case 14: return down_combine_valu_kernel<14, TM, true>;
      default: return nullptr;
    }
  } else {
    switch (jm) {
      case 2: return down_combine_valu_kernel<2, TM, false>;
      case 4: return down_combine_valu_kernel<4, TM, false>;
      case 7: return down_combine_valu_kernel<7, TM, false>;
      case 9: return down_combine_valu_kernel<9, TM, false>;
      case 14: return down_combine_valu_kernel<14, TM, false>;
      default: return nullptr;
    }
  }
}
DownKernel pick_down(int jm, int tokens, bool fp8) {
  if (fp8) return tokens == 1 ? pick_down_t<1, true>(jm) : pick_down_t<2, true>(jm);
  return tokens == 1 ? pick_down_t<1, false>(jm) : pick_down_t<2, false>(jm);
}

template <int TM, bool FP8, int MPL>
GateUpSdKernel2 pick_route_gate_up_t(int jm) {
  if constexpr (FP8) {
    switch (jm) {
      case 2: return route_gate_up_shared_gu_kernel<2, TM, true, MPL>;
      case 4: return route_gate_up_shared_gu_kernel<4, TM, true, MPL>;
      case 10: return route_gate_up_shared_gu_kernel<10, TM, true, MPL>;
      case 14: return route_gate_up_shared_gu_kernel<14, TM, true, MPL>;
      default: return nullptr;
    }
  } else {
    switch (jm) {
      case 2: return route_gate_up_shared_gu_kernel<2, TM, false, MPL>;
      case 4: return route_gate_up_shared_gu_kernel<4, TM, false, MPL>;
      case 5: return route_gate_up_shared_gu_kernel<5, TM, false, MPL>;
      case 7: return route_gate_up_shared_gu_kernel<7, TM, false, MPL>;
      case 8: return route_gate_up_shared_gu_kernel<8, TM, false, MPL>;
      default: return nullptr;
    }
  }
}
// experts per lane of the in-wave routing: 2 (E <= 128), 6 (E <= 384) or 16 (E <= 1024)
int route_mpl(int n_experts) { return n_experts <= 128 ? 2 : n_experts <= 384 ? 6 : 16; }
template <bool FP8>
GateUpSdKernel2 pick_route_gate_up_f(int jm, int tokens, int mpl) {
  if (mpl == 2) return tokens == 1 ? pick_route_gate_up_t<1, FP8, 2>(jm) : pick_route_gate_up_t<2, FP8, 2>(jm);
  if (mpl == 6) return tokens == 1 ? pick_route_gate_up_t<1, FP8, 6>(jm) : pick_route_gate_up_t<2, FP8, 6>(jm);
  return tokens == 1 ? pick_route_gate_up_t<1, FP8, 16>(jm) : pick_route_gate_up_t<2, FP8, 16>(jm);
}
GateUpSdKernel2 pick_route_gate_up(int jm, int tokens, int mpl, bool fp8) {
  return fp8 ? pick_route_gate_up_f<true>(jm, tokens, mpl) : pick_route_gate_up_f<false>(jm, tokens, mpl);
}

template <int TM, bool FP8, int KVS>
DownKernel pick_down_shared_t(int jm) {
  if constexpr (FP8) {
    switch (jm) {
      case 2: return down_combine_valu_kernel<2, TM, true, KVS>;
      case 4: return down_combine_valu_kernel<4, TM, true, KVS>;
      case 7: return down_combine_valu_kernel<7, TM, true, KVS>;
      case 14: return down_combine_valu_kernel<14, TM, true, KVS>;
      default: return nullptr;
    }
  } else {
    switch (jm) {
      case 2: return down_combine_valu_kernel<2, TM, false, KVS>;
      case 4: return down_combine_valu_kernel<4, TM, false, KVS>;
      case 7: return down_combine_valu_kernel<7, TM, false, KVS>;
      case 9: return down_combine_valu_kernel<9, TM, false, KVS>;
      case 14: return down_combine_valu_kernel<14, TM, false, KVS>;
      default: return nullptr;
    }
  }
}
template <bool FP8>
DownKernel pick_down_shared_f(int jm, int tokens, int kvs) {
  if (kvs == 5) return tokens == 1 ? pick_down_shared_t<1, FP8, 5>(jm) : pick_down_shared_t<2, FP8, 5>(jm);
  return tokens == 1 ? pick_down_shared_t<1, FP8, 10>(jm) : pick_down_shared_t<2, FP8, 10>(jm);
}
DownKernel pick_down_shared(int jm, int tokens, int kvs, bool fp8) {
  return fp8 ? pick_down_shared_f<true>(jm, tokens, kvs) : pick_down_shared_f<false>(jm, tokens, kvs);
}

int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (!cached[dev]) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    cached[dev] = v;
  }
  return cached[dev];
}

int valu_grid(int64_t columns, int blocks_per_cu) {
  const int64_t want = (int64_t)blocks_per_cu * device_cus();
  const int64_t need = (columns + kValuWaves - 1) / kValuWaves;
  return (int)(need < want ? need : want);
}

}  // namespace

bool gate_up_valu_supported(int tokens, int hidden, int max_tiles, bool fp8) {
  return tokens >= 1 && tokens <= kValuMaxTokens && hidden % 32 == 0 && hidden <= 8192 &&
         max_tiles <= kMaxLiveTiles && gate_up_jm(hidden, fp8) > 0;
}

bool down_valu_supported(int tokens, int top_k, int inter, bool fp8) {
  const int n = tokens * top_k;
  return tokens >= 1 && tokens <= kValuMaxTokens && inter % 32 == 0 && (int64_t)n * inter * 2 <= 64 * 1024 &&
         down_jm(n, inter, fp8) > 0;
}

hipError_t launch_gate_up_valu(const GateUpValuParams& p, int max_tiles, hipStream_t stream) {
  const dim3 grid(valu_grid((int64_t)max_tiles * p.inter, kGateUpBlocksPerCu));
  const size_t lds = (size_t)p.tokens * p.hidden * 2;
  auto kern = pick_gate_up(gate_up_jm(p.hidden, p.fp8), p.tokens, p.fp8);
  if (!kern) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, grid, dim3(kValuBlock), lds, stream, p, max_tiles);
  return hipGetLastError();
}

bool gate_up_shared_down_supported(int tokens, int hidden, int max_tiles, int shared_inter, bool fp8) {
  return gate_up_valu_supported(tokens, hidden, max_tiles, fp8) && shared_inter > 0 && shared_inter % 8 == 0 &&
         shared_inter <= 10 * 8 * 64;
}

hipError_t launch_gate_up_shared_down(const GateUpValuParams& p, int max_tiles, const MidValuParams& m,
                                      hipStream_t stream) {
  const int gu_blocks = valu_grid((int64_t)max_tiles * p.inter, kGateUpBlocksPerCu);
  const int sd_blocks = valu_grid(m.hidden, kSharedDownBlocksPerCu);
  const int kvd = m.shared_inter <= 5 * 8 * 64 ? 5 : 10;
  auto kern = pick_gate_up_sd(gate_up_jm(p.hidden, p.fp8), p.tokens, kvd, p.fp8);
  if (!kern) return hipErrorInvalidValue;
  const size_t lx = (size_t)p.tokens * p.hidden * 2, lh = (size_t)m.tokens * m.shared_inter * 2;
  hipLaunchKernelGGL(kern, dim3((unsigned)(gu_blocks + sd_blocks)), dim3(kValuBlock), lx > lh ? lx : lh, stream, p,
                     max_tiles, m, gu_blocks);
  return hipGetLastError();
}

hipError_t launch_route_gate_up_shared_down(const GateUpValuParams& p, const MidValuParams& m, hipStream_t stream) {
  // as many (tile, column) items as the routing can produce: T * k tiles of I columns
  const int gu_blocks = valu_grid((int64_t)p.tokens * p.top_k * p.inter, kGateUpBlocksPerCu);
  const int sd_blocks = valu_grid(m.hidden, kSharedDownBlocksPerCu);
  const int kvd = m.shared_inter <= 5 * 8 * 64 ? 5 : 10;
  auto kern = pick_gate_up_sd(gate_up_jm(p.hidden, p.fp8), p.tokens, kvd, p.fp8, route_mpl(p.n_experts));
  if (!kern) return hipErrorInvalidValue;
  const size_t lx = (size_t)p.tokens * p.hidden * 2, lh = (size_t)m.tokens * m.shared_inter * 2;
  hipLaunchKernelGGL(kern, dim3((unsigned)(gu_blocks + sd_blocks)), dim3(kValuBlock), lx > lh ? lx : lh, stream, p,
                     kMaxLiveTiles, m, gu_blocks);
  return hipGetLastError();
}

bool route_gate_up_shared_gu_supported(int tokens, int hidden, int n_experts, int top_k, int shared_inter, bool fp8) {
  return gate_up_valu_supported(tokens, hidden, kMaxLiveTiles, fp8) && tokens * top_k <= 64 && n_experts <= 1024 &&
         (shared_inter == 0 || shared_inter <= 5120);
}

hipError_t launch_route_gate_up_shared_gu(const GateUpValuParams& p, const FrontValuParams& f, hipStream_t stream) {
  // as many (tile, column) items as the routing can produce: T * k tiles of I columns
  const int gu_blocks = valu_grid((int64_t)p.tokens * p.top_k * p.inter, kGateUpBlocksPerCu);
  const int sh_blocks = f.sh_gu ? (f.shared_inter + 3) / 4 : 0;
  auto kern = pick_route_gate_up(gate_up_jm(p.hidden, p.fp8), p.tokens, route_mpl(p.n_experts), p.fp8);
  if (!kern) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, dim3((unsigned)(gu_blocks + sh_blocks)), dim3(kValuBlock), (size_t)p.tokens * p.hidden * 2,
                     stream, p, f, gu_blocks);
  return hipGetLastError();
}

bool down_combine_shared_supported(int tokens, int top_k, int inter, int shared_inter, bool fp8) {
  return down_valu_supported(tokens, top_k, inter, fp8) && shared_inter > 0 && shared_inter % 8 == 0 &&
         shared_inter <= 10 * 8 * 64 &&
         (int64_t)tokens * top_k * inter * 2 + (int64_t)tokens * shared_inter * 2 <= 64 * 1024;
}

hipError_t launch_down_combine_shared(const DownValuParams& p, hipStream_t stream) {
  const dim3 grid(valu_grid(p.hidden, kDownBlocksPerCu));
  const int n = p.tokens * p.top_k;
  const size_t lds = (size_t)n * p.inter * 2 + (size_t)p.tokens * p.shared_inter * 2;
  const int kvs = p.shared_inter <= 5 * 8 * 64 ? 5 : 10;
  auto kern = pick_down_shared(down_jm(n, p.inter, p.fp8), p.tokens, kvs, p.fp8);
  if (!kern) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, grid, dim3(kValuBlock), lds, stream, p);
  return hipGetLastError();
}

hipError_t launch_down_combine_valu(const DownValuParams& p, hipStream_t stream) {
  const dim3 grid(valu_grid(p.hidden, kDownBlocksPerCu));
  const int n = p.tokens * p.top_k;
  const size_t lds = (size_t)n * p.inter * 2;
  auto kern = pick_down(down_jm(n, p.inter, p.fp8), p.tokens, p.fp8);
  if (!kern) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kern, grid, dim3(kValuBlock), lds, stream, p);
  return hipGetLastError();
}

}  // namespace moe
