// Host-side launch interface between the C ABI (moe_ffn.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- router
struct RouterPlan {
  int mt;                // 16-token row tiles per block (1 or 4)
  int ksplit;            // number of partial logit matrices the top-k adds
  int chunks_per_split;  // 128-wide K chunks per range
  // > 0: W_r is split into three bf16 matrices (hi, mid, lo) in the
  // workspace and the dense pipelined GEMM runs each over this many K ranges
  // (ksplit = 3 * dense_kslices); 0: router_logits_kernel
  int dense_kslices;
  // the whole-round dense kernel over dense_kslices K ranges, the three terms
  // added in its registers (ksplit = dense_kslices)
  bool whole_round;
};
RouterPlan router_plan(int64_t tokens, int n_experts, int hidden);
// workspace bytes for the split weights (0 unless plan.dense_kslices > 0)
size_t router_w3_bytes(const RouterPlan& plan, int n_experts, int hidden);

// partial logits [ksplit][T][E] fp32; w3: router_w3_bytes of workspace
hipError_t launch_router_logits(const RouterPlan& plan, const uint16_t* x, const float* router_w, float* part,
                                int tokens, int n_experts, int hidden, uint16_t* w3, hipStream_t stream);
// few tokens: full fp32 logits [T][E] by a weight-streaming GEMV (logits optional);
// with `scores` non-null also s = sqrtsoftplus(l) at scores[t][e] and
// u = s + bias[e] at scores[T + t][e] (bias optional)
hipError_t launch_router_gemv(const uint16_t* x, const float* router_w, float* logits, int tokens, int n_experts,
                              int hidden, float* scores, const float* bias, hipStream_t stream);
// launch_router_gemv's scores (no logits) with the pre-FFN RMSNorm in front,
// for 1 or 2 tokens and hidden <= 5120; the normalised rows go to x_norm [T][H]
bool router_norm_gemv_supported(int tokens, int hidden);
hipError_t launch_router_norm_gemv(const uint16_t* x, const uint16_t* gamma, double eps, uint16_t* x_norm,
                                   const float* router_w, int tokens, int n_experts, int hidden, float* scores,
                                   const float* bias, hipStream_t stream);
// pre-FFN RMSNorm of T rows (x_norm may be x)
hipError_t launch_rmsnorm_rows(const uint16_t* x, const uint16_t* gamma, uint16_t* x_norm, int rows, int hidden,
                               double eps, hipStream_t stream);
// sum of the partials, sqrtsoftplus, biased top-k, weights
hipError_t launch_router_topk(const float* part, int ksplit, const float* bias, int tokens, int n_experts,
                              int top_k, float route_scale, int32_t* idx, float* w, float* gap,
                              hipStream_t stream);

// ---------------------------------------------------------------- permute
constexpr int kPermuteChunk = 1024;
inline int permute_chunks(int64_t n) { return (int)((n + kPermuteChunk - 1) / kPermuteChunk); }

// Tile of a grouped GEMM: rows [m_begin, m_end) of expert e's run.
struct GemmTile {
  int e, m_begin, m_end, pad;
};
// Few-token tiles also carry the source row (token) of each of their at most
// kTileRows rows: tile_rows[tile * kTileRows + r].
constexpr int kTileRows = 8;
inline int64_t max_gemm_tiles(int64_t n, int n_experts, int bm) {
  return (n + bm - 1) / bm + (n < n_experts ? n : n_experts);
}

struct PermuteScratch {
  int32_t* rank;          // [n]
  int32_t* chunk_counts;  // [nchunks][E]
  int32_t* chunk_base;    // [nchunks][E]
};
// Stable counting sort of the flat slots by expert; optionally also writes
// the tile table for a grouped GEMM with `bm` rows per tile (tiles != NULL).
hipError_t launch_permute(const int32_t* idx, int n, int n_experts, const PermuteScratch& s,
                          int32_t* offsets, int32_t* sorted_slots, int32_t* slot_pos, int bm, int max_tiles,
                          GemmTile* tiles, int32_t* tile_count, hipStream_t stream);
// Tile table from expert offsets alone.
// At most max_tiles tiles are written (the size of the tile array).
hipError_t launch_tile_table(const int32_t* offsets, int n_experts, int n_total, int bm, int max_tiles,
                             GemmTile* tiles, int32_t* tile_count, hipStream_t stream);

// ---------------------------------------------------------------- expert GEMMs
struct GemmParams {
  // grouped mode: tiles/tile_count from the permutation; dense mode: tiles == NULL, rows [0, M)
  const GemmTile* tiles;
  const int32_t* tile_count;
  int M;
  // A rows: A + (gather ? gather[p] / gather_div : p) * lda, bf16 [.][K]
  const int32_t* gather;
  int gather_div;
  const uint16_t* A;
  int64_t lda;
  int a_rows;  // rows of A; gathered row indices are clamped into [0, a_rows)
  int K;
  // B (weights), per expert: MXFP4 or MXFP8 codes/scales, or bf16, rows [.][K]
  const uint8_t* bq;
  const uint8_t* bs;
  const uint16_t* bh;
  int64_t b_expert_rows;  // B rows per expert
  int b_row_second;       // first row of the up half (SwiGLU)
  // output bf16 [.][N], row = position p
  int N;
  uint16_t* C;
  int64_t ldc;
  float limit;
  // fp32 slices of the dense kernel (launch_dense_f32): slice s = z * k_slices
  // + k-part, weights bh + z * b_slice_stride, output Cf + s * c_slice_stride
  float* Cf;
  int k_slices;
  int64_t b_slice_stride;
  int64_t c_slice_stride;
};
// rows per tile / 16 for the grouped GEMM (MXFP4, MXFP8 or bf16 weights);
// k_pipelined: every K of the problem is a multiple of 128
// weight codec of a grouped GEMM's B operand
enum WeightFormat : int { kWBf16 = 0, kWMxfp4 = 1, kWMxfp8 = 2 };
int expert_gemm_mt(int64_t n_rows, int n_groups, WeightFormat fmt, bool k_pipelined);
hipError_t launch_expert_gemm(const GemmParams& p, bool swiglu, WeightFormat fmt, int mt, int64_t grid_tiles,
                              hipStream_t stream);
// dense bf16 rows [0, M) of A against `slices` weight slices, fp32 outputs (see GemmParams)
hipError_t launch_dense_f32(const GemmParams& p, int slices, hipStream_t stream);
// the router logits on the whole-round dense kernel from kDenseRouterNtTokens
// tokens: p.bh = the three bf16 terms of W_r [3][N][K], p.k_slices K ranges,
// each written to partial slice Cf + r * c_slice_stride with the terms added
int dense_router_kslices(int M, int n_experts, int K);
// One dense bf16 matrix against at most 512 rows with K a multiple of 128:
// skinny_k_slices K ranges (0: unsupported) of fp32 partials from the
// weight-streaming skinny kernel into `part`, then their sum as
// launch_dense_sliced does.
int skinny_k_slices(int M, int n_rows, int K);
hipError_t launch_skinny_sliced(const GemmParams& p, bool swiglu, int k_slices, float* part, hipStream_t stream);
hipError_t launch_dense_router(const GemmParams& p, hipStream_t stream);
// One dense bf16 matrix (no tiles, no gather) split over K: k_slices fp32
// partial products into `part` ([k_slices][M][N or 2N] floats), then their sum
// (and clamp-SwiGLU with the up rows at b_row_second == N) to C in bf16.
int dense_k_slices(int M, int n_rows, int K);
hipError_t launch_dense_sliced(const GemmParams& p, bool swiglu, int k_slices, float* part, hipStream_t stream);

// Few-token (decode) projections: up to two problems in one launch.
struct GemvProblem {
  const GemmTile* tiles;       // grouped problem (routed experts); NULL: dense rows [0, M)
  const int32_t* tile_count;
  int M;
  int grid_tiles;              // grid.x blocks reserved for this problem (0: absent)
  const int32_t* gather;       // A row of position p: gather[p] / gather_div, else p
  int gather_div;
  int gather_len;              // entries of gather (MXFP4 problems read it with clamped indices)
  const int32_t* tile_rows;    // MXFP4 problems: source row of each tile row (overrides gather), or NULL
  const uint16_t* A;
  int64_t lda;
  int a_rows;
  const uint8_t* amx;          // MXFP4 problems: A rows already in two-term MXFP8 form
                               // (stride mx_row_bytes(K)), else NULL and A is converted
  int K;
  const uint8_t* bq;           // MXFP4 codes (NULL: bf16 weights in bh)
  const uint8_t* bs;
  int w8;                      // bq holds MXFP8 codes (E4M3, one a byte; K a multiple of 128)
  const uint16_t* bh;
  int64_t b_expert_rows;
  int b_row_second;
  int N;
  int col_tiles;               // N / 16
  uint16_t* C;
  int64_t ldc;
  uint8_t* cmx;                // MXFP4 gate/up with rows_cap <= kTileRows: write the output rows in
                               // two-term MXFP8 form (stride mx_row_bytes(N)) instead of C
};
struct GemvParams {
  GemvProblem p[2];
  int rows_cap;  // rows per tile (<= 16), also rows staged in LDS
  float limit;
};
size_t gemv_lds_bytes(int rows_cap, int k_max, bool fp4);
// fp4: one MXFP4 problem (p[0]; tiles of at most rows_cap <= 8 rows, grid over
// 64-column blocks), or MXFP8 with p[0].w8 (K a multiple of 128, no cmx).
// Otherwise up to two dense bf16 problems (bh).
hipError_t launch_expert_gemv(const GemvParams& prm, bool swiglu, bool fp4, hipStream_t stream);

// MXFP4 (or, with w8, MXFP8) few-token down projection, split-K form: one
// block per (tile, 16 output columns), its waves splitting K into ranges of
// kSplitKChunksDown 128-wide chunks.  Problem as for launch_expert_gemv with fp4.
constexpr int kSplitKChunksDown = 5;
bool splitk_supported(int rows_cap, int K);
hipError_t launch_expert_gemv_splitk(const GemvProblem& p, int rows_cap, hipStream_t stream);

// One-block routing of T tokens with T * top_k <= 64 from the scores of
// launch_router_gemv: top-k and weights, the stable permutation and the
// tile table (one tile per selected expert); also the two-term MXFP8 rows
// of x (xmx, stride mx_row_bytes(hidden)) when xmx is non-null.
struct RouteSmallParams {
  const uint16_t* x;
  uint8_t* xmx;
  const float* scores;  // [2][T][E]
  int tokens, n_experts, hidden, top_k;
  float route_scale;
  int32_t* idx;
  float* w;
  int32_t* sorted_slots;
  int32_t* slot_pos;
  GemmTile* tiles;
  int32_t* tile_count;
  int32_t* tile_rows;  // [max_tiles][kTileRows], optional
  int max_tiles;
};
constexpr int kRouteSmallMaxSlots = 64;

// Launch 1 of the few-token layer: router GEMV scores (as launch_router_gemv
// with scores) beside the shared expert's gate/up (dense bf16 problem,
// grid_tiles = 1; grid_tiles = 0 when there is no shared expert).
struct FrontParams {
  const uint16_t* x;
  const float* router_w;
  const float* bias;
  float* scores;
  int tokens, n_experts, hidden;
  GemvProblem shared;
  int rows_cap;
  float limit;
  uint8_t* xmx;  // non-NULL: also write x in two-term MXFP8 form (mx_device.h), [T][mx_row_bytes(H)]
};
hipError_t launch_decode_front(const FrontParams& f, hipStream_t stream);
// T <= 2 forms of the two launches: every weight row streamed by one wave
// on the vector ALUs (gemv_valu_device.h).  sh_gu / sh_dn NULL without a
// shared expert.
struct FrontValuParams {
  const uint16_t* x;
  const float* router_w;
  const float* bias;
  float* scores;           // [2][T][E]
  const uint16_t* sh_gu;   // [2 I_s][H] bf16
  uint16_t* h_sh;          // [T][I_s] bf16
  int shared_inter;
  int tokens, n_experts, hidden;
  float limit;
};
struct MidValuParams {
  const uint16_t* sh_dn;   // [H][I_s] bf16
  const uint16_t* h_sh;    // [T][I_s]
  uint16_t* y_sh;          // [T][H]
  int shared_inter, tokens, hidden;
};
bool decode_valu_supported(int tokens, int hidden, int shared_inter);
hipError_t launch_decode_front_valu(const FrontValuParams& f, hipStream_t stream);
hipError_t launch_decode_mid_valu(const RouteSmallParams& p, const MidValuParams& m, hipStream_t stream);
// Launch 2: the one-block routing beside the shared expert's down projection.
hipError_t launch_decode_mid(const RouteSmallParams& p, const GemvProblem& shared_down, int rows_cap,
                             hipStream_t stream);

// Routed down projection with the combine folded in, for T <= 8 tokens whose
// T * top_k rows of h fit in LDS: y[t] = y_shared[t] + sum_j w[t][j] o[t][j].
struct DownCombineParams {
  const uint8_t* hmx;          // [T*k] rows of h in two-term MXFP8 form (stride mx_row_bytes(inter)), position order
  const GemmTile* tiles;
  const int32_t* tile_count;
  const int32_t* sorted_slots;
  const float* topk_w;         // [T][k]
  const uint8_t* dn_q;
  const uint8_t* dn_s;
  const uint16_t* y_shared;    // [T][hidden] or NULL
  uint16_t* y;                 // [T][hidden]
  int tokens, top_k, n_experts, hidden, inter;
  int max_tiles;               // entries of tiles (<= 64)
};
constexpr int kDownCombineMaxTokens = 8;
constexpr int kDownCombineMaxInter = 2560;
size_t down_combine_lds_bytes(int tokens, int top_k, int inter);
hipError_t launch_down_combine(const DownCombineParams& p, hipStream_t stream);

// Routed projections for T <= 2 tokens on the vector ALUs, one wave per
// output column (expert_valu.hip).  gate/up: one block row per tile record
// of the one-block routing (tiles, tile_rows; empty records are skipped),
// h[pos] = SwiGLU.  down: every slot's h row against row n of its expert's
// W_dn, weighted and added to the shared expert's output: y directly.
struct GateUpValuParams {
  const uint16_t* x;          // [T][H] bf16
  const GemmTile* tiles;      // [max_tiles]
  const int32_t* tile_rows;   // [max_tiles][kTileRows]
  const uint8_t* gu_q;        // [E][2I][H/2] (MXFP8: [E][2I][H])
  const uint8_t* gu_s;        // [E][2I][H/32]
  uint16_t* h;                // [T*k][I] bf16, row = position
  int tokens, hidden, inter;
  float limit;
  bool fp8;                   // MXFP8 (E4M3) codes instead of MXFP4
  // routing in every wave (launch_route_gate_up_shared_gu): the router's
  // scores [2][T][E] instead of tiles/tile_rows; the first wave writes the
  // routing the later launches read (idx, w [T][k], slot_pos, sorted_slots [T*k])
  const float* scores;
  int n_experts, top_k;
  float route_scale;
  int32_t* idx;
  float* w;
  int32_t* slot_pos;
  int32_t* sorted_slots;
};
struct DownValuParams {
  const uint16_t* h;          // [T*k][I] bf16, row = position
  const int32_t* idx;         // [T][k]
  const float* topk_w;        // [T][k]
  const int32_t* slot_pos;    // [T*k]
  const uint8_t* dn_q;        // [E][H][I/2] (MXFP8: [E][H][I])
  const uint8_t* dn_s;        // [E][H][I/32]
  const uint16_t* y_shared;   // [T][H] or NULL
  uint16_t* y;                // [T][H]
  int tokens, top_k, hidden, inter;
  bool fp8;                   // MXFP8 (E4M3) codes instead of MXFP4
  // shared expert folded in (launch_down_combine_shared): row n of sh_dn
  // [H][I_s] bf16 against h_sh [T][I_s] is added to y[t][n] in fp32 (y_shared unused)
  const uint16_t* sh_dn;
  const uint16_t* h_sh;
  int shared_inter;
};
bool gate_up_valu_supported(int tokens, int hidden, int max_tiles, bool fp8 = false);
bool down_valu_supported(int tokens, int top_k, int inter, bool fp8 = false);
hipError_t launch_gate_up_valu(const GateUpValuParams& p, int max_tiles, hipStream_t stream);
hipError_t launch_down_combine_valu(const DownValuParams& p, hipStream_t stream);
// The streaming few-token layer (T <= 2), four launches:
//   1. router GEMV writing the scores (launch_router_gemv);
//   2. the routing block beside the shared gate/up;
//   3. routed gate/up beside the shared down projection;
//   4. routed down with the combine (launch_down_combine_valu).
hipError_t launch_decode_route_shared_gu(const FrontValuParams& f, const RouteSmallParams& p, hipStream_t stream);
bool gate_up_shared_down_supported(int tokens, int hidden, int max_tiles, int shared_inter, bool fp8 = false);
hipError_t launch_gate_up_shared_down(const GateUpValuParams& p, int max_tiles, const MidValuParams& m,
                                      hipStream_t stream);
// The three-launch streaming layer (T <= 2, T * k <= 64):
//   1. router GEMV writing the scores (launch_router_gemv / launch_router_norm_gemv);
//   2. routed gate/up, every wave routing for itself from the scores, beside
//      the shared expert's gate/up (f: x, sh_gu, h_sh, shared_inter, limit);
//   3. routed down with the combine and the shared expert's down projection
//      folded in (launch_down_combine_shared).
bool route_gate_up_shared_gu_supported(int tokens, int hidden, int n_experts, int top_k, int shared_inter, bool fp8);
hipError_t launch_route_gate_up_shared_gu(const GateUpValuParams& p, const FrontValuParams& f, hipStream_t stream);
// Without the pre-FFN norm: 1. router GEMV beside the shared gate/up
// (launch_decode_front_valu); 2. routed gate/up routing in every wave beside
// the shared down (this launcher); 3. routed down with the combine
// (launch_down_combine_valu).
hipError_t launch_route_gate_up_shared_down(const GateUpValuParams& p, const MidValuParams& m, hipStream_t stream);
bool down_combine_shared_supported(int tokens, int top_k, int inter, int shared_inter, bool fp8);
hipError_t launch_down_combine_shared(const DownValuParams& p, hipStream_t stream);

// Fused few-token routing: top-k of every token + permutation + tile table (T*k <= 1024).
hipError_t launch_route_permute_small(const float* part, int ksplit, const float* bias, int tokens, int n_experts,
                                      int top_k, float route_scale, int32_t* idx, float* w, float* gap,
                                      int32_t* offsets, int32_t* sorted_slots, int32_t* slot_pos, int bm,
                                      int max_tiles, GemmTile* tiles, int32_t* tile_count, hipStream_t stream);

// ---------------------------------------------------------------- two-term MXFP6 grouped GEMM (expert_mx6.hip)
// Activation rows in two-term MXFP6 records (mx6_device.h) times MXFP4
// weights on the block-scaled MFMA, tiles of up to mx6_tile_rows() rows of
// one expert.
struct Mx6Params {
  const GemmTile* tiles;       // [n_tiles] from the permutation, tile_count entries valid
  const int32_t* tile_count;
  const int32_t* gather;       // A record row of position p: gather[p] / gather_div, or p if NULL
  int gather_div;
  const uint8_t* A;            // [a_rows][mx6_row_bytes(K)]
  int64_t a_stride;
  int a_rows;
  int K;                       // multiple of 128
  const uint8_t* bq;           // [E][b_expert_rows][K/2] E2M1 codes ([..][K] E4M3 codes with w8)
  const uint8_t* bs;           // [E][b_expert_rows][K/32] E8M0 scales
  int w8;                      // MXFP8 weights (FP6 x FP8 at the FP8 rate)
  int64_t b_expert_rows;
  int b_row_second;            // SwiGLU: first row of the up half
  int N;                       // output columns (h columns for gate/up)
  uint16_t* C;                 // bf16 [.][ldc], row = position p
  int64_t ldc;
  uint8_t* Cmx;                // gate/up: h as two-term MXFP6 records instead of C (row stride ldcmx bytes)
  int64_t ldcmx;
  float limit;
};
// hidden and inter multiples of 128, at most 5120 (the scales of a block's weight rows fit its LDS)
bool mx6_supported(int hidden, int inter);
int mx6_tile_rows();
int64_t mx6_bytes(int64_t rows, int K);
// bf16 rows [rows][K] (row stride ld_src elements) -> records [rows][mx6_row_bytes(K)]
hipError_t launch_mx6_rows(const uint16_t* src, int64_t ld_src, int rows, int K, uint8_t* dst, hipStream_t stream);
hipError_t launch_expert_mx6(const Mx6Params& p, bool swiglu, int n_tiles, hipStream_t stream);

// ---------------------------------------------------------------- combine
hipError_t launch_combine(const uint16_t* y_slot, const int32_t* slot_pos, const float* w, const uint16_t* y_shared,
                          int tokens, int top_k, int hidden, uint16_t* y, hipStream_t stream);

}  // namespace moe
