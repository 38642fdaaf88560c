// Host-side launch interface between the C ABI (moe_ffn.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- router
struct RouterPlan {
  int mt;                // 16-token row tiles per block (1 or 4)
  int ksplit;            // number of K ranges, each a whole number of 128-wide chunks
  int chunks_per_split;  // 128-wide K chunks per range
};
RouterPlan router_plan(int64_t tokens, int n_experts, int hidden);

// partial logits [ksplit][T][E] fp32
hipError_t launch_router_logits(const RouterPlan& plan, const uint16_t* x, const float* router_w, float* part,
                                int tokens, int n_experts, int hidden, hipStream_t stream);
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
                          int32_t* offsets, int32_t* sorted_slots, int32_t* slot_pos, int bm, GemmTile* tiles,
                          int32_t* tile_count, hipStream_t stream);
// Tile table from expert offsets alone.
hipError_t launch_tile_table(const int32_t* offsets, int n_experts, int n_total, int bm, GemmTile* tiles,
                             int32_t* tile_count, hipStream_t stream);

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
  // B (weights), per expert: MXFP4 codes/scales or bf16, rows [.][K]
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
};
int expert_gemm_mt(int64_t n_rows, int n_groups);
hipError_t launch_expert_gemm(const GemmParams& p, bool swiglu, bool fp4, int mt, int64_t grid_tiles,
                              hipStream_t stream);

// ---------------------------------------------------------------- combine
hipError_t launch_combine(const uint16_t* y_slot, const int32_t* slot_pos, const float* w, const uint16_t* y_shared,
                          int tokens, int top_k, int hidden, uint16_t* y, hipStream_t stream);

}  // namespace moe
