// Device functions of the stable counting-sort permutation, shared by the
// permutation kernels and the fused decode routing kernel.
#pragma once

#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

__device__ __forceinline__ int clamp_expert(int e, int n_experts) {
  return e < 0 ? 0 : (e >= n_experts ? n_experts - 1 : e);
}

__device__ __forceinline__ int bits_for(int n_experts) {
  int b = 0;
  while ((1 << b) < n_experts) ++b;
  return b;
}

// Within-wave stable rank of this lane's expert id and the number of lanes
// sharing it; lanes with ok == false take part in no match.
__device__ __forceinline__ void wave_match_rank(int e, bool ok, int ebits, int* rank, int* count) {
  const int lane = threadIdx.x & 63;
  uint64_t mask = __ballot(ok);
  for (int b = 0; b < ebits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t m = __ballot(ok && bit);
    mask &= bit ? m : ~m;
  }
  const uint64_t lower = lane == 0 ? 0ull : (~0ull >> (64 - lane));
  *rank = __popcll(mask & lower);
  *count = __popcll(mask);
}

// Chunk-local ranks.  cnt: shared [16][E] uint16.  Returns this thread's rank
// within the chunk (valid only when f < n).
__device__ __forceinline__ int chunk_rank(const int32_t* __restrict__ idx, int n, int n_experts, int chunk,
                                          uint16_t* cnt, int* e_out) {
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int i = tid; i < 16 * n_experts; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  const int f = chunk * kPermuteChunk + tid;
  const bool ok = f < n;
  const int e = ok ? clamp_expert(idx[f], n_experts) : 0;
  int rk, c;
  wave_match_rank(e, ok, bits_for(n_experts), &rk, &c);
  if (ok && rk == 0) cnt[wave * n_experts + e] = (uint16_t)c;
  __syncthreads();
  int before = 0;
  if (ok)
    for (int w = 0; w < wave; ++w) before += cnt[w * n_experts + e];
  *e_out = e;
  return before + rk;
}

// Tile table of a grouped GEMM: expert e's run [off_e, off_e + count_e) cut
// into tiles of bm rows.  Called by every thread of one block with
// this thread's (count, offset) for expert tid (count 0 for tid >= E).
// Offsets and counts are clamped into [0, n_total] and at most max_tiles
// tiles are written, so an inconsistent caller-supplied offset table cannot
// lead to an access outside the tile table or the row range.
__device__ __forceinline__ void write_tile_table(int count, int offset, int n_experts, int bm, int n_total,
                                                 int max_tiles, GemmTile* __restrict__ tiles,
                                                 int32_t* __restrict__ tile_count, int* scan_scratch) {
  const int e = threadIdx.x;
  offset = min(max(offset, 0), n_total);
  count = min(max(count, 0), n_total - offset);
  const int nt = (e < n_experts) ? (count + bm - 1) / bm : 0;
  int total;
  const int start = block_exclusive_scan(nt, scan_scratch, &total);
  for (int i = 0; i < nt && start + i < max_tiles; ++i) {
    GemmTile t;
    t.e = e;
    t.m_begin = offset + i * bm;
    t.m_end = min(offset + (i + 1) * bm, offset + count);
    t.pad = 0;
    tiles[start + i] = t;
  }
  if (threadIdx.x == 0) *tile_count = min(total, max_tiles);
}

// Whole permutation of n <= 1024 flat slots by one block of 1024 threads:
// chunk-local ranks, expert offsets by a block scan, scatter, tile table.
// `cnt` is dynamic shared memory of permute_block_lds_bytes(n_experts) bytes;
// idx may point to global or shared memory.
__host__ __device__ inline size_t permute_block_lds_bytes(int n_experts) {
  return (((size_t)16 * n_experts * sizeof(uint16_t) + 3) & ~(size_t)3) + (size_t)n_experts * sizeof(int32_t) + 4;
}

__device__ __forceinline__ void permute_block(const int32_t* idx, int n, int n_experts, uint16_t* cnt,
                                              int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_slots,
                                              int32_t* __restrict__ slot_pos, int bm, int max_tiles,
                                              GemmTile* __restrict__ tiles, int32_t* __restrict__ tile_count) {
  __shared__ int scratch[16];
  int32_t* off_sh = reinterpret_cast<int32_t*>(cnt + ((16 * n_experts + 1) & ~1));
  int e;
  const int r = chunk_rank(idx, n, n_experts, 0, cnt, &e);
  const int ee = threadIdx.x;
  int total = 0;
  if (ee < n_experts)
    for (int w = 0; w < 16; ++w) total += cnt[w * n_experts + ee];
  const int excl = block_exclusive_scan(ee < n_experts ? total : 0, scratch, nullptr);
  if (ee < n_experts) {
    offsets[ee] = excl;
    off_sh[ee] = excl;
  }
  if (ee == 0) offsets[n_experts] = n;
  __syncthreads();
  const int f = threadIdx.x;
  if (f < n) {
    const int pos = off_sh[e] + r;
    sorted_slots[pos] = f;
    slot_pos[f] = pos;
  }
  if (tiles) write_tile_table(total, excl, n_experts, bm, n, max_tiles, tiles, tile_count, scratch);
}

}  // namespace moe
