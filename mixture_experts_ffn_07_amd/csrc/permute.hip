// Permutation of the T*k (token, slot) pairs into expert-contiguous order:
// a stable counting sort of the flat slot f = t*k + j by its expert.
//
// Deterministic and stable without a global sort:
//   count   -- per chunk of 1024 flat slots (16 waves of 64), each slot's rank
//              among the earlier slots of the same expert in its chunk.
//              Inside a wave, lanes with equal expert ids are matched by one
//              ballot per bit of the id (log2 E ballots), then a popcount of
//              the lower lanes gives the rank; across waves of the chunk the
//              per-wave counts are added through LDS.  Per-chunk expert
//              counts go to global memory.
//   scan    -- one block: per expert, exclusive prefix over chunks; block-wide
//              exclusive prefix over experts gives the expert offsets; also the
//              tile table of the grouped GEMM.
//   scatter -- position = expert offset + chunk base + rank.
// When T*k fits one chunk all three run in one block of one launch.
#include "moe_device.h"
#include "moe_internal.h"
#include "permute_device.h"

namespace moe {

__global__ __launch_bounds__(1024) void permute_count_kernel(const int32_t* __restrict__ idx, int n, int n_experts,
                                                             int32_t* __restrict__ rank,
                                                             int32_t* __restrict__ chunk_counts) {
  extern __shared__ uint16_t cnt[];
  int e;
  const int r = chunk_rank(idx, n, n_experts, blockIdx.x, cnt, &e);
  const int f = blockIdx.x * kPermuteChunk + threadIdx.x;
  if (f < n) rank[f] = r;
  for (int ee = threadIdx.x; ee < n_experts; ee += blockDim.x) {
    int tot = 0;
    for (int w = 0; w < 16; ++w) tot += cnt[w * n_experts + ee];
    chunk_counts[(size_t)blockIdx.x * n_experts + ee] = tot;
  }
}

__global__ __launch_bounds__(1024) void permute_scan_kernel(const int32_t* __restrict__ chunk_counts, int nchunks,
                                                            int n_experts, int n, int32_t* __restrict__ chunk_base,
                                                            int32_t* __restrict__ offsets, int bm, int max_tiles,
                                                            GemmTile* __restrict__ tiles,
                                                            int32_t* __restrict__ tile_count) {
  __shared__ int scratch[16];
  const int e = threadIdx.x;
  int total = 0;
  if (e < n_experts)
    for (int c = 0; c < nchunks; ++c) total += chunk_counts[(size_t)c * n_experts + e];
  const int excl = block_exclusive_scan(e < n_experts ? total : 0, scratch, nullptr);
  if (e < n_experts) {
    offsets[e] = excl;
    int run = excl;
    for (int c = 0; c < nchunks; ++c) {
      chunk_base[(size_t)c * n_experts + e] = run;
      run += chunk_counts[(size_t)c * n_experts + e];
    }
  }
  if (e == 0) offsets[n_experts] = n;
  if (tiles) write_tile_table(total, excl, n_experts, bm, n, max_tiles, tiles, tile_count, scratch);
}

__global__ __launch_bounds__(256) void permute_scatter_kernel(const int32_t* __restrict__ idx, int n, int n_experts,
                                                              const int32_t* __restrict__ rank,
                                                              const int32_t* __restrict__ chunk_base,
                                                              int32_t* __restrict__ sorted_slots,
                                                              int32_t* __restrict__ slot_pos) {
  const int f = blockIdx.x * 256 + threadIdx.x;
  if (f >= n) return;
  const int e = clamp_expert(idx[f], n_experts);
  const int pos = chunk_base[(size_t)(f / kPermuteChunk) * n_experts + e] + rank[f];
  sorted_slots[pos] = f;
  slot_pos[f] = pos;
}

// n <= 1024: count, scan, scatter and tile table in one block.
__global__ __launch_bounds__(1024) void permute_single_kernel(const int32_t* __restrict__ idx, int n, int n_experts,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ sorted_slots,
                                                              int32_t* __restrict__ slot_pos, int bm, int max_tiles,
                                                              GemmTile* __restrict__ tiles,
                                                              int32_t* __restrict__ tile_count) {
  extern __shared__ uint16_t cnt[];  // [16][E] uint16, then [E] int32 offsets
  permute_block(idx, n, n_experts, cnt, offsets, sorted_slots, slot_pos, bm, max_tiles, tiles, tile_count);
}

__global__ __launch_bounds__(1024) void tile_table_kernel(const int32_t* __restrict__ offsets, int n_experts, int bm,
                                                          int n_total, int max_tiles, GemmTile* __restrict__ tiles,
                                                          int32_t* __restrict__ tile_count) {
  __shared__ int scratch[16];
  const int e = threadIdx.x;
  int count = 0, off = 0;
  if (e < n_experts) {
    off = offsets[e];
    count = offsets[e + 1] - off;
  }
  write_tile_table(count, off, n_experts, bm, n_total, max_tiles, tiles, tile_count, scratch);
}

hipError_t launch_permute(const int32_t* idx, int n, int n_experts, const PermuteScratch& s, int32_t* offsets,
                          int32_t* sorted_slots, int32_t* slot_pos, int bm, int max_tiles, GemmTile* tiles,
                          int32_t* tile_count, hipStream_t stream) {
  const size_t cnt_bytes = (size_t)16 * n_experts * sizeof(uint16_t);
  if (n <= kPermuteChunk) {
    const size_t shm = permute_block_lds_bytes(n_experts);
    hipLaunchKernelGGL(permute_single_kernel, dim3(1), dim3(1024), shm, stream, idx, n, n_experts, offsets,
                       sorted_slots, slot_pos, bm, max_tiles, tiles, tile_count);
    return hipGetLastError();
  }
  const int nchunks = permute_chunks(n);
  hipLaunchKernelGGL(permute_count_kernel, dim3(nchunks), dim3(1024), cnt_bytes, stream, idx, n, n_experts, s.rank,
                     s.chunk_counts);
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(1024), 0, stream, s.chunk_counts, nchunks, n_experts, n,
                     s.chunk_base, offsets, bm, max_tiles, tiles, tile_count);
  hipLaunchKernelGGL(permute_scatter_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, idx, n, n_experts, s.rank,
                     s.chunk_base, sorted_slots, slot_pos);
  return hipGetLastError();
}

hipError_t launch_tile_table(const int32_t* offsets, int n_experts, int n_total, int bm, int max_tiles,
                             GemmTile* tiles, int32_t* tile_count, hipStream_t stream) {
  hipLaunchKernelGGL(tile_table_kernel, dim3(1), dim3(1024), 0, stream, offsets, n_experts, bm, n_total, max_tiles,
                     tiles, tile_count);
  return hipGetLastError();
}

}  // namespace moe
