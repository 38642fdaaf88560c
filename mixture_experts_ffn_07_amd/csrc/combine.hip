// Weighted combine back to token order:
//   y[t] = y_shared[t] + sum_{j<k} w[t,j] * y_slot[slot_pos[t*k + j]]
// fp32 accumulation starting from the shared expert's output, the routed terms
// added in slot order j = 0..k-1, one rounding to bf16.  (The layer's output
// is the shared expert plus the weighted routed experts: one always-on shared
// expert, n_shared_experts = 1 in DeepseekV41Config.)
#include "moe_device.h"
#include "moe_internal.h"

namespace moe {

// Block: 256 threads x 8 columns = 2048 columns of one token.
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y_slot,
                                                      const int32_t* __restrict__ slot_pos,
                                                      const float* __restrict__ w,
                                                      const uint16_t* __restrict__ y_shared, int tokens, int top_k,
                                                      int hidden, uint16_t* __restrict__ y) {
  const int t = blockIdx.x;
  const int h = (blockIdx.y * 256 + threadIdx.x) * 8;
  if (t >= tokens || h >= hidden) return;
  float acc[8];
  if (y_shared) {
    const uint4 v = *reinterpret_cast<const uint4*>(y_shared + (int64_t)t * hidden + h);
    const uint32_t vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = bf16_to_f32((uint16_t)(vv[i] & 0xffffu));
      acc[2 * i + 1] = bf16_to_f32((uint16_t)(vv[i] >> 16));
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  }
  // Positions and weights of all k slots first, then all k rows, so each
  // group of loads issues together (k <= 16).
  const int n = tokens * top_k;
  int pos[16];
  float wj[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int64_t f = min((int64_t)t * top_k + j, (int64_t)n - 1);
    pos[j] = min(max(slot_pos[f], 0), n - 1);  // stays in y_slot for any slot_pos
    wj[j] = j < top_k ? w[f] : 0.f;
  }
  uint4 v[16];
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (j < top_k) v[j] = *reinterpret_cast<const uint4*>(y_slot + (int64_t)pos[j] * hidden + h);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    if (j < top_k) {
      const uint32_t vv[4] = {v[j].x, v[j].y, v[j].z, v[j].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] = fmaf(wj[j], bf16_to_f32((uint16_t)(vv[i] & 0xffffu)), acc[2 * i]);
        acc[2 * i + 1] = fmaf(wj[j], bf16_to_f32((uint16_t)(vv[i] >> 16)), acc[2 * i + 1]);
      }
    }
  }
  uint4 o;
  o.x = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
  o.y = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
  o.z = (uint32_t)f32_to_bf16(acc[4]) | ((uint32_t)f32_to_bf16(acc[5]) << 16);
  o.w = (uint32_t)f32_to_bf16(acc[6]) | ((uint32_t)f32_to_bf16(acc[7]) << 16);
  *reinterpret_cast<uint4*>(y + (int64_t)t * hidden + h) = o;
}

hipError_t launch_combine(const uint16_t* y_slot, const int32_t* slot_pos, const float* w, const uint16_t* y_shared,
                          int tokens, int top_k, int hidden, uint16_t* y, hipStream_t stream) {
  dim3 grid(tokens, (hidden + 2047) / 2048);
  hipLaunchKernelGGL(combine_kernel, grid, dim3(256), 0, stream, y_slot, slot_pos, w, y_shared, tokens, top_k, hidden,
                     y);
  return hipGetLastError();
}

}  // namespace moe
