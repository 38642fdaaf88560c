// Pre-FFN RMSNorm of whole rows (the layer's optional first step; formula and
// precision in norm_device.h).  One wave per row, rows grid-strided over the
// launch.  Rows of up to 64 * 8 * NV elements are held in registers, so x is
// read from HBM once and x_norm written once: 4 bytes of traffic per element,
// the HBM bound of this kernel.  Longer rows take a second pass over x for
// the normalisation (the row is then re-read from the caches).
#include "moe_internal.h"
#include "norm_device.h"

namespace moe {
namespace {

constexpr int kNormBlock = 256;  // four rows per block

template <int NV>  // 16-byte vectors per lane held in registers
__global__ __launch_bounds__(kNormBlock) void rmsnorm_rows_kernel(const uint16_t* x, const uint16_t* __restrict__ gamma,
                                                                 uint16_t* x_norm, int rows, int hidden, double eps) {
  const int lane = threadIdx.x & 63;
  const int nwaves = gridDim.x * (kNormBlock / 64);
  const int nv = hidden / 8;  // 16-byte vectors per row
  const u32x4_t* g4 = reinterpret_cast<const u32x4_t*>(gamma);
  for (int row = blockIdx.x * (kNormBlock / 64) + (threadIdx.x >> 6); row < rows; row += nwaves) {
    const u32x4_t* xr = reinterpret_cast<const u32x4_t*>(x + (size_t)row * hidden);
    u32x4_t* yr = reinterpret_cast<u32x4_t*>(x_norm + (size_t)row * hidden);
    double acc = 0.0;
    if (nv <= 64 * NV) {  // wave-uniform: the whole row in registers
      u32x4_t v[NV];
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int c = 64 * i + lane;
        v[i] = c < nv ? xr[c] : u32x4_t{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) acc = add_squares4(v[i][2], v[i][3], add_squares4(v[i][0], v[i][1], acc));
      const double r = rms_recip(wave_sum_f64(acc), hidden, eps);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int c = 64 * i + lane;
        if (c < nv) {
          const u32x4_t g = g4[c];
          yr[c] = u32x4_t{norm_pair(v[i][0], g[0], r), norm_pair(v[i][1], g[1], r), norm_pair(v[i][2], g[2], r),
                          norm_pair(v[i][3], g[3], r)};
        }
      }
    } else {
      for (int c = lane; c < nv; c += 64) {
        const u32x4_t a = xr[c];
        acc = add_squares4(a[2], a[3], add_squares4(a[0], a[1], acc));
      }
      const double r = rms_recip(wave_sum_f64(acc), hidden, eps);
      for (int c = lane; c < nv; c += 64) {
        const u32x4_t a = xr[c];
        const u32x4_t g = g4[c];
        yr[c] = u32x4_t{norm_pair(a[0], g[0], r), norm_pair(a[1], g[1], r), norm_pair(a[2], g[2], r),
                        norm_pair(a[3], g[3], r)};
      }
    }
  }
}

}  // namespace

hipError_t launch_rmsnorm_rows(const uint16_t* x, const uint16_t* gamma, uint16_t* x_norm, int rows, int hidden,
                               double eps, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  const int per_block = kNormBlock / 64;
  int blocks = (rows + per_block - 1) / per_block;
  if (blocks > 4096) blocks = 4096;
  const int nv = hidden / 8;
  auto kern = nv <= 64 * 4 ? rmsnorm_rows_kernel<4> : nv <= 64 * 8 ? rmsnorm_rows_kernel<8> : rmsnorm_rows_kernel<16>;
  hipLaunchKernelGGL(kern, dim3(blocks), dim3(kNormBlock), 0, stream, x, gamma, x_norm, rows, hidden, eps);
  return hipGetLastError();
}

}  // namespace moe
