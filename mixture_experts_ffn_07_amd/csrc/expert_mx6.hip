// Routed grouped GEMMs for many tokens on gfx950's block-scaled matrix
// instruction: two-term MXFP6 activations (mx6_device.h) times the experts'
// MXFP4 weights as stored (E2M1 codes, E8M0 scale per 32 along K: Strata
// DEEPSEEK41 notes, opening paragraph; the MAX API's float4_e2m1fnx2),
// v_mfma_scale_f32_16x16x128_f8f6f4 with fp32 accumulation, the clamped
// SwiGLU (swiglu_limit, DeepseekV41Config) in the gate/up epilogue.  MXFP8
// weights (E4M3 codes with the same E8M0 scales: the MAX API's
// float8_e4m3fn) take the same kernel as the instruction's 8-bit operand,
// FP6 x FP8 at the FP8 rate.
//
// FP6 x FP4 runs at the FP4 rate on gfx950 (measured 7.9 PFLOP/s on a
// register-only probe, against 4.4 for FP8 x FP4 and 2.3 for bf16), so the
// two terms cost two FP4-rate instructions per 16 x 16 x 128 step: 1.7x the
// bf16 rate on exactly dequantised weights, with the weights never expanded.
//
// Block: 4 waves (one per SIMD), a tile of up to 96 rows of one expert
// against 512 weight rows (gate/up: 256 columns of h, the gate and up rows
// of each; down: 512 output columns).  Wave w owns 128 of the weight rows as
// 8 MFMA column tiles and every row tile, so its accumulators take up to
// 6 x 8 x 4 registers (the wave runs alone on its SIMD, 512 registers; 128
// rows would need all 256 accumulation registers and spill the operands).
//   * Weights go from memory straight to registers (each weight byte is read
//     by one wave only), two chunks per burst, two to three chunks ahead of
//     the MFMAs.
//   * The tile's activation records go global -> registers -> LDS (two
//     stages), four chunks ahead, and every wave reads its MFMA operands from
//     LDS: the record layout is the operand layout, so a row tile costs five
//     LDS reads per lane and chunk (no bank conflicts on the 16-byte reads:
//     the 208-byte row stride puts 8 consecutive rows on 8 different bank
//     quads).
//   * The weight scales of the block's rows go to LDS whole in the prologue.
// Chunk loads are ordinary buffer loads whose waits the compiler places.
// The per-lane offset of a row past the end (weight rows beyond N,
// activation pieces beyond the tile) is kOob, which the buffer range check
// turns into a zero; the chunk enters as the scalar offset, which that check
// does not cover, so chunk indices are always clamped into the matrix.
#include "moe_device.h"
#include "moe_internal.h"
#include "mx_device.h"
#include "mx6_device.h"

namespace moe {

namespace {

typedef __bf16 bf16x32_t __attribute__((__vector_size__(32 * sizeof(__bf16))));
typedef float f32x16_t __attribute__((__vector_size__(16 * sizeof(float))));
typedef uint32_t u32x2_t __attribute__((__vector_size__(2 * sizeof(uint32_t))));
typedef uint32_t u32x16_t __attribute__((__vector_size__(16 * sizeof(uint32_t))));

// E8M0 byte of 2^(floor(log2 amax) - 2), 127 for amax == 0, held in [0, 254].
__device__ __forceinline__ int mx6_scale_code(float amax) {
  if (!(amax > 0.f)) return 127;
  const int ex = (int)((__float_as_uint(amax) >> 23) & 0xff);  // biased floor(log2 amax) for normal amax
  return min(max(ex - 2, 0), 254);
}

// ============================================================== bf16 rows -> two-term MXFP6 records
// A unit is one row and 128-wide chunk: 256 bytes in, one 208-byte record
// out.  With contiguous rows (ld_src = K, ld_dst = the record row) the units
// of a block are one contiguous input range and one contiguous output range,
// so both go through LDS as whole 16-byte pieces per lane (every load and
// store instruction covers 4 KB); each thread converts one unit from LDS
// (unit stride 272 bytes: the 16-byte reads of 8 consecutive units fall on
// 8 different bank quads).
constexpr int kMx6ConvUnits = 256;                 // units per block, one per thread
constexpr int kMx6ConvIn = 272;                    // LDS bytes per staged input unit

// one unit: 16 input pieces (bf16 x 8 each) -> 52 record dwords
__device__ __forceinline__ void mx6_convert_unit(const u32x4_t (&v)[16], uint32_t (&rec)[52]) {
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    float x[32];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        x[8 * q + 2 * w] = __uint_as_float(v[4 * g + q][w] << 16);
        x[8 * q + 2 * w + 1] = __uint_as_float(v[4 * g + q][w] & 0xffff0000u);
      }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
    const int c1 = mx6_scale_code(amax);
    const float s1 = __uint_as_float((uint32_t)c1 << 23);
    u32x16_t xw;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int w = 0; w < 4; ++w) xw[4 * q + w] = v[4 * g + q][w];
    const bf16x32_t xb = __builtin_bit_cast(bf16x32_t, xw);  // value 2 w in the low half of dword w
    // converts divide by the scale, round to nearest even, saturate at +-7.5;
    // the bf16 form packs value i into bits [6 i, 6 i + 6)
    const auto hi = __builtin_amdgcn_cvt_scalef32_pk32_fp6_bf16(xb, s1);
    const auto hv = __builtin_amdgcn_cvt_scalef32_pk32_f32_fp6(hi, s1);
    f32x16_t ev, od;  // the f32 form interleaves its two halves: value 2 i from ev, 2 i + 1 from od
    float amax_r = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      ev[i] = x[2 * i] - hv[2 * i];
      od[i] = x[2 * i + 1] - hv[2 * i + 1];
      amax_r = fmaxf(amax_r, fmaxf(fabsf(ev[i]), fabsf(od[i])));
    }
    const int c2 = mx6_scale_code(amax_r);
    const auto lo = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(ev, od, __uint_as_float((uint32_t)c2 << 23));
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      rec[4 * g + d] = (uint32_t)hi[d];
      rec[24 + 4 * g + d] = (uint32_t)lo[d];
    }
    rec[16 + 2 * g] = (uint32_t)hi[4];
    rec[17 + 2 * g] = (uint32_t)hi[5];
    rec[40 + 2 * g] = (uint32_t)lo[4];
    rec[41 + 2 * g] = (uint32_t)lo[5];
    rec[48 + g] = (uint32_t)c1 | ((uint32_t)c2 << 8);
  }
}

// contiguous rows: block b converts units [256 b, 256 b + 256) of `units`
__global__ __launch_bounds__(256) void mx6_rows_kernel(const uint16_t* __restrict__ src, int64_t units,
                                                       uint8_t* __restrict__ dst) {
  __shared__ __attribute__((aligned(16))) uint8_t buf[kMx6ConvUnits * kMx6ConvIn];
  const int t = (int)threadIdx.x;
  const int64_t u0 = (int64_t)blockIdx.x * kMx6ConvUnits;
  const int nu = (int)min((int64_t)kMx6ConvUnits, units - u0);
  const u32x4_t* in = reinterpret_cast<const u32x4_t*>(src) + u0 * 16;
  // 16 pieces per unit: piece p -> unit p / 16, slot p % 16
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int p = t + 256 * i;
    if (p < 16 * nu)
      *reinterpret_cast<u32x4_t*>(buf + (p >> 4) * kMx6ConvIn + 16 * (p & 15)) = __builtin_nontemporal_load(in + p);
  }
  __syncthreads();
  uint32_t rec[52];
  if (t < nu) {
    u32x4_t v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = *reinterpret_cast<const u32x4_t*>(buf + t * kMx6ConvIn + 16 * i);
    mx6_convert_unit(v, rec);
  }
  __syncthreads();
  if (t < nu) {
#pragma unroll
    for (int i = 0; i < 13; ++i)
      *reinterpret_cast<u32x4_t*>(buf + t * kMx6Rec + 16 * i) =
          u32x4_t{rec[4 * i], rec[4 * i + 1], rec[4 * i + 2], rec[4 * i + 3]};
  }
  __syncthreads();
  u32x4_t* out = reinterpret_cast<u32x4_t*>(dst + u0 * kMx6Rec);
#pragma unroll
  for (int i = 0; i < 13; ++i) {
    const int p = t + 256 * i;
    if (p < 13 * nu) out[p] = *reinterpret_cast<const u32x4_t*>(buf + 16 * p);
  }
}

// strided rows (ld_src != K or ld_dst != the record row): one thread per
// unit, reading and writing directly
__global__ __launch_bounds__(256) void mx6_rows_strided_kernel(const uint16_t* __restrict__ src, int64_t ld_src,
                                                               int rows, int K, uint8_t* __restrict__ dst,
                                                               int64_t ld_dst) {
  const int chunks = K / 128;
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (t >= (int64_t)rows * chunks) return;
  const int r = (int)(t / chunks), c = (int)(t % chunks);
  const u32x4_t* s = reinterpret_cast<const u32x4_t*>(src + (int64_t)r * ld_src + (int64_t)c * 128);
  u32x4_t v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) v[i] = __builtin_nontemporal_load(s + i);
  uint32_t rec[52];
  mx6_convert_unit(v, rec);
  u32x4_t* d = reinterpret_cast<u32x4_t*>(dst + (int64_t)r * ld_dst + (int64_t)c * kMx6Rec);
#pragma unroll
  for (int i = 0; i < 13; ++i) d[i] = u32x4_t{rec[4 * i], rec[4 * i + 1], rec[4 * i + 2], rec[4 * i + 3]};
}

// ============================================================== grouped GEMM
// Global-to-LDS load of 16 bytes per lane: lane l's bytes land at LDS byte
// address lds + 16 l.  Written in asm so that the compiler does not treat
// the LDS it writes as possibly read by every later LDS load (it would then
// wait for all loads in flight before each one); the kernel waits for these
// loads itself.  M0 carries the LDS address as an input operand ("{m0}"),
// so the compiler writes M0 itself; the asm opens with the one wait state
// gfx950 needs between an SALU write of M0 and the load.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p);
}
__device__ __forceinline__ void load_lds16(const void* g, uint32_t lds) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(lds) : "memory");
}

constexpr int kMx6Rows = kMx6TileRows;             // rows per tile
// bytes per LDS stage: the tile's records, rounded up to whole rounds of 256
// 16-byte pieces (every thread writes the same number of pieces, the ones
// past the records to slots nothing reads, so the writes need no branch)
constexpr int kMx6Stage = (kMx6Rows * kMx6Rec + 4095) / 4096 * 4096;

__device__ __forceinline__ f32x4_t mfma_f6f4(const i32x8_t& a, const u32x4_t& b, int sa_word, int sb, f32x4_t c,
                                             int term) {
  const i32x8_t bw = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  // A: FP6 E2M3 (format 2), B: FP4 E2M1 (format 4); the A scale byte is byte `term` of sa_word
  return term == 0 ? __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bw, c, 2, 4, 0, sa_word, 0, sb)
                   : __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bw, c, 2, 4, 1, sa_word, 0, sb);
}

// A: FP6 E2M3 (format 2), B: FP8 E4M3 (format 0), 32 codes per lane in the
// instruction's 8-bit operand layout (b0: K offsets [16 g, 16 g + 16) of the
// chunk, b1: [64 + 16 g, 80 + 16 g)); runs at the FP8 rate.
__device__ __forceinline__ f32x4_t mfma_f6f8(const i32x8_t& a, const u32x4_t& b0, const u32x4_t& b1, int sa_word,
                                             int sb, f32x4_t c, int term) {
  const i32x8_t bw = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3], (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  return term == 0 ? __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bw, c, 2, 0, 0, sa_word, 0, sb)
                   : __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bw, c, 2, 0, 1, sa_word, 0, sb);
}

// The block's weight scale bytes (K / 32 per weight row) go to LDS whole,
// once, in the block's prologue: the weight rows of a block are one or two
// runs of consecutive matrix rows, so their scales are one or two contiguous
// byte ranges, read as 16-byte pieces.  (Per-lane byte loads touched a cache
// line per row and chunk and measured 35% of the kernel's time; groups of a
// few chunks per row re-fetched each scale line once per group, because the
// weight stream evicts it from L2 in between.)
// W8 (MXFP8 weights, 128 code bytes per row and chunk): a wave owns half the
// weight rows, so its weight registers and the block's activation bytes per
// weight byte stay those of the MXFP4 form, and its MFMAs per chunk (at the
// FP8 rate) take the same time.
template <bool W8>
struct Mx6Shape {
  static constexpr int kWaveTiles = W8 ? 4 : 8;         // MFMA column tiles (16 weight rows) per wave
  static constexpr int kWaveRows = 16 * kWaveTiles;     // weight rows per wave
  static constexpr int kBlockRows = 4 * kWaveRows;      // weight rows per block
  static constexpr int kRowBytes(int K) { return W8 ? K : K / 2; }  // code bytes per weight row
};
constexpr int kMx6MaxK = 5120;                              // scales of a block's rows fit kMx6SBytes
constexpr int kMx6SBytes = Mx6Shape<false>::kBlockRows * (kMx6MaxK / 32);  // LDS bytes of the block's scales
template <bool W8>
constexpr int kMx6SPieces = Mx6Shape<W8>::kBlockRows * (kMx6MaxK / 32) / 16 / 256;  // scale pieces per thread
constexpr int kMx6ABufs = 4;                                // activation register buffers (chunks in flight)
constexpr int kMx6Unroll = 4;                               // steps per loop iteration

// Gate/up epilogue writing h as two-term MXFP6 records (the down
// projection's A operand) instead of bf16 rows: the block's 256 h columns
// (128 with MXFP8 weights) are two (one) 128-wide chunks of every row.  The
// bf16 values go to LDS as units of one row and chunk (stride kMx6ConvIn),
// each thread converts one unit exactly as mx6_rows_kernel converts bf16
// rows, and the records leave through LDS as whole 16-byte pieces (a row's
// records are adjacent in memory).  The LDS of the main loop is free: its
// last step ended at a barrier after every read.
template <int MT, bool W8>
__device__ __forceinline__ void mx6_epilogue_records(const Mx6Params& p,
                                                     const f32x4_t (&acc)[MT][Mx6Shape<W8>::kWaveTiles],
                                                     uint8_t* stage, uint8_t* sall, int m_begin, int rows, int n0) {
  using S = Mx6Shape<W8>;
  constexpr int JW = S::kWaveTiles;
  constexpr int kCh = S::kBlockRows / 2 / 128;  // 128-wide h chunks per block row: 2 (MXFP4), 1 (MXFP8)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  static_assert(kCh * kMx6Rows * kMx6ConvIn <= kMx6SBytes && kCh * kMx6Rows * kMx6Rec <= 2 * kMx6Stage,
                "the epilogue's units fit the main loop's LDS");
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * m + 4 * g + i;  // rows past the tile are converted but never stored
#pragma unroll
      for (int j = 0; j < JW / 2; ++j) {
        const int c = (S::kWaveRows / 2) * wave + 16 * j + n;  // block column, 0 .. 128 kCh - 1
        *reinterpret_cast<uint16_t*>(sall + (kCh * r + (c >> 7)) * kMx6ConvIn + 2 * (c & 127)) =
            f32_to_bf16(clamped_swiglu(acc[m][j][i], acc[m][j + JW / 2][i], p.limit));
      }
    }
  __syncthreads();
  const int t = (int)threadIdx.x;
  if (t < kCh * 16 * MT) {
    u32x4_t v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = *reinterpret_cast<const u32x4_t*>(sall + t * kMx6ConvIn + 16 * i);
    uint32_t rec[52];
    mx6_convert_unit(v, rec);
#pragma unroll
    for (int i = 0; i < 13; ++i)
      *reinterpret_cast<u32x4_t*>(stage + t * kMx6Rec + 16 * i) =
          u32x4_t{rec[4 * i], rec[4 * i + 1], rec[4 * i + 2], rec[4 * i + 3]};
  }
  __syncthreads();
  // row r's kCh records: pieces [13 kCh r, 13 kCh (r + 1)) of the stage, to
  // Cmx + row * ldcmx + (n0 / 128) * kMx6Rec; a chunk at or past N is not stored
  constexpr int kRowPieces = kCh * kMx6Rec / 16;
  for (int q = t; q < rows * kRowPieces; q += 256) {
    const int r = q / kRowPieces, k = q - r * kRowPieces;
    if (n0 + 128 * (k / (kMx6Rec / 16)) >= p.N) continue;
    *reinterpret_cast<u32x4_t*>(p.Cmx + (int64_t)(m_begin + r) * p.ldcmx + (int64_t)(n0 / 128) * kMx6Rec + 16 * k) =
        *reinterpret_cast<const u32x4_t*>(stage + 16 * q);
  }
}

template <bool SWIGLU, int MT, bool W8>
__device__ __forceinline__ void mx6_tile(const Mx6Params& p, uint8_t* stage, uint8_t* sall, int e, int m_begin,
                                         int rows, int n0) {
  using S = Mx6Shape<W8>;
  constexpr int JW = S::kWaveTiles;
  constexpr int kMx6WaveRows = S::kWaveRows, kMx6BlockRows = S::kBlockRows;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15, g = lane >> 4;
  const int K = p.K, nchunks = K / 128;
  constexpr int kRowsRun = 16 * MT;
  constexpr int kPieces = kRowsRun * 13;                    // 16-byte pieces of the tile per chunk
  constexpr int kPerThread = (kPieces + 255) / 256;

  // weight rows of this block (expert-relative): SwiGLU, two runs of
  // kMx6BlockRows / 2 rows (gate rows n0.., up rows b_row_second + n0..);
  // otherwise one run of kMx6BlockRows rows from n0
  const int64_t qbytes = p.b_expert_rows * S::kRowBytes(K), sbytes = p.b_expert_rows * (K / 32);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.bq + (int64_t)e * qbytes, (uint32_t)qbytes);
  // activation pieces this thread stages: piece q = tid + 256 i of the
  // stage (row q / 13, part q % 13); LDS byte 16 q.  Rows past the tile
  // repeat its last row.
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(p.A, (uint32_t)((int64_t)p.a_rows * p.a_stride));
  // (the gather reads go out together, with no branch between them)
  int src[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) src[i] = m_begin + min(((int)threadIdx.x + 256 * i) / 13, rows - 1);
  if (p.gather) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) src[i] = p.gather[src[i]];
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) src[i] /= p.gather_div;
  }
  uint32_t a_off[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int q = (int)threadIdx.x + 256 * i;
    const int r = min(max(src[i], 0), p.a_rows - 1);
    a_off[i] = q < kPieces ? (uint32_t)r * (uint32_t)p.a_stride + 16u * (uint32_t)(q % 13) : kOob;
  }
  // the block's scales: piece q = tid + 256 i of the runs laid end to end
  // (run bytes = run rows * K / 32, a multiple of 16) -> LDS byte 16 q, by
  // global-to-LDS loads issued before the chunk loads (no registers; waited
  // for at the end of the prologue).  A piece past the runs, or past the
  // expert's matrix, re-reads the expert's first piece into LDS no one
  // reads.
  constexpr int kRuns = SWIGLU ? 2 : 1, kRunRows = kMx6BlockRows / kRuns;
  const int srow_bytes = K / 32, run_pieces = kRunRows * srow_bytes / 16;
  {
    const uint8_t* sbase = p.bs + (int64_t)e * sbytes;
#pragma unroll
    for (int i = 0; i < kMx6SPieces<W8>; ++i) {
      const int q = (int)threadIdx.x + 256 * i;
      const int run = q / run_pieces, part = q - run * run_pieces;
      const int64_t off = (int64_t)(run * p.b_row_second + n0) * srow_bytes + 16 * part;
      const bool ok = run < kRuns && off + 16 <= sbytes;
      load_lds16(sbase + (ok ? off : 0), lds_addr(sall + 16 * (256 * i + 64 * wave)));
    }
  }

  // block row r (= kMx6WaveRows w + 16 j + n: wave w, column tile j, lane
  // column n) -> expert-relative weight row, or -1 past N.  Gate/up: the
  // first JW / 2 tiles of a wave are gate rows, the others the matching up
  // rows, so the wave's SwiGLU pairs stay in its registers.
  auto weight_row = [&](int r) {
    const int w = r / kMx6WaveRows, j = (r >> 4) % JW, nn = r & 15;
    if constexpr (SWIGLU) {
      const int col = n0 + (kMx6WaveRows / 2) * w + 16 * (j % (JW / 2)) + nn;
      return col < p.N ? col + (j / (JW / 2)) * p.b_row_second : -1;
    } else {
      const int col = n0 + kMx6WaveRows * w + 16 * j + nn;
      return col < p.N ? col : -1;
    }
  };
  uint32_t q_off[JW];
#pragma unroll
  for (int j = 0; j < JW; ++j) {
    const int row = weight_row(kMx6WaveRows * wave + 16 * j + n);
    q_off[j] = row >= 0 ? (uint32_t)row * (uint32_t)S::kRowBytes(K) + 16u * (uint32_t)g : kOob;
  }

  // NB weight buffers, filled two chunks at a time (see step)
  constexpr int NB = 4;
  u32x4_t areg[kMx6ABufs][kPerThread];
  u32x4_t bq[NB][JW];
  u32x4_t bq2[W8 ? NB : 1][JW];  // MXFP8: the second 16-byte piece of each lane's codes
  f32x4_t acc[MT][JW];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int j = 0; j < JW; ++j) acc[m][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // per-lane offsets stay fixed; the chunk enters as the scalar offset
  // (a piece or row past the end has a per-lane offset of kOob and reads zero)
  auto load_a = [&](int c, int abuf) {
#pragma unroll
    for (int i = 0; i < kPerThread; ++i)
      areg[abuf][i] =
          __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ra, (int)a_off[i], kMx6Rec * c, 0));
  };
  // no branch around the writes: a divergent one makes the compiler wait for
  // every load in flight before the write
  auto store_a = [&](int s, int abuf) {
    uint8_t* st = stage + s * kMx6Stage + 16 * threadIdx.x;
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) *reinterpret_cast<u32x4_t*>(st + 4096 * i) = areg[abuf][i];
  };
  // two chunks per burst, the same rows back to back: each row is read 128
  // contiguous bytes (a whole cache line) at a time
  // (MXFP8: one chunk is already 128 contiguous bytes of a row, read as two
  // 16-byte pieces per lane)
  auto load_b2 = [&](int c0, int c1, int buf0, int buf1) {
#pragma unroll
    for (int j = 0; j < JW; ++j) {
      if constexpr (W8) {
        bq[buf0][j] =
            __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)q_off[j], 128 * c0, 0));
        bq2[buf0][j] =
            __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)q_off[j], 128 * c0 + 64, 0));
        bq[buf1][j] =
            __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)q_off[j], 128 * c1, 0));
        bq2[buf1][j] =
            __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)q_off[j], 128 * c1 + 64, 0));
      } else {
        bq[buf0][j] =
            __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)q_off[j], 64 * c0, 0));
        bq[buf1][j] =
            __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rq, (int)q_off[j], 64 * c1, 0));
      }
    }
  };
  // A operands of one row tile: the hi and lo terms and the scale word
  struct AFrag {
    i32x8_t hi, lo;
    int sc;
  };
  auto read_a = [&](const uint8_t* rec) {
    const u32x4_t h0 = *reinterpret_cast<const u32x4_t*>(rec + 16 * g);
    const u32x2_t h1 = *reinterpret_cast<const u32x2_t*>(rec + 64 + 8 * g);
    const u32x4_t l0 = *reinterpret_cast<const u32x4_t*>(rec + 96 + 16 * g);
    const u32x2_t l1 = *reinterpret_cast<const u32x2_t*>(rec + 160 + 8 * g);
    AFrag f;
    f.sc = *reinterpret_cast<const int*>(rec + 192 + 4 * g);
    f.hi = i32x8_t{(int)h0[0], (int)h0[1], (int)h0[2], (int)h0[3], (int)h1[0], (int)h1[1], 0, 0};
    f.lo = i32x8_t{(int)l0[0], (int)l0[1], (int)l0[2], (int)l0[3], (int)l1[0], (int)l1[1], 0, 0};
    return f;
  };
  // LDS scale rows: column tile j's lane column n sits at row
  // scale_row0 + scale_drow(j) of the runs (the step is wave-uniform)
  const int scale_row0 = SWIGLU ? (kMx6WaveRows / 2) * wave + n : kMx6WaveRows * wave + n;
  auto scale_drow = [&](int j) {
    return SWIGLU ? (j / (JW / 2)) * kRunRows + 16 * (j % (JW / 2)) : 16 * j;
  };
  const uint8_t* sb_lane = sall + scale_row0 * srow_bytes + g;
  // row tile m + 1's LDS reads are issued before row tile m's MFMAs (two
  // operand sets live), fenced so the compiler does not hoist further
  auto compute = [&](int s, int buf, int c) {
    // this lane's scale byte of each column tile: chunk c, lane group g
    int sb[JW];
#pragma unroll
    for (int j = 0; j < JW; ++j) sb[j] = sb_lane[scale_drow(j) * srow_bytes + 4 * c];
    const uint8_t* st = stage + s * kMx6Stage + n * kMx6Rec;
    AFrag cur = read_a(st);
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      AFrag nxt;
      if (m + 1 < MT) nxt = read_a(st + (m + 1) * 16 * kMx6Rec);
#pragma unroll
      for (int j = 0; j < JW; ++j) {
        if constexpr (W8) {
          acc[m][j] = mfma_f6f8(cur.hi, bq[buf][j], bq2[buf][j], cur.sc, sb[j], acc[m][j], 0);
          acc[m][j] = mfma_f6f8(cur.lo, bq[buf][j], bq2[buf][j], cur.sc, sb[j], acc[m][j], 1);
        } else {
          acc[m][j] = mfma_f6f4(cur.hi, bq[buf][j], cur.sc, sb[j], acc[m][j], 0);
          acc[m][j] = mfma_f6f4(cur.lo, bq[buf][j], cur.sc, sb[j], acc[m][j], 1);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if (m + 1 < MT) cur = nxt;
    }
  };
  // One chunk c (weights in register buffer c % NB, activations in LDS
  // stage c % 2): publish chunk c + 1's activations (register buffer
  // (c + 1) % kMx6ABufs) to the other LDS stage and reuse that buffer for
  // chunk c + 1 + kMx6ABufs; on even steps issue the weights of chunks
  // c + 2 and c + 3 (one burst); compute chunk c.  Loads complete in issue
  // order, so the wait for chunk c + 1's activations also covers every load
  // issued before them.  The last steps load the last chunk again instead of
  // chunks past the end (the scalar offset is outside the buffer range
  // check) and never use it, so the loop has no branch but the compute
  // guard of its last steps.
  const int last = nchunks - 1;
  auto step = [&](int c, int buf, int u) {
    const int ab = (u + 1) % kMx6ABufs;
    store_a((c + 1) & 1, ab);
    load_a(min(c + 1 + kMx6ABufs, last), ab);
    if ((u & 1) == 0) load_b2(min(c + 2, last), min(c + 3, last), (buf + 2) % NB, (buf + 3) % NB);
    if (c < nchunks) compute(c & 1, buf, c);
    __syncthreads();
  };

#pragma unroll
  for (int i = 0; i < kMx6ABufs; ++i) load_a(min(i, last), i);
  load_b2(0, min(1, last), 0, 1);
  store_a(0, 0);
  load_a(min(kMx6ABufs, last), 0);
  // the scale loads were issued before the (kMx6ABufs + 1) kPerThread
  // activation and the first burst's weight loads above (2 JW, MXFP8 4 JW),
  // and loads complete in issue order: this wait leaves at most those in
  // flight (any other load issued after the scales only makes it stricter)
  constexpr int kBurstLoads = (W8 ? 4 : 2) * JW;
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"((kMx6ABufs + 1) * kPerThread + kBurstLoads) : "memory");
  __syncthreads();
  static_assert(kMx6Unroll % NB == 0 && kMx6Unroll % kMx6ABufs == 0, "the buffer indices repeat per iteration");
  for (int c = 0; c < nchunks; c += kMx6Unroll) {
#pragma unroll
    for (int u = 0; u < kMx6Unroll; ++u) step(c + u, u % NB, u);
  }

  // epilogue: lane 16 g + n holds rows 4 g + i of each row tile, column n of each column tile
  if constexpr (SWIGLU) {
    if (p.Cmx) {
      mx6_epilogue_records<MT, W8>(p, acc, stage, sall, m_begin, rows, n0);
      return;
    }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * m + 4 * g + i;
      if (r >= rows) continue;
      uint16_t* crow = p.C + (int64_t)(m_begin + r) * p.ldc;
      if constexpr (SWIGLU) {
#pragma unroll
        for (int j = 0; j < JW / 2; ++j) {
          const int col = n0 + (kMx6WaveRows / 2) * wave + 16 * j + n;
          if (col < p.N) crow[col] = f32_to_bf16(clamped_swiglu(acc[m][j][i], acc[m][j + JW / 2][i], p.limit));
        }
      } else {
#pragma unroll
        for (int j = 0; j < JW; ++j) {
          const int col = n0 + kMx6WaveRows * wave + 16 * j + n;
          if (col < p.N) crow[col] = f32_to_bf16(acc[m][j][i]);
        }
      }
    }
}

// h columns (gate/up) or output columns (down) per block
template <bool SWIGLU, bool W8>
constexpr int kMx6BlockCols = SWIGLU ? Mx6Shape<W8>::kBlockRows / 2 : Mx6Shape<W8>::kBlockRows;

// XCD-aware block order (as the pipelined kernels): block b runs on XCD
// b % 8, which takes the tiles t with t % 8 == its index and runs a tile's
// column blocks back to back, so the tile's activation records stay in that
// XCD's L2 while its column blocks read them.  An expert's consecutive row
// tiles run at about the same time on different XCDs and share their weight
// reads through the memory-side cache (grouping them on one XCD measured
// slower: 1873 -> 1930-2130 us for the 16384-token gate/up).  One block per
// CU, one wave per SIMD (512 registers a wave).
template <bool SWIGLU, bool W8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void expert_mx6_kernel(const Mx6Params p, int n_tiles, int col_blocks) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[2 * kMx6Stage];
  __shared__ __attribute__((aligned(16))) uint8_t sall[kMx6SBytes];
  const int b = (int)blockIdx.x, x = b & 7, q = b >> 3;
  const int tile = 8 * (q / col_blocks) + x, cb = q % col_blocks;
  if (tile >= n_tiles || tile >= *p.tile_count) return;
  const GemmTile tl = p.tiles[tile];
  const int m_begin = tl.m_begin, rows = min(tl.m_end, tl.m_begin + kMx6Rows) - tl.m_begin;
  if (rows <= 0) return;
  const int n0 = cb * kMx6BlockCols<SWIGLU, W8>;
  const int mt = min(kMx6Rows / 16, 2 * ((rows + 31) / 32));
  switch (mt) {
    case 2: mx6_tile<SWIGLU, 2, W8>(p, stage, sall, tl.e, m_begin, rows, n0); break;
    case 4: mx6_tile<SWIGLU, 4, W8>(p, stage, sall, tl.e, m_begin, rows, n0); break;
    default: mx6_tile<SWIGLU, 6, W8>(p, stage, sall, tl.e, m_begin, rows, n0); break;
  }
}

}  // namespace

bool mx6_supported(int hidden, int inter) {
  return hidden % 128 == 0 && inter % 128 == 0 && hidden <= kMx6MaxK && inter <= kMx6MaxK;
}

int mx6_tile_rows() { return kMx6TileRows; }

int64_t mx6_bytes(int64_t rows, int K) { return rows * mx6_row_bytes(K); }

hipError_t launch_mx6_rows(const uint16_t* src, int64_t ld_src, int rows, int K, uint8_t* dst, hipStream_t stream) {
  const int64_t units = (int64_t)rows * (K / 128);
  if (units == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((units + 255) / 256);
  if (ld_src == K)  // contiguous rows in, contiguous records out
    hipLaunchKernelGGL(mx6_rows_kernel, dim3(blocks), dim3(256), 0, stream, src, units, dst);
  else
    hipLaunchKernelGGL(mx6_rows_strided_kernel, dim3(blocks), dim3(256), 0, stream, src, ld_src, rows, K, dst,
                       mx6_row_bytes(K));
  return hipGetLastError();
}

hipError_t launch_expert_mx6(const Mx6Params& p, bool swiglu, int n_tiles, hipStream_t stream) {
  const int cols = p.w8 ? (swiglu ? kMx6BlockCols<true, true> : kMx6BlockCols<false, true>)
                        : (swiglu ? kMx6BlockCols<true, false> : kMx6BlockCols<false, false>);
  const int col_blocks = (p.N + cols - 1) / cols;
  const dim3 grid((unsigned)((n_tiles + 7) / 8 * 8 * col_blocks));
  auto kern = p.w8 ? (swiglu ? expert_mx6_kernel<true, true> : expert_mx6_kernel<false, true>)
                   : (swiglu ? expert_mx6_kernel<true, false> : expert_mx6_kernel<false, false>);
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, p, n_tiles, col_blocks);
  return hipGetLastError();
}

}  // namespace moe
