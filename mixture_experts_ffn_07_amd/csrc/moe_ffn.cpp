// C ABI of the MoE FFN layer: argument checks, workspace layout and the launch
// sequence of each entry point (declared in include/moe_ffn.h, and the timing
// call in include/moe_ffn_profile.h).
#include "../../include/moe_ffn.h"
#include "../../include/moe_ffn_profile.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <mutex>
#include <string>

#include "mx_device.h"

#include "moe_internal.h"

namespace {

thread_local std::string g_last_error;

moe_status fail(moe_status s, const char* what) {
  g_last_error = what;
  return s;
}

moe_status fail_hip(hipError_t err, const char* where) {
  char buf[256];
  std::snprintf(buf, sizeof(buf), "%s: %s", where, hipGetErrorString(err));
  g_last_error = buf;
  return MOE_ERR_HIP;
}

// Scratch memory of moe_layer_forward_noalloc: a device array in this code
// object, so every GPU the library runs on holds its own copy until the
// process ends.  In host code `scratch` names a host-side stand-in, not
// device memory: the kernels get the device address from
// hipGetSymbolAddress, taken once per device (scratch_ptr below).
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on device `dev`, which must be the current
// device; looked up on the first call for that device.
moe_status scratch_ptr(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(MOE_ERR_UNSUPPORTED, "device index beyond the 64 the library tracks");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return fail_hip(err, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(MOE_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return MOE_OK;
}

// Side stream of the many-token layer: the shared expert (independent of
// the routing) runs on it beside the router, top-k, permutation and routed
// GEMMs of the caller's stream, forked and joined by events.  One stream and
// one event pair per device, created by the first call that can use them
// (not under graph capture); the lock keeps each call's record and wait
// sequence whole when several host threads call at once.
struct SideStream {
  hipStream_t st = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool failed = false;  // creation failed once: the single-stream form serves
};
std::mutex g_side_mu[kMaxDevices];
SideStream g_side[kMaxDevices];

// The side stream of device `dev` (its lock held), or nullptr when the
// single-stream form must serve.
SideStream* side_stream(int dev, hipStream_t caller) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  SideStream& s = g_side[dev];
  if (s.st && s.fork && s.join) return &s;
  if (s.failed) return nullptr;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (caller && hipStreamIsCapturing(caller, &cap) != hipSuccess) return nullptr;
  if (cap != hipStreamCaptureStatusNone) return nullptr;
  if (!s.st && hipStreamCreateWithFlags(&s.st, hipStreamNonBlocking) != hipSuccess) {
    s.st = nullptr;
    s.failed = true;
    return nullptr;
  }
  if ((!s.fork && hipEventCreateWithFlags(&s.fork, hipEventDisableTiming) != hipSuccess) ||
      (!s.join && hipEventCreateWithFlags(&s.join, hipEventDisableTiming) != hipSuccess)) {
    s.failed = true;  // the stream and any event made stay unused until the process ends
    return nullptr;
  }
  return &s;
}

// Optional per-kernel timing: an event recorded after every launch.
struct Timeline {
  static constexpr int kMax = 32;
  hipEvent_t ev[kMax + 1];
  const char* names[kMax];
  int n = 0;
};

// Record the end of the kernel just launched (no-op without a timeline).
hipError_t mark(Timeline* tl, const char* name, hipStream_t st) {
  if (!tl || tl->n >= Timeline::kMax) return hipSuccess;
  tl->names[tl->n] = name;
  return hipEventRecord(tl->ev[++tl->n], st);
}

constexpr int64_t kMaxTokens = int64_t(1) << 22;
// few-token path: T <= 8 rows staged in at most 64 KB of LDS per block
constexpr int64_t kDecodeMaxTokens = 8;
constexpr size_t kDecodeMaxLds = 64 * 1024;
constexpr int kMaxDim = 65536;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

moe_status check_config(const moe_config* c) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "cfg is NULL");
  if (c->hidden <= 0 || c->hidden % 32 || c->hidden > kMaxDim)
    return fail(MOE_ERR_INVALID_ARG, "hidden must be a positive multiple of 32, at most 65536");
  if (c->inter <= 0 || c->inter % 32 || c->inter > kMaxDim)
    return fail(MOE_ERR_INVALID_ARG, "inter must be a positive multiple of 32, at most 65536");
  if (c->n_experts < 1 || c->n_experts > 1024) return fail(MOE_ERR_INVALID_ARG, "n_experts must be in [1, 1024]");
  if (c->top_k < 1 || c->top_k > 16 || c->top_k > c->n_experts)
    return fail(MOE_ERR_INVALID_ARG, "top_k must be in [1, min(n_experts, 16)]");
  if (c->n_shared != 0 && c->n_shared != 1) return fail(MOE_ERR_INVALID_ARG, "n_shared must be 0 or 1");
  if (c->n_shared == 1 && (c->shared_inter <= 0 || c->shared_inter % 32 || c->shared_inter > kMaxDim))
    return fail(MOE_ERR_INVALID_ARG, "shared_inter must be a positive multiple of 32, at most 65536");
  if (c->score_func != 0) return fail(MOE_ERR_UNSUPPORTED, "score_func must be 0 (sqrtsoftplus)");
  if (!std::isfinite(c->route_scale)) return fail(MOE_ERR_INVALID_ARG, "route_scale must be finite");
  if (!(c->swiglu_limit > 0.f)) return fail(MOE_ERR_INVALID_ARG, "swiglu_limit must be > 0");
  if (c->expert_format != 0 && c->expert_format != 1)
    return fail(MOE_ERR_INVALID_ARG, "expert_format must be 0 (MXFP4) or 1 (MXFP8)");
  return MOE_OK;
}

moe_status check_tokens(int64_t tokens) {
  if (tokens < 0 || tokens > kMaxTokens) return fail(MOE_ERR_INVALID_ARG, "tokens must be in [0, 2^22]");
  return MOE_OK;
}

// Matrices some kernels address through a 32-bit buffer descriptor, whose
// out-of-range offset is kOob: each must stay below kOob bytes.  Called with
// a checked config.
moe_status check_buffer_extents(const moe_config* c, int64_t T) {
  const int64_t H = c->hidden, I = c->inter, k = c->top_k, E = c->n_experts;
  const int64_t Is = c->n_shared ? c->shared_inter : 0;
  const int64_t code = c->expert_format == 1 ? 2 : 1;  // code bytes per two elements
  struct Extent {
    const char* what;
    int64_t bytes;
  };
  const Extent ext[] = {
      {"x [tokens][hidden] bf16", T * H * 2},
      {"the routed activations [tokens*top_k][inter] bf16", T * k * I * 2},
      {"the shared activations [tokens][shared_inter] bf16", T * Is * 2},
      {"one routed expert's gate/up codes", 2 * I * H * code / 2},
      {"one routed expert's down codes", H * I * code / 2},
      {"the shared gate/up matrix", 2 * Is * H * 2},
      {"the shared down matrix", H * Is * 2},
      {"the router matrix", E * H * 4},
  };
  for (const Extent& e : ext) {
    if (e.bytes >= (int64_t)moe::kOob) {
      static thread_local char buf[200];
      std::snprintf(buf, sizeof(buf), "%s would take %lld bytes, at or above the 2^31 - 16 a buffer may have; "
                    "split the tokens into smaller calls", e.what, (long long)e.bytes);
      return fail(MOE_ERR_UNSUPPORTED, buf);
    }
  }
  return MOE_OK;
}

moe_status need(const void* p, size_t align, const char* name) {
  static thread_local char buf[160];
  if (!p) {
    std::snprintf(buf, sizeof(buf), "%s is NULL", name);
    return fail(MOE_ERR_INVALID_ARG, buf);
  }
  if (!aligned(p, align)) {
    std::snprintf(buf, sizeof(buf), "%s is not %zu-byte aligned", name, align);
    return fail(MOE_ERR_ALIGNMENT, buf);
  }
  return MOE_OK;
}

moe_status check_routed_weights(const moe_config* c, const moe_weights* w, bool need_router, bool need_experts) {
  if (!w) return fail(MOE_ERR_INVALID_ARG, "weights is NULL");
  moe_status s;
  if (need_router) {
    if ((s = need(w->router_w, 16, "router_w")) != MOE_OK) return s;
    if (w->router_bias && !aligned(w->router_bias, 4)) return fail(MOE_ERR_ALIGNMENT, "router_bias is not 4-byte aligned");
  }
  if (need_experts) {
    if ((s = need(w->gu_q, 16, "gu_q")) != MOE_OK) return s;
    if ((s = need(w->gu_s, 16, "gu_s")) != MOE_OK) return s;
    if ((s = need(w->dn_q, 16, "dn_q")) != MOE_OK) return s;
    if ((s = need(w->dn_s, 16, "dn_s")) != MOE_OK) return s;
    if (c->n_shared == 1) {
      if ((s = need(w->sh_gu, 16, "sh_gu")) != MOE_OK) return s;
      if ((s = need(w->sh_dn, 16, "sh_dn")) != MOE_OK) return s;
    } else if (w->sh_gu || w->sh_dn) {
      return fail(MOE_ERR_INVALID_ARG, "sh_gu/sh_dn must be NULL when n_shared == 0");
    }
  }
  return MOE_OK;
}

moe_status check_norm(const moe_config* c, const uint16_t* gamma) {
  moe_status s;
  if ((s = need(gamma, 16, "norm_gamma")) != MOE_OK) return s;
  if (!std::isfinite(c->norm_eps) || !(c->norm_eps > 0.f)) return fail(MOE_ERR_INVALID_ARG, "norm_eps must be finite and > 0");
  return MOE_OK;
}

// ---------------------------------------------------------------- workspace layout
struct Region {
  size_t off = 0, bytes = 0;
};

struct WsLayout {
  moe::RouterPlan router;
  moe::WeightFormat fmt = moe::kWMxfp4;  // routed experts' codec
  bool decode = false;  // few tokens: GEMV router, fused routing, weight-streaming projections
  int bm = 16;          // rows per routed GEMM tile
  int gemm_mt = 1, shared_mt = 1;
  bool shared_skinny = false;   // shared expert on the skinny kernel (shared_ks_* K ranges)
  // shared expert at 128..1023 tokens: the dense kernel over K slices (0: off)
  int shared_ks_gu = 0, shared_ks_dn = 0;
  int64_t max_tiles = 0, shared_tiles = 0;
  bool route_small = false;   // decode with T * k <= 64: scores from the router GEMV, one-block routing
  bool down_combine = false;  // decode: routed down projection with the combine folded in
  bool splitk_dn = false;     // decode: routed down by the split-K MXFP4 kernel
  bool valu_gu = false;       // decode, T <= 2: routed gate/up one wave per column on the vector ALUs
  bool valu_dn = false;       // decode, T <= 2: routed down + combine one wave per column on the vector ALUs
  bool stream4 = false;       // decode, T <= 2: router; routing + shared gate/up; routed gate/up + shared
                              // down; routed down + combine
  bool norm_in_router = false;  // stream4 with the pre-FFN norm folded into the router launch
  bool stream3 = false;         // stream4 in three launches: every routed gate/up wave routes for itself,
                                // the shared gate/up streams beside it, the shared down joins the combine
  bool mx6 = false;             // many tokens, MXFP4: routed gate/up on two-term MXFP6 activations (expert_mx6.hip)
  bool mx6_dn = false;          // ... and the routed down projection too
  Region xq, hq, x_norm, w3, logits, scores, xmx, tile_rows, hmx, rank, chunk_counts, chunk_base, tiles, tile_count, idx, w, offsets, sorted, slot_pos, h,
      y_slot, h_sh, y_sh, sh_part;
  size_t total = 0;
};

WsLayout plan_workspace_impl(const moe_config* c, int64_t tokens, bool allow_decode) {
  WsLayout L;
  const int64_t n = tokens * c->top_k;
  const int E = c->n_experts;
  L.router = moe::router_plan(tokens, E, c->hidden);
  L.fmt = c->expert_format == 1 ? moe::kWMxfp8 : moe::kWMxfp4;
  L.gemm_mt = moe::expert_gemm_mt(n, (int)(n < E ? n : E), L.fmt, c->hidden % 128 == 0 && c->inter % 128 == 0);
  L.shared_mt = moe::expert_gemm_mt(tokens, 1, moe::kWBf16, false);
  if (L.shared_mt == 1 && tokens > 16) L.shared_mt = 2;  // 32-row tiles: the weights read half as often
  const int k_fp4 = c->hidden > c->inter ? c->hidden : c->inter;
  const int k_bf16 = c->n_shared ? (c->hidden > c->shared_inter ? c->hidden : c->shared_inter) : 0;
  const bool fp8 = L.fmt == moe::kWMxfp8;
  L.decode = allow_decode && tokens >= 1 && tokens <= kDecodeMaxTokens && n <= moe::kPermuteChunk &&
             moe::gemv_lds_bytes((int)tokens, k_fp4, true) <= kDecodeMaxLds &&
             moe::gemv_lds_bytes((int)tokens, k_bf16, false) <= kDecodeMaxLds;
  if (L.decode) {
    L.route_small = n <= moe::kRouteSmallMaxSlots;
    L.down_combine = tokens <= moe::kDownCombineMaxTokens && n <= 64 && c->inter <= moe::kDownCombineMaxInter &&
                     moe::down_combine_lds_bytes((int)tokens, c->top_k, c->inter) <= kDecodeMaxLds;
    // the split-K down projection plus a separate combine measured faster than
    // the fused down+combine kernel (11.8 + 4.1 us against 19.8 us at T = 1)
    L.splitk_dn = moe::splitk_supported((int)tokens, c->inter);
    L.down_combine = L.down_combine && !L.splitk_dn && !fp8;  // its kernel reads MXFP4 weights
    L.valu_dn = L.route_small && moe::down_valu_supported((int)tokens, c->top_k, c->inter, fp8);
    L.router.ksplit = 1;  // full logits from the GEMV router
    L.router.dense_kslices = 0;
    L.bm = (int)tokens;   // an expert gets at most T rows: one tile per expert
  } else {
    L.bm = 16 * L.gemm_mt;
    // K multiples of 128: the block-scaled MFMA on two-term MXFP6 rows, in
    // tiles of its own height, at any row count past the few-token kernels
    // (it streams the weights straight to registers: 64 tokens, routed
    // gate/up 664 -> 533 us against the 32-row bf16 kernel); MXFP8 weights
    // too, as its 8-bit operand (64 tokens 1227 -> 962 us, 4096 tokens
    // 2325 -> 2132 us against the bf16 kernels on dequantised E4M3)
    L.mx6 = moe::mx6_supported(c->hidden, c->inter);
    // it takes tiles of up to mx6_tile_rows() rows: 128-row tiles become
    // tiles of that height; 32-row tiles stay, since the down projection's
    // 32-row kernel, which shares the tile table, computes 32 rows per tile
    if (L.mx6 && L.bm > moe::mx6_tile_rows()) L.bm = moe::mx6_tile_rows();
    // the down projection (K = I, 18 chunks at I = 2304) takes it too when
    // the tiles are its own height (experts averaging more than 16 rows), h
    // then leaving the gate/up epilogue as MXFP6 records.  With a pass of its
    // own writing the records (4096 tokens 710 + 55 us against 768 us on the
    // 512-row bf16 kernel; 16384 tokens 1099 + 97 against 1106) the layer
    // gained 1.7% and 0.3%.  With 32-row tiles (64 and 320 tokens) the
    // 32-row bf16 kernel is faster (64 tokens: 300 against 284 us).  MXFP8
    // weights take it at every tile height: against the 16-row bf16 kernel at
    // 16-row tiles, 16 tokens 672 -> 647 us, 64 tokens 1707 -> 1645, 320
    // tokens 2840 -> 2588, 700 tokens 3412 -> 2852
    L.mx6_dn = L.mx6 && (L.bm == moe::mx6_tile_rows() || L.fmt == moe::kWMxfp8);
  }
  L.max_tiles = moe::max_gemm_tiles(n, E, L.bm);
  {
    // each expert holds at most T rows, so at most ceil(T / bm) tiles
    const int64_t per_expert = (tokens + L.bm - 1) / L.bm;
    const int64_t bound = (n < E ? n : E) * per_expert;
    if (bound < L.max_tiles) L.max_tiles = bound;
  }
  if (L.decode) {
    L.valu_gu = L.route_small && moe::gate_up_valu_supported((int)tokens, c->hidden, (int)L.max_tiles, fp8);
    if (L.valu_gu || L.valu_dn) L.down_combine = false;  // h stays bf16
    L.stream4 = L.valu_gu && L.valu_dn &&
              moe::decode_valu_supported((int)tokens, c->hidden, c->n_shared ? c->shared_inter : 0) &&
              (c->n_shared == 0 ||
               moe::gate_up_shared_down_supported((int)tokens, c->hidden, (int)L.max_tiles, c->shared_inter, fp8));
    L.norm_in_router = L.stream4 && moe::router_norm_gemv_supported((int)tokens, c->hidden);
    L.stream3 = L.stream4 &&
                moe::route_gate_up_shared_gu_supported((int)tokens, c->hidden, E, c->top_k,
                                                       c->n_shared ? c->shared_inter : 0, fp8) &&
                (c->n_shared == 0 ||
                 moe::down_combine_shared_supported((int)tokens, c->top_k, c->inter, c->shared_inter, fp8));
  }
  L.shared_tiles = (tokens + 16 * L.shared_mt - 1) / (16 * L.shared_mt);
  if (c->n_shared == 1 && !L.decode && tokens <= 512) {
    // the skinny weight-streaming kernel over K ranges when both K are
    // multiples of 128 (64 tokens: 52 + 28 -> 28 + 18 us), else 32-row tiles
    const int gu = moe::skinny_k_slices((int)tokens, 2 * c->shared_inter, c->hidden);
    const int dn = moe::skinny_k_slices((int)tokens, c->hidden, c->shared_inter);
    if (gu > 0 && dn > 0) {
      L.shared_skinny = true;
      L.shared_ks_gu = gu;
      L.shared_ks_dn = dn;
    }
  }
  if (c->n_shared == 1 && !L.decode && !L.shared_skinny && tokens >= 128 && tokens < 1024) {
    // 16-row tiles would re-read the shared weights once per tile (320
    // tokens: 184 + 114 -> 101 + 75 us); below 128 tokens the slices are too
    // short and their partial sums cost more (64 tokens: 57 + 31 -> 89 + 62 us)
    L.shared_ks_gu = moe::dense_k_slices((int)tokens, 2 * c->shared_inter, c->hidden);
    L.shared_ks_dn = moe::dense_k_slices((int)tokens, c->hidden, c->shared_inter);
  }
  const int64_t nchunks = moe::permute_chunks(n);
  size_t off = 0;
  auto take = [&](Region& r, size_t bytes) {
    r.off = off;
    r.bytes = bytes;
    off += (bytes + 255) & ~size_t(255);
  };
  take(L.x_norm, sizeof(uint16_t) * (size_t)tokens * c->hidden);
  take(L.w3, moe::router_w3_bytes(L.router, E, c->hidden));
  take(L.logits, sizeof(float) * (size_t)L.router.ksplit * tokens * E);
  take(L.scores, L.route_small ? sizeof(float) * 2 * (size_t)tokens * E : 0);
  take(L.xmx, L.route_small ? (size_t)tokens * moe::mx_row_bytes(c->hidden) : 0);
  take(L.tile_rows, L.route_small ? sizeof(int32_t) * moe::kTileRows * L.max_tiles : 0);
  take(L.hmx, L.down_combine ? (size_t)n * moe::mx_row_bytes(c->inter) : 0);
  take(L.rank, sizeof(int32_t) * n);
  take(L.chunk_counts, sizeof(int32_t) * nchunks * E);
  take(L.chunk_base, sizeof(int32_t) * nchunks * E);
  take(L.tiles, sizeof(moe::GemmTile) * L.max_tiles);
  take(L.tile_count, sizeof(int32_t) * 4);
  take(L.idx, sizeof(int32_t) * n);
  take(L.w, sizeof(float) * n);
  take(L.offsets, sizeof(int32_t) * (E + 1));
  take(L.sorted, sizeof(int32_t) * n);
  take(L.slot_pos, sizeof(int32_t) * n);
  take(L.xq, L.mx6 ? (size_t)moe::mx6_bytes(tokens, c->hidden) : 0);
  take(L.hq, L.mx6_dn ? (size_t)moe::mx6_bytes(n, c->inter) : 0);
  take(L.h, L.mx6_dn ? 0 : sizeof(uint16_t) * n * c->inter);  // MXFP6 down: h only as records (hq)
  take(L.y_slot, sizeof(uint16_t) * n * c->hidden);
  const int64_t is = c->n_shared ? c->shared_inter : 0;
  take(L.h_sh, sizeof(uint16_t) * tokens * is);
  {
    const size_t gu = (size_t)L.shared_ks_gu * tokens * 2 * is, dn = (size_t)L.shared_ks_dn * tokens * c->hidden;
    take(L.sh_part, sizeof(float) * (gu > dn ? gu : dn));
  }
  take(L.y_sh, sizeof(uint16_t) * (c->n_shared ? tokens * c->hidden : 0));
  L.total = off;
  return L;
}

WsLayout plan_workspace(const moe_config* c, int64_t tokens) {
  WsLayout L = plan_workspace_impl(c, tokens, true);
  // MXFP8 weights outside the one/two-token streaming form take the
  // few-token MFMA kernels when both K are multiples of 128 (whole 32-code
  // pieces per lane), else the general launch sequence
  if (L.fmt == moe::kWMxfp8 && L.decode && !L.stream4 && (c->hidden % 128 != 0 || c->inter % 128 != 0))
    L = plan_workspace_impl(c, tokens, false);
  return L;
}

template <typename T>
T* at(void* ws, const Region& r) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + r.off);
}

moe_status check_ws(void* ws, size_t ws_bytes, const WsLayout& L) {
  if (!ws) return fail(MOE_ERR_WORKSPACE, "ws is NULL");
  if (!aligned(ws, 256)) return fail(MOE_ERR_ALIGNMENT, "ws is not 256-byte aligned");
  if (ws_bytes < L.total) return fail(MOE_ERR_WORKSPACE, "ws_bytes is smaller than moe_workspace_bytes()");
  return MOE_OK;
}

// ---------------------------------------------------------------- launch sequences (arguments already checked)
moe_status run_route(const moe_config* c, const moe_weights* w, const uint16_t* x, int64_t T, int32_t* idx,
                     float* wts, float* gap, void* ws, const WsLayout& L, hipStream_t st, Timeline* tl) {
  float* part = at<float>(ws, L.logits);
  hipError_t err = L.decode
                       ? moe::launch_router_gemv(x, w->router_w, part, (int)T, c->n_experts, c->hidden, nullptr,
                                                 nullptr, st)
                       : moe::launch_router_logits(L.router, x, w->router_w, part, (int)T, c->n_experts, c->hidden,
                                                   at<uint16_t>(ws, L.w3), st);
  if (err == hipSuccess) err = mark(tl, "router_logits", st);
  if (err != hipSuccess) return fail_hip(err, "router logits launch");
  err = moe::launch_router_topk(part, L.router.ksplit, w->router_bias, (int)T, c->n_experts, c->top_k,
                                c->route_scale, idx, wts, gap, st);
  if (err == hipSuccess) err = mark(tl, "router_topk", st);
  if (err != hipSuccess) return fail_hip(err, "router top-k launch");
  return MOE_OK;
}

moe_status run_permute(const moe_config* c, const int32_t* idx, int64_t T, int32_t* offsets, int32_t* sorted,
                       int32_t* slot_pos, void* ws, const WsLayout& L, bool with_tiles, hipStream_t st,
                       Timeline* tl) {
  moe::PermuteScratch s{at<int32_t>(ws, L.rank), at<int32_t>(ws, L.chunk_counts), at<int32_t>(ws, L.chunk_base)};
  hipError_t err = moe::launch_permute(idx, (int)(T * c->top_k), c->n_experts, s, offsets, sorted, slot_pos,
                                       L.bm, (int)L.max_tiles, with_tiles ? at<moe::GemmTile>(ws, L.tiles) : nullptr,
                                       at<int32_t>(ws, L.tile_count), st);
  if (err == hipSuccess) err = mark(tl, "permute", st);
  if (err != hipSuccess) return fail_hip(err, "permute launch");
  return MOE_OK;
}

// Few tokens: weight-streaming projections, one tile per expert (routed) or
// one for all T rows (shared).
moe::GemvParams routed_gemv(const moe_config* c, const moe_weights* w, const uint16_t* x, const uint8_t* xmx,
                            int64_t T, const int32_t* sorted, void* ws, const WsLayout& L, bool gate_up,
                            uint16_t* y_slot) {
  const int H = c->hidden, I = c->inter;
  moe::GemvParams g{};
  g.rows_cap = (int)T;
  g.limit = c->swiglu_limit;
  moe::GemvProblem& r = g.p[0];
  r.w8 = L.fmt == moe::kWMxfp8;
  r.tiles = at<moe::GemmTile>(ws, L.tiles);
  r.tile_count = at<int32_t>(ws, L.tile_count);
  r.grid_tiles = (int)L.max_tiles;
  if (gate_up) {  // A = gathered token rows of x, B = W_gu[e] [2I][H], C = h
    r.gather = sorted;
    r.gather_div = c->top_k;
    r.gather_len = (int)(T * c->top_k);
    r.A = x;
    r.amx = xmx;
    r.lda = H;
    r.a_rows = (int)T;
    r.K = H;
    r.bq = w->gu_q;
    r.bs = w->gu_s;
    r.b_expert_rows = 2 * (int64_t)I;
    r.b_row_second = I;
    r.N = I;
    r.C = at<uint16_t>(ws, L.h);
    r.ldc = I;
  } else {  // A = h rows in position order, B = W_dn[e] [H][I], C = y_slot
    r.A = at<uint16_t>(ws, L.h);
    r.lda = I;
    r.a_rows = (int)(T * c->top_k);
    r.K = I;
    r.bq = w->dn_q;
    r.bs = w->dn_s;
    r.b_expert_rows = H;
    r.N = H;
    r.C = y_slot;
    r.ldc = H;
  }
  r.col_tiles = r.N / 16;
  return g;
}

moe::GemvParams shared_gemv(const moe_config* c, const moe_weights* w, const uint16_t* x, int64_t T, void* ws,
                            const WsLayout& L, bool gate_up, uint16_t* y_shared) {
  const int H = c->hidden, Is = c->shared_inter;
  moe::GemvParams g{};
  g.rows_cap = (int)T;
  g.limit = c->swiglu_limit;
  moe::GemvProblem& s = g.p[0];
  s.M = (int)T;
  s.grid_tiles = 1;
  s.a_rows = (int)T;
  if (gate_up) {
    s.A = x;
    s.lda = H;
    s.K = H;
    s.bh = w->sh_gu;
    s.b_expert_rows = 2 * (int64_t)Is;
    s.b_row_second = Is;
    s.N = Is;
    s.C = at<uint16_t>(ws, L.h_sh);
    s.ldc = Is;
  } else {
    s.A = at<uint16_t>(ws, L.h_sh);
    s.lda = Is;
    s.K = Is;
    s.bh = w->sh_dn;
    s.b_expert_rows = H;
    s.N = H;
    s.C = y_shared;
    s.ldc = H;
  }
  s.col_tiles = s.N / 16;
  return g;
}

moe_status run_shared_decode(const moe_config* c, const moe_weights* w, const uint16_t* x, int64_t T,
                             uint16_t* y_shared, void* ws, const WsLayout& L, hipStream_t st, Timeline* tl) {
  hipError_t err = moe::launch_expert_gemv(shared_gemv(c, w, x, T, ws, L, true, y_shared), true, false, st);
  if (err == hipSuccess) err = mark(tl, "shared_gate_up", st);
  if (err != hipSuccess) return fail_hip(err, "shared gate/up launch");
  err = moe::launch_expert_gemv(shared_gemv(c, w, x, T, ws, L, false, y_shared), false, false, st);
  if (err == hipSuccess) err = mark(tl, "shared_down", st);
  if (err != hipSuccess) return fail_hip(err, "shared down launch");
  return MOE_OK;
}

moe_status run_experts_decode(const moe_config* c, const moe_weights* w, const uint16_t* x, int64_t T,
                              const int32_t* sorted, uint16_t* y_slot, uint16_t* y_shared, void* ws,
                              const WsLayout& L, hipStream_t st, Timeline* tl) {
  hipError_t err =
      moe::launch_expert_gemv(routed_gemv(c, w, x, nullptr, T, sorted, ws, L, true, y_slot), true, true, st);
  if (err == hipSuccess) err = mark(tl, "routed_gate_up", st);
  if (err != hipSuccess) return fail_hip(err, "routed gate/up launch");
  err = moe::launch_expert_gemv(routed_gemv(c, w, x, nullptr, T, sorted, ws, L, false, y_slot), false, true, st);
  if (err == hipSuccess) err = mark(tl, "routed_down", st);
  if (err != hipSuccess) return fail_hip(err, "routed down launch");
  if (c->n_shared == 1) return run_shared_decode(c, w, x, T, y_shared, ws, L, st, tl);
  return MOE_OK;
}

// Few-token layer, T <= 2, streaming form (see launch_decode_route_shared_gu).
// With norm_gamma (and L.norm_in_router) the router launch normalises x and
// writes the rows the later launches read.
moe_status layer_forward_decode4(const moe_config* c, const moe_weights* w, const uint16_t* x, int64_t T,
                                 uint16_t* y, int32_t* idx, float* wts, void* ws, const WsLayout& L, hipStream_t st,
                                 Timeline* tl, const uint16_t* norm_gamma) {
  const int E = c->n_experts;
  const uint16_t* x_in = x;
  if (norm_gamma) x = at<uint16_t>(ws, L.x_norm);
  uint16_t* y_sh = c->n_shared ? at<uint16_t>(ws, L.y_sh) : nullptr;
  uint16_t* h_sh = c->n_shared ? at<uint16_t>(ws, L.h_sh) : nullptr;
  int32_t* slot_pos = at<int32_t>(ws, L.slot_pos);
  moe::GemmTile* tiles = at<moe::GemmTile>(ws, L.tiles);

  moe::FrontValuParams f{};
  f.x = x;
  f.router_w = w->router_w;
  f.bias = w->router_bias;
  f.scores = at<float>(ws, L.scores);
  f.sh_gu = c->n_shared ? w->sh_gu : nullptr;
  f.h_sh = h_sh;
  f.shared_inter = c->n_shared ? c->shared_inter : 0;
  f.tokens = (int)T;
  f.n_experts = E;
  f.hidden = c->hidden;
  f.limit = c->swiglu_limit;
  moe::RouteSmallParams rp{};
  rp.x = x;
  rp.xmx = nullptr;
  rp.scores = f.scores;
  rp.tokens = (int)T;
  rp.n_experts = E;
  rp.hidden = c->hidden;
  rp.top_k = c->top_k;
  rp.route_scale = c->route_scale;
  rp.idx = idx;
  rp.w = wts;
  rp.sorted_slots = at<int32_t>(ws, L.sorted);
  rp.slot_pos = slot_pos;
  rp.tiles = tiles;
  rp.tile_count = at<int32_t>(ws, L.tile_count);
  rp.tile_rows = at<int32_t>(ws, L.tile_rows);
  rp.max_tiles = (int)L.max_tiles;
  hipError_t err;
  if (L.stream3 && !norm_gamma && c->n_shared) {
    // 1. router scores beside the shared gate/up; 2. routed gate/up (in-wave
    // routing) beside the shared down; 3. routed down + combine
    err = moe::launch_decode_front_valu(f, st);
    if (err == hipSuccess) err = mark(tl, "router_scores_shared_gate_up", st);
    if (err != hipSuccess) return fail_hip(err, "router/shared gate-up launch");
    moe::GateUpValuParams g{};
    g.x = x;
    g.gu_q = w->gu_q;
    g.gu_s = w->gu_s;
    g.h = at<uint16_t>(ws, L.h);
    g.tokens = (int)T;
    g.hidden = c->hidden;
    g.inter = c->inter;
    g.limit = c->swiglu_limit;
    g.fp8 = L.fmt == moe::kWMxfp8;
    g.scores = f.scores;
    g.n_experts = E;
    g.top_k = c->top_k;
    g.route_scale = c->route_scale;
    g.idx = idx;
    g.w = wts;
    g.slot_pos = slot_pos;
    g.sorted_slots = rp.sorted_slots;
    moe::MidValuParams m{};
    m.sh_dn = w->sh_dn;
    m.h_sh = h_sh;
    m.y_sh = y_sh;
    m.shared_inter = c->shared_inter;
    m.tokens = (int)T;
    m.hidden = c->hidden;
    err = moe::launch_route_gate_up_shared_down(g, m, st);
    if (err == hipSuccess) err = mark(tl, "route_gate_up_shared_down", st);
    if (err != hipSuccess) return fail_hip(err, "routed gate/up launch");
    moe::DownValuParams dv{};
    dv.h = g.h;
    dv.idx = idx;
    dv.topk_w = wts;
    dv.slot_pos = slot_pos;
    dv.dn_q = w->dn_q;
    dv.dn_s = w->dn_s;
    dv.y_shared = y_sh;
    dv.y = y;
    dv.tokens = (int)T;
    dv.top_k = c->top_k;
    dv.hidden = c->hidden;
    dv.inter = c->inter;
    dv.fp8 = g.fp8;
    err = moe::launch_down_combine_valu(dv, st);
    if (err == hipSuccess) err = mark(tl, "routed_down_combine", st);
    if (err != hipSuccess) return fail_hip(err, "down/combine launch");
    return MOE_OK;
  }
  if (norm_gamma) {
    err = moe::launch_router_norm_gemv(x_in, norm_gamma, (double)c->norm_eps, at<uint16_t>(ws, L.x_norm),
                                       w->router_w, (int)T, E, c->hidden, f.scores, w->router_bias, st);
    if (err == hipSuccess) err = mark(tl, "norm_router_scores", st);
  } else {
    err = moe::launch_router_gemv(x, w->router_w, nullptr, (int)T, E, c->hidden, f.scores, w->router_bias, st);
    if (err == hipSuccess) err = mark(tl, "router_scores", st);
  }
  if (err != hipSuccess) return fail_hip(err, "router launch");
  if (L.stream3) {
    moe::GateUpValuParams g{};
    g.x = x;
    g.gu_q = w->gu_q;
    g.gu_s = w->gu_s;
    g.h = at<uint16_t>(ws, L.h);
    g.tokens = (int)T;
    g.hidden = c->hidden;
    g.inter = c->inter;
    g.limit = c->swiglu_limit;
    g.fp8 = L.fmt == moe::kWMxfp8;
    g.scores = f.scores;
    g.n_experts = E;
    g.top_k = c->top_k;
    g.route_scale = c->route_scale;
    g.idx = idx;
    g.w = wts;
    g.slot_pos = slot_pos;
    g.sorted_slots = rp.sorted_slots;
    err = moe::launch_route_gate_up_shared_gu(g, f, st);
    if (err == hipSuccess) err = mark(tl, "route_gate_up_shared_gate_up", st);
    if (err != hipSuccess) return fail_hip(err, "routed and shared gate/up launch");
    moe::DownValuParams dv{};
    dv.h = g.h;
    dv.idx = idx;
    dv.topk_w = wts;
    dv.slot_pos = slot_pos;
    dv.dn_q = w->dn_q;
    dv.dn_s = w->dn_s;
    dv.y = y;
    dv.tokens = (int)T;
    dv.top_k = c->top_k;
    dv.hidden = c->hidden;
    dv.inter = c->inter;
    dv.fp8 = g.fp8;
    if (c->n_shared) {
      dv.sh_dn = w->sh_dn;
      dv.h_sh = h_sh;
      dv.shared_inter = c->shared_inter;
      err = moe::launch_down_combine_shared(dv, st);
      if (err == hipSuccess) err = mark(tl, "routed_down_shared_down_combine", st);
    } else {
      err = moe::launch_down_combine_valu(dv, st);
      if (err == hipSuccess) err = mark(tl, "routed_down_combine", st);
    }
    if (err != hipSuccess) return fail_hip(err, "down/combine launch");
    return MOE_OK;
  }
  err = moe::launch_decode_route_shared_gu(f, rp, st);
  if (err == hipSuccess) err = mark(tl, "route_shared_gate_up", st);
  if (err != hipSuccess) return fail_hip(err, "routing/shared gate-up launch");

  moe::GateUpValuParams g{};
  g.x = x;
  g.tiles = tiles;
  g.tile_rows = rp.tile_rows;
  g.gu_q = w->gu_q;
  g.gu_s = w->gu_s;
  g.h = at<uint16_t>(ws, L.h);
  g.tokens = (int)T;
  g.hidden = c->hidden;
  g.inter = c->inter;
  g.limit = c->swiglu_limit;
  g.fp8 = L.fmt == moe::kWMxfp8;
  if (c->n_shared) {
    moe::MidValuParams m{};
    m.sh_dn = w->sh_dn;
    m.h_sh = h_sh;
    m.y_sh = y_sh;
    m.shared_inter = c->shared_inter;
    m.tokens = (int)T;
    m.hidden = c->hidden;
    err = moe::launch_gate_up_shared_down(g, (int)L.max_tiles, m, st);
    if (err == hipSuccess) err = mark(tl, "routed_gate_up_shared_down", st);
  } else {
    err = moe::launch_gate_up_valu(g, (int)L.max_tiles, st);
    if (err == hipSuccess) err = mark(tl, "routed_gate_up", st);
  }
  if (err != hipSuccess) return fail_hip(err, "routed gate/up launch");

  moe::DownValuParams dv{};
  dv.h = g.h;
  dv.idx = idx;
  dv.topk_w = wts;
  dv.slot_pos = slot_pos;
  dv.dn_q = w->dn_q;
  dv.dn_s = w->dn_s;
  dv.y_shared = y_sh;
  dv.y = y;
  dv.tokens = (int)T;
  dv.top_k = c->top_k;
  dv.hidden = c->hidden;
  dv.inter = c->inter;
  dv.fp8 = g.fp8;
  err = moe::launch_down_combine_valu(dv, st);
  if (err == hipSuccess) err = mark(tl, "routed_down_combine", st);
  if (err != hipSuccess) return fail_hip(err, "down/combine launch");
  return MOE_OK;
}

// Few-token layer.  With T * k <= 64 (one-block routing):
//   1. router GEMV scores beside the shared expert's gate/up,
//   2. routing block (top-k, permutation, tiles, MXFP8 x) beside the shared down,
//   3. routed gate/up (MXFP4 x MXFP8),
//   4. routed down with the combine folded in (or down, then combine).
// Otherwise the router GEMV writes logits for the fused top-k + permute
// kernel and the shared expert gets launches of its own.
moe_status layer_forward_decode(const moe_config* c, const moe_weights* w, const uint16_t* x, int64_t T,
                                uint16_t* y, int32_t* idx, float* wts, void* ws, const WsLayout& L,
                                hipStream_t st, Timeline* tl) {
  const int E = c->n_experts;
  int32_t* sorted = at<int32_t>(ws, L.sorted);
  int32_t* slot_pos = at<int32_t>(ws, L.slot_pos);
  moe::GemmTile* tiles = at<moe::GemmTile>(ws, L.tiles);
  int32_t* tile_count = at<int32_t>(ws, L.tile_count);
  uint16_t* y_sh = c->n_shared ? at<uint16_t>(ws, L.y_sh) : nullptr;
  uint16_t* y_slot = at<uint16_t>(ws, L.y_slot);
  hipError_t err;
  moe_status s;

  uint8_t* xmx = nullptr;
  const bool valu = L.route_small && moe::decode_valu_supported((int)T, c->hidden, c->n_shared ? c->shared_inter : 0);
  if (L.route_small) {
    float* scores = at<float>(ws, L.scores);
    if (valu) {
      moe::FrontValuParams f{};
      f.x = x;
      f.router_w = w->router_w;
      f.bias = w->router_bias;
      f.scores = scores;
      f.sh_gu = c->n_shared ? w->sh_gu : nullptr;
      f.h_sh = c->n_shared ? at<uint16_t>(ws, L.h_sh) : nullptr;
      f.shared_inter = c->n_shared ? c->shared_inter : 0;
      f.tokens = (int)T;
      f.n_experts = E;
      f.hidden = c->hidden;
      f.limit = c->swiglu_limit;
      err = moe::launch_decode_front_valu(f, st);
    } else {
      moe::FrontParams f{};
      f.x = x;
      f.router_w = w->router_w;
      f.bias = w->router_bias;
      f.scores = scores;
      f.tokens = (int)T;
      f.n_experts = E;
      f.hidden = c->hidden;
      if (c->n_shared) f.shared = shared_gemv(c, w, x, T, ws, L, true, y_sh).p[0];
      f.rows_cap = (int)T;
      f.limit = c->swiglu_limit;
      f.xmx = L.valu_gu ? nullptr : at<uint8_t>(ws, L.xmx);  // converted beside the router, not in the routing block
      err = moe::launch_decode_front(f, st);
    }
    if (err == hipSuccess) err = mark(tl, "router_shared_gate_up", st);
    if (err != hipSuccess) return fail_hip(err, "router/shared gate-up launch");
    xmx = at<uint8_t>(ws, L.xmx);
    moe::RouteSmallParams rp{};
    rp.x = x;
    rp.xmx = L.valu_gu || !valu ? nullptr : xmx;  // the vector-ALU gate/up reads bf16 x; launch 1 converted it
    rp.scores = scores;
    rp.tokens = (int)T;
    rp.n_experts = E;
    rp.hidden = c->hidden;
    rp.top_k = c->top_k;
    rp.route_scale = c->route_scale;
    rp.idx = idx;
    rp.w = wts;
    rp.sorted_slots = sorted;
    rp.slot_pos = slot_pos;
    rp.tiles = tiles;
    rp.tile_count = tile_count;
    rp.tile_rows = at<int32_t>(ws, L.tile_rows);
    rp.max_tiles = (int)L.max_tiles;
    if (valu) {
      moe::MidValuParams m{};
      m.sh_dn = c->n_shared ? w->sh_dn : nullptr;
      m.h_sh = c->n_shared ? at<uint16_t>(ws, L.h_sh) : nullptr;
      m.y_sh = y_sh;
      m.shared_inter = c->n_shared ? c->shared_inter : 0;
      m.tokens = (int)T;
      m.hidden = c->hidden;
      err = moe::launch_decode_mid_valu(rp, m, st);
    } else {
      moe::GemvProblem sd{};
      if (c->n_shared) sd = shared_gemv(c, w, x, T, ws, L, false, y_sh).p[0];
      err = moe::launch_decode_mid(rp, sd, (int)T, st);
    }
    if (err == hipSuccess) err = mark(tl, "route_shared_down", st);
    if (err != hipSuccess) return fail_hip(err, "routing/shared down launch");
  } else {
    if (c->n_shared && (s = run_shared_decode(c, w, x, T, y_sh, ws, L, st, tl)) != MOE_OK) return s;
    float* logits = at<float>(ws, L.logits);
    err = moe::launch_router_gemv(x, w->router_w, logits, (int)T, E, c->hidden, nullptr, nullptr, st);
    if (err == hipSuccess) err = mark(tl, "router_logits", st);
    if (err != hipSuccess) return fail_hip(err, "router launch");
    err = moe::launch_route_permute_small(logits, 1, w->router_bias, (int)T, E, c->top_k, c->route_scale, idx, wts,
                                          nullptr, at<int32_t>(ws, L.offsets), sorted, slot_pos, L.bm,
                                          (int)L.max_tiles, tiles, tile_count, st);
    if (err == hipSuccess) err = mark(tl, "route_permute", st);
    if (err != hipSuccess) return fail_hip(err, "routing launch");
  }

  moe::GemvParams gu = routed_gemv(c, w, x, xmx, T, sorted, ws, L, true, y_slot);
  if (L.route_small) gu.p[0].tile_rows = at<int32_t>(ws, L.tile_rows);
  if (L.valu_gu) {
    moe::GateUpValuParams g{};
    g.x = x;
    g.tiles = tiles;
    g.tile_rows = at<int32_t>(ws, L.tile_rows);
    g.gu_q = w->gu_q;
    g.gu_s = w->gu_s;
    g.h = at<uint16_t>(ws, L.h);
    g.tokens = (int)T;
    g.hidden = c->hidden;
    g.inter = c->inter;
    g.limit = c->swiglu_limit;
    g.fp8 = L.fmt == moe::kWMxfp8;
    err = moe::launch_gate_up_valu(g, (int)L.max_tiles, st);
  } else {
    if (L.down_combine) gu.p[0].cmx = at<uint8_t>(ws, L.hmx);  // h in MXFP8 form for the down step
    err = moe::launch_expert_gemv(gu, true, true, st);
  }
  if (err == hipSuccess) err = mark(tl, "routed_gate_up", st);
  if (err != hipSuccess) return fail_hip(err, "routed gate/up launch");

  if (L.valu_dn) {
    moe::DownValuParams dv{};
    dv.h = at<uint16_t>(ws, L.h);
    dv.idx = idx;
    dv.topk_w = wts;
    dv.slot_pos = slot_pos;
    dv.dn_q = w->dn_q;
    dv.dn_s = w->dn_s;
    dv.y_shared = y_sh;
    dv.y = y;
    dv.tokens = (int)T;
    dv.top_k = c->top_k;
    dv.hidden = c->hidden;
    dv.inter = c->inter;
    dv.fp8 = L.fmt == moe::kWMxfp8;
    err = moe::launch_down_combine_valu(dv, st);
    if (err == hipSuccess) err = mark(tl, "routed_down_combine", st);
    if (err != hipSuccess) return fail_hip(err, "down/combine launch");
    return MOE_OK;
  }
  if (L.down_combine) {
    moe::DownCombineParams dp{};
    dp.hmx = at<uint8_t>(ws, L.hmx);
    dp.tiles = tiles;
    dp.tile_count = tile_count;
    dp.sorted_slots = sorted;
    dp.topk_w = wts;
    dp.dn_q = w->dn_q;
    dp.dn_s = w->dn_s;
    dp.y_shared = y_sh;
    dp.y = y;
    dp.tokens = (int)T;
    dp.top_k = c->top_k;
    dp.n_experts = E;
    dp.hidden = c->hidden;
    dp.inter = c->inter;
    dp.max_tiles = (int)L.max_tiles;
    err = moe::launch_down_combine(dp, st);
    if (err == hipSuccess) err = mark(tl, "routed_down_combine", st);
    if (err != hipSuccess) return fail_hip(err, "down/combine launch");
    return MOE_OK;
  }
  moe::GemvParams dn = routed_gemv(c, w, x, nullptr, T, sorted, ws, L, false, y_slot);
  if (L.route_small) dn.p[0].tile_rows = nullptr;  // down rows are the tile's own positions
  err = L.splitk_dn ? moe::launch_expert_gemv_splitk(dn.p[0], dn.rows_cap, st)
                    : moe::launch_expert_gemv(dn, false, true, st);
  if (err == hipSuccess) err = mark(tl, "routed_down", st);
  if (err != hipSuccess) return fail_hip(err, "routed down launch");
  err = moe::launch_combine(y_slot, slot_pos, wts, y_sh, (int)T, c->top_k, c->hidden, y, st);
  if (err == hipSuccess) err = mark(tl, "combine", st);
  if (err != hipSuccess) return fail_hip(err, "combine launch");
  return MOE_OK;
}

moe_status run_shared(const moe_config* c, const moe_weights* w, const uint16_t* x, int64_t T, uint16_t* y_shared,
                      void* ws, const WsLayout& L, hipStream_t st, Timeline* tl);

moe_status run_down(const moe_config* c, const moe_weights* w, int64_t T, const uint16_t* h, uint16_t* y_slot,
                    uint16_t* y_shared, const uint16_t* x, void* ws, const WsLayout& L, hipStream_t st,
                    Timeline* tl, bool shared);

// Routed gate/up + down over the tile table in ws, then (with `shared`) the
// shared expert.
moe_status run_experts(const moe_config* c, const moe_weights* w, const uint16_t* x, int64_t T,
                       const int32_t* sorted, uint16_t* y_slot, uint16_t* y_shared, void* ws, const WsLayout& L,
                       hipStream_t st, Timeline* tl, bool shared = true) {
  const int H = c->hidden, I = c->inter;
  uint16_t* h = at<uint16_t>(ws, L.h);
  // few tokens: the MFMA GEMVs (MXFP4; MXFP8 with both K multiples of 128, as
  // their 8-bit weight pieces need; other MXFP8 shapes take the grouped GEMM)
  if (L.decode && (L.fmt == moe::kWMxfp4 || (H % 128 == 0 && I % 128 == 0)))
    return run_experts_decode(c, w, x, T, sorted, y_slot, y_shared, ws, L, st, tl);
  // every grouped kernel below computes up to 16 * gemm_mt rows of a tile
  // (the MXFP6 one up to mx6_tile_rows()): a taller tile table would leave rows out
  if (L.bm > 16 * L.gemm_mt || (L.mx6 && L.bm > moe::mx6_tile_rows()))
    return fail(MOE_ERR_UNSUPPORTED, "internal: tile table taller than the grouped kernels' tiles");
  hipError_t err;
  if (L.mx6) {
    const int n = (int)(T * c->top_k);
    uint8_t* xq = at<uint8_t>(ws, L.xq);
    uint8_t* hq = at<uint8_t>(ws, L.hq);
    err = moe::launch_mx6_rows(x, H, (int)T, H, xq, st);
    if (err == hipSuccess) err = mark(tl, "mx6_x", st);
    if (err != hipSuccess) return fail_hip(err, "x to MXFP6 launch");
    moe::Mx6Params q{};
    q.tiles = at<moe::GemmTile>(ws, L.tiles);
    q.tile_count = at<int32_t>(ws, L.tile_count);
    q.w8 = L.fmt == moe::kWMxfp8;
    // gate/up: A = x records of the tile's tokens, B = W_gu[e] [2I][H], C = h [n][I]
    q.gather = sorted;
    q.gather_div = c->top_k;
    q.A = xq;
    q.a_stride = moe::mx6_bytes(1, H);
    q.a_rows = (int)T;
    q.K = H;
    q.bq = w->gu_q;
    q.bs = w->gu_s;
    q.b_expert_rows = 2 * (int64_t)I;
    q.b_row_second = I;
    q.N = I;
    q.C = h;
    q.ldc = I;
    // with the MXFP6 down projection the epilogue writes h as its records
    q.Cmx = L.mx6_dn ? hq : nullptr;
    q.ldcmx = moe::mx6_bytes(1, I);
    q.limit = c->swiglu_limit;
    err = moe::launch_expert_mx6(q, true, (int)L.max_tiles, st);
    if (err == hipSuccess) err = mark(tl, "routed_gate_up", st);
    if (err != hipSuccess) return fail_hip(err, "routed gate/up launch");
    if (!L.mx6_dn) return run_down(c, w, T, h, y_slot, y_shared, x, ws, L, st, tl, shared);
    // down: A = h records in position order, B = W_dn[e] [H][I], C = y_slot [n][H]
    q.Cmx = nullptr;
    q.gather = nullptr;
    q.A = hq;
    q.a_stride = moe::mx6_bytes(1, I);
    q.a_rows = n;
    q.K = I;
    q.bq = w->dn_q;
    q.bs = w->dn_s;
    q.b_expert_rows = H;
    q.b_row_second = 0;
    q.N = H;
    q.C = y_slot;
    q.ldc = H;
    err = moe::launch_expert_mx6(q, false, (int)L.max_tiles, st);
    if (err == hipSuccess) err = mark(tl, "routed_down", st);
    if (err != hipSuccess) return fail_hip(err, "routed down launch");
    return shared ? run_shared(c, w, x, T, y_shared, ws, L, st, tl) : MOE_OK;
  }
  moe::GemmParams p{};
  p.tiles = at<moe::GemmTile>(ws, L.tiles);
  p.tile_count = at<int32_t>(ws, L.tile_count);
  // gate/up: A = gathered token rows of x, B = W_gu[e] [2I][H], C = h [n][I]
  p.gather = sorted;
  p.gather_div = c->top_k;
  p.A = x;
  p.lda = H;
  p.a_rows = (int)T;
  p.K = H;
  p.bq = w->gu_q;
  p.bs = w->gu_s;
  p.b_expert_rows = 2 * (int64_t)I;
  p.b_row_second = I;
  p.N = I;
  p.C = h;
  p.ldc = I;
  p.limit = c->swiglu_limit;
  err = moe::launch_expert_gemm(p, true, L.fmt, L.gemm_mt, L.max_tiles, st);
  if (err == hipSuccess) err = mark(tl, "routed_gate_up", st);
  if (err != hipSuccess) return fail_hip(err, "routed gate/up launch");
  return run_down(c, w, T, h, y_slot, y_shared, x, ws, L, st, tl, shared);
}

// Routed down projection on bf16 h over the tile table, then the shared expert.
moe_status run_down(const moe_config* c, const moe_weights* w, int64_t T, const uint16_t* h, uint16_t* y_slot,
                    uint16_t* y_shared, const uint16_t* x, void* ws, const WsLayout& L, hipStream_t st,
                    Timeline* tl, bool shared) {
  const int H = c->hidden, I = c->inter;
  moe::GemmParams p{};
  p.tiles = at<moe::GemmTile>(ws, L.tiles);
  p.tile_count = at<int32_t>(ws, L.tile_count);
  p.limit = c->swiglu_limit;
  // down: A = h rows in position order, B = W_dn[e] [H][I], C = y_slot [n][H]
  p.gather = nullptr;
  p.A = h;
  p.lda = I;
  p.a_rows = (int)(T * c->top_k);
  p.K = I;
  p.bq = w->dn_q;
  p.bs = w->dn_s;
  p.b_expert_rows = H;
  p.b_row_second = 0;
  p.N = H;
  p.C = y_slot;
  p.ldc = H;
  hipError_t err = moe::launch_expert_gemm(p, false, L.fmt, L.gemm_mt, L.max_tiles, st);
  if (err == hipSuccess) err = mark(tl, "routed_down", st);
  if (err != hipSuccess) return fail_hip(err, "routed down launch");
  return shared ? run_shared(c, w, x, T, y_shared, ws, L, st, tl) : MOE_OK;
}

// The shared expert for the general path (after the routed GEMMs, or on the
// side stream beside them).
moe_status run_shared(const moe_config* c, const moe_weights* w, const uint16_t* x, int64_t T, uint16_t* y_shared,
                      void* ws, const WsLayout& L, hipStream_t st, Timeline* tl) {
  const int H = c->hidden;
  hipError_t err;
  if (c->n_shared == 1) {
    const int Is = c->shared_inter;
    uint16_t* hs = at<uint16_t>(ws, L.h_sh);
    moe::GemmParams q{};
    q.M = (int)T;
    q.A = x;
    q.lda = H;
    q.a_rows = (int)T;
    q.K = H;
    q.bh = w->sh_gu;
    q.b_expert_rows = 2 * (int64_t)Is;
    q.b_row_second = Is;
    q.N = Is;
    q.C = hs;
    q.ldc = Is;
    q.limit = c->swiglu_limit;
    float* sh_part = at<float>(ws, L.sh_part);
    err = L.shared_skinny  ? moe::launch_skinny_sliced(q, true, L.shared_ks_gu, sh_part, st)
          : L.shared_ks_gu ? moe::launch_dense_sliced(q, true, L.shared_ks_gu, sh_part, st)
                           : moe::launch_expert_gemm(q, true, moe::kWBf16, L.shared_mt, L.shared_tiles, st);
    if (err == hipSuccess) err = mark(tl, "shared_gate_up", st);
    if (err != hipSuccess) return fail_hip(err, "shared gate/up launch");
    q.A = hs;
    q.lda = Is;
    q.a_rows = (int)T;
    q.K = Is;
    q.bh = w->sh_dn;
    q.b_expert_rows = H;
    q.b_row_second = 0;
    q.N = H;
    q.C = y_shared;
    q.ldc = H;
    err = L.shared_skinny  ? moe::launch_skinny_sliced(q, false, L.shared_ks_dn, sh_part, st)
          : L.shared_ks_dn ? moe::launch_dense_sliced(q, false, L.shared_ks_dn, sh_part, st)
                           : moe::launch_expert_gemm(q, false, moe::kWBf16, L.shared_mt, L.shared_tiles, st);
    if (err == hipSuccess) err = mark(tl, "shared_down", st);
    if (err != hipSuccess) return fail_hip(err, "shared down launch");
  }
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_config* cfg, int64_t tokens) {
  if (check_config(cfg) != MOE_OK || check_tokens(tokens) != MOE_OK || check_buffer_extents(cfg, tokens) != MOE_OK)
    return 0;
  return plan_workspace(cfg, tokens).total;
}

moe_status moe_rmsnorm(const moe_config* cfg, const uint16_t* gamma, const uint16_t* x, int64_t tokens,
                       uint16_t* x_norm, void* stream) {
  moe_status s;
  if ((s = check_config(cfg)) != MOE_OK || (s = check_tokens(tokens)) != MOE_OK) return s;
  if ((s = check_norm(cfg, gamma)) != MOE_OK) return s;
  if ((s = need(x, 16, "x")) != MOE_OK || (s = need(x_norm, 16, "x_norm")) != MOE_OK) return s;
  if (tokens == 0) return MOE_OK;
  hipError_t err = moe::launch_rmsnorm_rows(x, gamma, x_norm, (int)tokens, cfg->hidden, (double)cfg->norm_eps,
                                            static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail_hip(err, "rmsnorm launch");
  return MOE_OK;
}

moe_status moe_route(const moe_config* cfg, const moe_weights* w, const uint16_t* x, int64_t tokens,
                     int32_t* topk_idx, float* topk_w, float* tie_gap, void* ws, size_t ws_bytes, void* stream) {
  moe_status s;
  if ((s = check_config(cfg)) != MOE_OK || (s = check_tokens(tokens)) != MOE_OK ||
      (s = check_buffer_extents(cfg, tokens)) != MOE_OK)
    return s;
  if ((s = check_routed_weights(cfg, w, true, false)) != MOE_OK) return s;
  if ((s = need(x, 16, "x")) != MOE_OK || (s = need(topk_idx, 4, "topk_idx")) != MOE_OK ||
      (s = need(topk_w, 4, "topk_w")) != MOE_OK)
    return s;
  if (tie_gap && !aligned(tie_gap, 4)) return fail(MOE_ERR_ALIGNMENT, "tie_gap is not 4-byte aligned");
  const WsLayout L = plan_workspace(cfg, tokens);
  if ((s = check_ws(ws, ws_bytes, L)) != MOE_OK) return s;
  if (tokens == 0) return MOE_OK;
  return run_route(cfg, w, x, tokens, topk_idx, topk_w, tie_gap, ws, L, static_cast<hipStream_t>(stream), nullptr);
}

moe_status moe_permute(const moe_config* cfg, const int32_t* topk_idx, int64_t tokens, int32_t* expert_offsets,
                       int32_t* sorted_slots, int32_t* slot_pos, void* ws, size_t ws_bytes, void* stream) {
  moe_status s;
  if ((s = check_config(cfg)) != MOE_OK || (s = check_tokens(tokens)) != MOE_OK) return s;
  if ((s = need(topk_idx, 4, "topk_idx")) != MOE_OK || (s = need(expert_offsets, 4, "expert_offsets")) != MOE_OK ||
      (s = need(sorted_slots, 4, "sorted_slots")) != MOE_OK || (s = need(slot_pos, 4, "slot_pos")) != MOE_OK)
    return s;
  const WsLayout L = plan_workspace(cfg, tokens);
  if ((s = check_ws(ws, ws_bytes, L)) != MOE_OK) return s;
  if (tokens == 0) return MOE_OK;
  return run_permute(cfg, topk_idx, tokens, expert_offsets, sorted_slots, slot_pos, ws, L, false,
                     static_cast<hipStream_t>(stream), nullptr);
}

moe_status moe_expert_ffn(const moe_config* cfg, const moe_weights* w, const uint16_t* x, int64_t tokens,
                          const int32_t* expert_offsets, const int32_t* sorted_slots, uint16_t* y_slot,
                          uint16_t* y_shared, void* ws, size_t ws_bytes, void* stream) {
  moe_status s;
  if ((s = check_config(cfg)) != MOE_OK || (s = check_tokens(tokens)) != MOE_OK ||
      (s = check_buffer_extents(cfg, tokens)) != MOE_OK)
    return s;
  if ((s = check_routed_weights(cfg, w, false, true)) != MOE_OK) return s;
  if ((s = need(x, 16, "x")) != MOE_OK || (s = need(expert_offsets, 4, "expert_offsets")) != MOE_OK ||
      (s = need(sorted_slots, 4, "sorted_slots")) != MOE_OK || (s = need(y_slot, 16, "y_slot")) != MOE_OK)
    return s;
  if (cfg->n_shared == 1) {
    if ((s = need(y_shared, 16, "y_shared")) != MOE_OK) return s;
  } else if (y_shared) {
    return fail(MOE_ERR_INVALID_ARG, "y_shared must be NULL when n_shared == 0");
  }
  const WsLayout L = plan_workspace(cfg, tokens);
  if ((s = check_ws(ws, ws_bytes, L)) != MOE_OK) return s;
  if (tokens == 0) return MOE_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t err = moe::launch_tile_table(expert_offsets, cfg->n_experts, (int)(tokens * cfg->top_k), L.bm, (int)L.max_tiles,
                                          at<moe::GemmTile>(ws, L.tiles), at<int32_t>(ws, L.tile_count), st);
  if (err != hipSuccess) return fail_hip(err, "tile table launch");
  return run_experts(cfg, w, x, tokens, sorted_slots, y_slot, y_shared, ws, L, st, nullptr);
}

moe_status moe_combine(const moe_config* cfg, const uint16_t* y_slot, const int32_t* slot_pos, const float* topk_w,
                       const uint16_t* y_shared, int64_t tokens, uint16_t* y, void* stream) {
  moe_status s;
  if ((s = check_config(cfg)) != MOE_OK || (s = check_tokens(tokens)) != MOE_OK) return s;
  if ((s = need(y_slot, 16, "y_slot")) != MOE_OK || (s = need(slot_pos, 4, "slot_pos")) != MOE_OK ||
      (s = need(topk_w, 4, "topk_w")) != MOE_OK || (s = need(y, 16, "y")) != MOE_OK)
    return s;
  if (y_shared && !aligned(y_shared, 16)) return fail(MOE_ERR_ALIGNMENT, "y_shared is not 16-byte aligned");
  if (tokens == 0) return MOE_OK;
  hipError_t err = moe::launch_combine(y_slot, slot_pos, topk_w, y_shared, (int)tokens, cfg->top_k, cfg->hidden, y,
                                       static_cast<hipStream_t>(stream));
  if (err != hipSuccess) return fail_hip(err, "combine launch");
  return MOE_OK;
}

}  // extern "C"

namespace {

// Checks of moe_layer_forward's arguments other than the workspace.
moe_status check_layer_args(const moe_config* cfg, const moe_weights* w, const uint16_t* x, int64_t tokens,
                            const uint16_t* y, const int32_t* topk_idx_out, const float* topk_w_out) {
  moe_status s;
  if ((s = check_config(cfg)) != MOE_OK || (s = check_tokens(tokens)) != MOE_OK ||
      (s = check_buffer_extents(cfg, tokens)) != MOE_OK)
    return s;
  if ((s = check_routed_weights(cfg, w, true, true)) != MOE_OK) return s;
  if ((s = need(x, 16, "x")) != MOE_OK || (s = need(y, 16, "y")) != MOE_OK) return s;
  if (w->norm_gamma && (s = check_norm(cfg, w->norm_gamma)) != MOE_OK) return s;
  if (topk_idx_out && !aligned(topk_idx_out, 4)) return fail(MOE_ERR_ALIGNMENT, "topk_idx_out is not 4-byte aligned");
  if (topk_w_out && !aligned(topk_w_out, 4)) return fail(MOE_ERR_ALIGNMENT, "topk_w_out is not 4-byte aligned");
  return MOE_OK;
}

moe_status layer_forward_impl(const moe_config* cfg, const moe_weights* w, const uint16_t* x, int64_t tokens,
                              uint16_t* y, int32_t* topk_idx_out, float* topk_w_out, void* ws, size_t ws_bytes,
                              hipStream_t st, Timeline* tl, bool side_ok) {
  moe_status s;
  if ((s = check_layer_args(cfg, w, x, tokens, y, topk_idx_out, topk_w_out)) != MOE_OK) return s;
  const WsLayout L = plan_workspace(cfg, tokens);
  if ((s = check_ws(ws, ws_bytes, L)) != MOE_OK) return s;
  if (tokens == 0) return MOE_OK;
  int32_t* idx = topk_idx_out ? topk_idx_out : at<int32_t>(ws, L.idx);
  float* wts = topk_w_out ? topk_w_out : at<float>(ws, L.w);
  int32_t* offsets = at<int32_t>(ws, L.offsets);
  int32_t* sorted = at<int32_t>(ws, L.sorted);
  int32_t* slot_pos = at<int32_t>(ws, L.slot_pos);
  const uint16_t* gamma = w->norm_gamma;
  if (gamma && L.norm_in_router) return layer_forward_decode4(cfg, w, x, tokens, y, idx, wts, ws, L, st, tl, gamma);
  if (gamma) {
    uint16_t* xn = at<uint16_t>(ws, L.x_norm);
    hipError_t err = moe::launch_rmsnorm_rows(x, gamma, xn, (int)tokens, cfg->hidden, (double)cfg->norm_eps, st);
    if (err == hipSuccess) err = mark(tl, "rmsnorm", st);
    if (err != hipSuccess) return fail_hip(err, "rmsnorm launch");
    x = xn;
  }
  if (L.stream4) return layer_forward_decode4(cfg, w, x, tokens, y, idx, wts, ws, L, st, tl, nullptr);
  if (L.decode) return layer_forward_decode(cfg, w, x, tokens, y, idx, wts, ws, L, st, tl);
  uint16_t* y_slot = at<uint16_t>(ws, L.y_slot);
  uint16_t* y_sh = cfg->n_shared ? at<uint16_t>(ws, L.y_sh) : nullptr;
  // From 17 to 512 tokens (the skinny shared-expert kernel) the shared expert
  // runs on the side stream (its inputs are x and its weights, its workspace
  // regions its own), joined before the combine: its latency-bound launches
  // then fill the CUs that the router, top-k and permutation leave idle
  // (64 tokens 905 -> 884 us, 320 tokens 1469 -> 1428 us).  With more
  // tokens it competes with the routed GEMMs for the CUs and is not faster.
  SideStream* side = nullptr;
  std::unique_lock<std::mutex> side_lock;
  int dev = -1;
  if (side_ok && !tl && cfg->n_shared && L.shared_skinny && hipGetDevice(&dev) == hipSuccess && dev >= 0 &&
      dev < kMaxDevices) {
    // the side stream is the current device's: a caller's stream of another
    // device keeps the single-stream order
    hipDevice_t sdev = dev;
    if (!st || (hipStreamGetDevice(st, &sdev) == hipSuccess && (int)sdev == dev)) {
      side_lock = std::unique_lock<std::mutex>(g_side_mu[dev]);
      side = side_stream(dev, st);
    }
  }
  hipError_t err;
  if (side) {
    if ((err = hipEventRecord(side->fork, st)) != hipSuccess) return fail_hip(err, "hipEventRecord(fork)");
    if ((err = hipStreamWaitEvent(side->st, side->fork, 0)) != hipSuccess)
      return fail_hip(err, "hipStreamWaitEvent(fork)");
    if ((s = run_shared(cfg, w, x, tokens, y_sh, ws, L, side->st, nullptr)) != MOE_OK) return s;
    if ((err = hipEventRecord(side->join, side->st)) != hipSuccess) return fail_hip(err, "hipEventRecord(join)");
  }
  if ((s = run_route(cfg, w, x, tokens, idx, wts, nullptr, ws, L, st, tl)) != MOE_OK) return s;
  if ((s = run_permute(cfg, idx, tokens, offsets, sorted, slot_pos, ws, L, true, st, tl)) != MOE_OK) return s;
  if ((s = run_experts(cfg, w, x, tokens, sorted, y_slot, y_sh, ws, L, st, tl, !side)) != MOE_OK) return s;
  if (side && (err = hipStreamWaitEvent(st, side->join, 0)) != hipSuccess) return fail_hip(err, "hipStreamWaitEvent(join)");
  err = moe::launch_combine(y_slot, slot_pos, wts, y_sh, (int)tokens, cfg->top_k, cfg->hidden, y, st);
  if (err == hipSuccess) err = mark(tl, "combine", st);
  if (err != hipSuccess) return fail_hip(err, "combine launch");
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_layer_forward(const moe_config* cfg, const moe_weights* w, const uint16_t* x, int64_t tokens,
                             uint16_t* y, int32_t* topk_idx_out, float* topk_w_out, void* ws, size_t ws_bytes,
                             void* stream) {
  return layer_forward_impl(cfg, w, x, tokens, y, topk_idx_out, topk_w_out, ws, ws_bytes,
                            static_cast<hipStream_t>(stream), nullptr, true);
}

moe_status moe_layer_forward_noalloc(const moe_config* cfg, const moe_weights* w, const uint16_t* x, int64_t tokens,
                                     uint16_t* y, int32_t* topk_idx_out, float* topk_w_out, void* stream) {
  moe_status s;
  if ((s = check_layer_args(cfg, w, x, tokens, y, topk_idx_out, topk_w_out)) != MOE_OK) return s;
  const size_t need = plan_workspace(cfg, tokens).total;
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES) {
    static thread_local char buf[200];
    std::snprintf(buf, sizeof(buf), "this shape needs %zu bytes of scratch, more than the %u the no-allocation entry "
                  "point holds; call moe_layer_forward with a workspace", need, (unsigned)MOE_NOALLOC_SCRATCH_BYTES);
    return fail(MOE_ERR_UNSUPPORTED, buf);
  }
  if (tokens == 0) return MOE_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return fail_hip(err, "hipGetDevice");
  if (st) {
    hipDevice_t sdev = -1;
    if ((err = hipStreamGetDevice(st, &sdev)) != hipSuccess) return fail_hip(err, "hipStreamGetDevice");
    if ((int)sdev != dev) return fail(MOE_ERR_INVALID_ARG, "stream belongs to a device other than the current one");
  }
  void* ws = nullptr;
  if ((s = scratch_ptr(dev, &ws)) != MOE_OK) return s;
  return layer_forward_impl(cfg, w, x, tokens, y, topk_idx_out, topk_w_out, ws, (size_t)MOE_NOALLOC_SCRATCH_BYTES,
                            st, nullptr, false);
}

moe_status moe_layer_forward_timed(const moe_config* cfg, const moe_weights* w, const uint16_t* x, int64_t tokens,
                                   uint16_t* y, void* ws, size_t ws_bytes, void* stream, float* kernel_ms,
                                   const char** kernel_names, int32_t max_kernels, int32_t* n_kernels) {
  if (!kernel_ms || !kernel_names || !n_kernels || max_kernels < 0)
    return fail(MOE_ERR_INVALID_ARG, "kernel_ms, kernel_names and n_kernels are required");
  *n_kernels = 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  Timeline tl;
  int created = 0;
  hipError_t err = hipSuccess;
  for (; created <= Timeline::kMax && err == hipSuccess; ++created) err = hipEventCreate(&tl.ev[created]);
  moe_status s = MOE_OK;
  if (err != hipSuccess) {
    --created;
    s = fail_hip(err, "hipEventCreate");
  } else if ((err = hipEventRecord(tl.ev[0], st)) != hipSuccess) {
    s = fail_hip(err, "hipEventRecord");
  } else {
    s = layer_forward_impl(cfg, w, x, tokens, y, nullptr, nullptr, ws, ws_bytes, st, &tl, false);
    if (s == MOE_OK && tl.n > 0 && (err = hipEventSynchronize(tl.ev[tl.n])) != hipSuccess)
      s = fail_hip(err, "hipEventSynchronize");
    if (s == MOE_OK) {
      for (int i = 0; i < tl.n && i < max_kernels; ++i) {
        float ms = 0.f;
        if ((err = hipEventElapsedTime(&ms, tl.ev[i], tl.ev[i + 1])) != hipSuccess) {
          s = fail_hip(err, "hipEventElapsedTime");
          break;
        }
        kernel_ms[i] = ms;
        kernel_names[i] = tl.names[i];
      }
      *n_kernels = tl.n;
    }
  }
  for (int i = 0; i < created; ++i) (void)hipEventDestroy(tl.ev[i]);
  return s;
}

const char* moe_status_str(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported";
    case MOE_ERR_ALIGNMENT: return "misaligned pointer";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

int32_t moe_abi_version(void) { return MOE_FFN_ABI_VERSION; }

}  // extern "C"
