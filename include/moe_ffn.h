/*
 * moe_ffn.h -- C ABI of the routed mixture-of-experts FFN layer of
 * DeepSeek-V4.1-Flash on AMD Instinct MI355X (gfx950).
 *
 * The layer (max.pipelines.architectures.deepseekV41 API reference,
 * DeepseekV41Config; checkpoint config.json on the "DeepSeek V4.1" atlas page):
 *   a router over E routed experts with the "sqrtsoftplus" score function,
 *   top-k selection, k weights renormalised and scaled by route_scale;
 *   gated-MLP (SwiGLU) experts with swiglu_limit; one always-on shared expert;
 *   routed experts stored as MXFP4 and the rest as BF16 (Strata DEEPSEEK41
 *   notes, opening paragraph).  With T tokens and hidden size H:
 *
 *     l[t,e]  = sum_h x[t,h] * W_r[e,h]                     (fp32 accumulate)
 *     s[t,e]  = sqrt(log(1 + exp(l[t,e])))
 *     u[t,e]  = s[t,e] + bias[e]             (bias optional, selection only)
 *     idx[t]  = the k experts of largest u, ties to the lower index,
 *               ordered by u descending
 *     w[t,j]  = route_scale * s[t,idx_j] / sum_j' s[t,idx_j']
 *     h       = silu(min(x W_g^T, L)) * clamp(x W_u^T, -L, L)
 *     o_e     = h W_d^T
 *     y[t]    = o_shared(x[t]) + sum_j w[t,j] * o_{idx_j}(x[t])
 *
 *   With a norm gain gamma (moe_weights.norm_gamma non-NULL), the layer
 *   first replaces each row by its RMSNorm (eps = moe_config.norm_eps,
 *   1e-20 in DeepseekV41Config's rms_norm_eps and config.json's norm_eps):
 *     x[t,h] <- bf16( x[t,h] / sqrt(mean_h' x[t,h']^2 + eps) * gamma[h] )
 *   rounded once, to nearest even.  The norm type is not disclosed on the
 *   'DeepSeek-V4.1-Flash' architecture sheet; RMSNorm is the reading taken.
 *
 * Conventions that hold for every entry point:
 *
 *   Memory.  Every tensor pointer is a DEVICE pointer owned by the caller
 *   (for instance the data pointer of a torch tensor); the library never
 *   allocates device memory, frees or synchronises (moe_layer_forward
 *   creates one side stream and two events per device, once: see there).
 *   Config and weight structs are host memory, read only during the call.
 *   Scratch memory comes from the caller's workspace `ws` of `ws_bytes`
 *   bytes, at least moe_workspace_bytes(cfg, tokens).
 *
 *   Layout.  Row-major, the contracted dimension contiguous.  bf16 travels as
 *   its 16-bit pattern (uint16_t).  MXFP4 matrices [R][K] are two arrays:
 *   codes uint8 [R][K/2], E2M1 element 2i in the low nibble of byte i and
 *   element 2i+1 in the high nibble; scales uint8 [R][K/32], an E8M0 byte
 *   (value 2^(s-127)) for each 32 consecutive elements of a row.  MXFP8
 *   matrices (expert_format 1) are the same with one E4M3 code per byte:
 *   codes uint8 [R][K], E4M3 "fn" (bias 7, no infinities, 0x7F/0xFF NaN;
 *   float8_e4m3fn in the MAX API's SUPPORTED_ENCODINGS).  Expert e of a
 *   stacked tensor starts at e * (rows * row_bytes).
 *
 *   Streams.  `stream` is a hipStream_t passed as void*; NULL is the default
 *   stream.  Work is enqueued asynchronously; results are valid once the
 *   stream reaches that point.  Calls that share a workspace must be ordered
 *   on one stream.
 *
 *   Errors.  Arguments are checked on the host before anything is enqueued;
 *   a failed check returns its code and enqueues nothing.  Checked: non-null
 *   required pointers; 16-byte alignment of tensor pointers (4-byte for the
 *   int32/fp32 per-token arrays; 256-byte for ws); H, I and I_s positive
 *   multiples of 32, at most 65536; 1 <= E <= 1024; 1 <= k <= min(E, 16);
 *   n_shared in {0, 1}; score_func == 0; expert_format in {0, 1}; route_scale finite;
 *   swiglu_limit > 0 (may be +inf); 0 <= tokens <= 2^22; ws_bytes large
 *   enough.  Some kernels address a matrix through a 32-bit buffer
 *   descriptor, so every one of these must stay below 2^31 - 16 bytes:
 *   x [T][H] and h [T*k][I] bf16 (the routed inner activations, T*k*I*2
 *   bytes), the shared expert's [T][I_s] bf16 activations, one routed
 *   expert's gate/up or down codes, the shared gate/up and down matrices and
 *   the router matrix; a call that would pass this limit returns
 *   MOE_ERR_UNSUPPORTED (at H 5120, I 2304, k 6: at most 77,672 tokens a
 *   call; split larger batches).  tokens == 0 returns MOE_OK and enqueues
 *   nothing.  A failed
 *   kernel launch returns MOE_ERR_HIP.  Data are not checked: NaN/Inf
 *   inputs, E8M0 byte 0xFF, expert ids outside [0, E) or an offset table
 *   that is not a permutation give unspecified values, but every access
 *   stays inside the buffers described here.
 *   moe_last_error() describes the last failure of the calling thread.
 */
#ifndef MOE_FFN_H
#define MOE_FFN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_FFN_ABI_VERSION 2

typedef enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* null pointer, bad size or value            */
  MOE_ERR_UNSUPPORTED = 2,  /* valid in principle, not supported here      */
  MOE_ERR_ALIGNMENT = 3,    /* a pointer is not aligned as required        */
  MOE_ERR_WORKSPACE = 4,    /* ws is NULL or ws_bytes is too small         */
  MOE_ERR_HIP = 5           /* a HIP runtime call or launch failed         */
} moe_status;

/* Layer shape and constants (DeepseekV41Config: hidden_size,
 * n_routed_experts, num_experts_per_tok, moe_intermediate_size,
 * n_shared_experts, routed_scaling_factor, swiglu_limit; config.json:
 * score_func, route_scale). */
typedef struct moe_config {
  int32_t hidden;        /* H: 5120 */
  int32_t n_experts;     /* E: 384 */
  int32_t top_k;         /* k: 6 */
  int32_t inter;         /* I: routed expert width, 2304 */
  int32_t n_shared;      /* 0 or 1 */
  int32_t shared_inter;  /* I_s: shared expert width, 2304 (ignored if n_shared == 0) */
  float route_scale;     /* rho: 1.5, multiplies the routed weights only */
  float swiglu_limit;    /* L: 10.0 */
  int32_t score_func;    /* 0 = sqrtsoftplus (the only one) */
  float norm_eps;        /* eps of the pre-FFN RMSNorm, 1e-20; read only when a norm gain is given,
                            then finite and > 0 */
  int32_t expert_format; /* routed expert weights: 0 = MXFP4 (E2M1 codes, two a byte),
                            1 = MXFP8 (E4M3 "fn" codes, one a byte); E8M0 scale per 32 either way */
} moe_config;

/* Weights: device pointers, layouts as in the header comment. */
typedef struct moe_weights {
  const float* router_w;     /* [E][H] fp32                                      */
  const float* router_bias;  /* [E] fp32 selection bias, or NULL for none         */
  const uint8_t* gu_q;       /* [E][2I][H/2]  MXFP4 codes ([E][2I][H] MXFP8); rows 0..I-1 gate, */
  const uint8_t* gu_s;       /* [E][2I][H/32] E8M0 scales; rows I..2I-1 up        */
  const uint8_t* dn_q;       /* [E][H][I/2]   MXFP4 codes ([E][H][I] MXFP8) of the down projection */
  const uint8_t* dn_s;       /* [E][H][I/32]  E8M0 scales                         */
  const uint16_t* sh_gu;     /* [2I_s][H] bf16, gate rows then up rows; NULL iff n_shared == 0 */
  const uint16_t* sh_dn;     /* [H][I_s] bf16; NULL iff n_shared == 0             */
  const uint16_t* norm_gamma; /* [H] bf16 gain of the pre-FFN RMSNorm, or NULL: no norm.
                                 Read by moe_layer_forward only. */
} moe_weights;

/* Bytes of workspace every entry point below needs for `tokens` tokens
 * (the maximum over them).  Returns 0 for an invalid config, or for a token
 * count past the buffer limit stated under Errors. */
size_t moe_workspace_bytes(const moe_config* cfg, int64_t tokens);

/* Pre-FFN RMSNorm of T rows: x_norm[t] = bf16(x[t] / sqrt(mean(x[t]^2) + eps)
 * * gamma), eps = cfg->norm_eps, rounded once to nearest even (the layer
 * formula above).  x, x_norm: bf16 [T][H]; gamma: bf16 [H].  x_norm may be
 * x itself (in place); other overlaps are unspecified.  Needs no workspace.
 * Checked as above, plus: gamma non-NULL and 16-byte aligned, norm_eps
 * finite and > 0.  The other entry points take x as given: to run them on
 * normalised rows, call this first (moe_layer_forward does it itself). */
moe_status moe_rmsnorm(const moe_config* cfg, const uint16_t* gamma, const uint16_t* x, int64_t tokens,
                       uint16_t* x_norm, void* stream);

/* Router: logits, sqrtsoftplus scores, top-k, weights.
 * x: bf16 [T][H].  Outputs: topk_idx int32 [T][k] in selection order,
 * topk_w fp32 [T][k], tie_gap fp32 [T] = u(k) - u(k+1) (+inf if k == E),
 * nullable.  Score function: config.json score_func "sqrtsoftplus"
 * ("DeepSeek V4.1" atlas page); k: num_experts_per_tok; scale:
 * routed_scaling_factor (DeepseekV41Config). */
moe_status moe_route(const moe_config* cfg, const moe_weights* w, const uint16_t* x, int64_t tokens,
                     int32_t* topk_idx, float* topk_w, float* tie_gap,
                     void* ws, size_t ws_bytes, void* stream);

/* Permutation of the T*k (token, slot) pairs into expert-contiguous order:
 * a stable counting sort of flat slot f = t*k + j by expert topk_idx[f].
 * Outputs: expert_offsets int32 [E+1] (start of each expert's run, last
 * entry T*k), sorted_slots int32 [T*k] (flat slot at each position,
 * ascending within an expert), slot_pos int32 [T*k] (inverse). */
moe_status moe_permute(const moe_config* cfg, const int32_t* topk_idx, int64_t tokens,
                       int32_t* expert_offsets, int32_t* sorted_slots, int32_t* slot_pos,
                       void* ws, size_t ws_bytes, void* stream);

/* Expert FFNs.  For each position p in expert e's run (flat slot
 * f = sorted_slots[p], token t = f / k): y_slot[p] = o_e(x[t]) as bf16
 * [T*k][H], computed with the MXFP4 (or, by expert_format, MXFP8) gated
 * MLP of expert e (clamped SwiGLU, "experts are gated MLPs":
 * 'DeepSeek-V4.1-Flash' architecture sheet).
 * If n_shared == 1, also y_shared[t] = o_shared(x[t]) as bf16 [T][H]
 * (BF16 weights, same clamp); y_shared must be NULL iff n_shared == 0.
 * expert_offsets and sorted_slots as produced by moe_permute. */
moe_status moe_expert_ffn(const moe_config* cfg, const moe_weights* w, const uint16_t* x, int64_t tokens,
                          const int32_t* expert_offsets, const int32_t* sorted_slots,
                          uint16_t* y_slot, uint16_t* y_shared,
                          void* ws, size_t ws_bytes, void* stream);

/* Combine: y[t] = y_shared[t] + sum_{j<k} topk_w[t][j] * y_slot[slot_pos[t*k+j]]
 * with the j terms added in order, in fp32, rounded once to bf16 [T][H].
 * y_shared may be NULL (no shared expert). */
moe_status moe_combine(const moe_config* cfg, const uint16_t* y_slot, const int32_t* slot_pos,
                       const float* topk_w, const uint16_t* y_shared, int64_t tokens,
                       uint16_t* y, void* stream);

/* The whole layer: y bf16 [T][H] from x bf16 [T][H], with the RMSNorm in
 * front when w->norm_gamma is non-NULL (then norm_eps is checked as for
 * moe_rmsnorm; x itself is not modified).  topk_idx_out [T][k] and
 * topk_w_out [T][k] receive the routing when non-NULL.
 * From 17 to 512 tokens the shared expert's launches go to a side stream
 * that the library holds per device (created, at default priority, with its
 * two events by the first such call that is not under graph capture; until
 * then, under capture without it, and when `stream` belongs to another
 * device than the current one, one stream serves): an event recorded
 * on `stream` orders them after the caller's earlier work, and `stream`
 * waits for them before the combine, so every result is in `stream`'s order
 * as above and a capture of `stream` holds both branches. */
moe_status moe_layer_forward(const moe_config* cfg, const moe_weights* w, const uint16_t* x, int64_t tokens,
                             uint16_t* y, int32_t* topk_idx_out, float* topk_w_out,
                             void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * layer as moe_layer_forward, with the same arguments minus the workspace.
 * Its scratch memory is a device array of MOE_NOALLOC_SCRATCH_BYTES (16 MiB)
 * inside the library, one per GPU, which each GPU the library runs on holds
 * until the process ends; the call allocates nothing.  Shapes whose
 * moe_workspace_bytes exceeds that return MOE_ERR_UNSUPPORTED before
 * anything is enqueued (at the full layer shape, up to about 120 tokens a
 * call fit).  Every call on a GPU shares that GPU's array, which keeps the
 * last call's contents (no kernel reads scratch it has not written in the
 * same call): calls that overlap on one GPU -- on different streams, or
 * from several threads -- race and give unspecified results; order them on
 * one stream.  `stream` must belong to the calling thread's current device
 * (else MOE_ERR_INVALID_ARG); the first call on a device looks up that
 * device's copy of the array (a failure returns MOE_ERR_HIP). */
#define MOE_NOALLOC_SCRATCH_BYTES (16u << 20)
moe_status moe_layer_forward_noalloc(const moe_config* cfg, const moe_weights* w, const uint16_t* x, int64_t tokens,
                                     uint16_t* y, int32_t* topk_idx_out, float* topk_w_out, void* stream);

/* Static description of a status code. */
const char* moe_status_str(moe_status s);

/* Description of the calling thread's last failed call ("" if none). */
const char* moe_last_error(void);

/* MOE_FFN_ABI_VERSION of the built library. */
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FFN_H */
