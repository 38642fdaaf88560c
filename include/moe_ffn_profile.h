/*
 * moe_ffn_profile.h -- kernel-level timing of the MoE FFN layer, for
 * profiling tools and benchmarks.  Not part of the layer's contract in
 * moe_ffn.h: unlike every call declared there, the call below creates HIP
 * events and WAITS for its stream.
 *
 * Types, layouts, argument checks and error codes are those of moe_ffn.h.
 */
#ifndef MOE_FFN_PROFILE_H
#define MOE_FFN_PROFILE_H

#include "moe_ffn.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Kernel-level timing of moe_layer_forward (the layer formula of moe_ffn.h):
 * enqueues the same kernels with the same launch configuration on `stream`,
 * with a HIP event recorded before the first kernel and after each one,
 * then WAITS for the stream to reach the last event.  kernel_ms[i] receives
 * the time between the events around kernel i, kernel_names[i] a static
 * string naming it; at most max_kernels entries are written and *n_kernels
 * receives the number of kernels launched.  Routing outputs are not
 * returned.  Creates and destroys its own events.  kernel_ms, kernel_names
 * and n_kernels must be non-NULL and max_kernels >= 0 (else
 * MOE_ERR_INVALID_ARG); the other arguments are checked as for
 * moe_layer_forward. */
moe_status moe_layer_forward_timed(const moe_config* cfg, const moe_weights* w, const uint16_t* x, int64_t tokens,
                                   uint16_t* y, void* ws, size_t ws_bytes, void* stream, float* kernel_ms,
                                   const char** kernel_names, int32_t max_kernels, int32_t* n_kernels);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FFN_PROFILE_H */
