/*
 * gla_plan.h -- launch-plan controls of libgla's chunked forward and backward.
 *
 * For tests and tuning sweeps.  The calls of gla.h choose their launch plan
 * from the sizes alone; the calls here run the same kernels with parts of
 * that choice fixed by the caller, so that every plan can be exercised and
 * timed on any size.  Results agree with gla.h's within rounding (plans group
 * the same fp32 sums differently).  The method and every argument shared with
 * gla.h are as described there (Laplace 3B post, sections "Challenge 1" and
 * "Challenge 3"; plans split a sequence as the "only the state update is
 * sequential" structure of the chunked form allows).
 */
#ifndef GLA_PLAN_H
#define GLA_PLAN_H

#include "gla.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * A launch plan; each field 0 (chain: -1) leaves that choice to the library.
 *   segments  sequence segments run in parallel, 1 .. 16 (a state-only
 *             prologue per segment, a scan over segments, then the chunks of
 *             every segment from its start state)
 *   chain     bf16 forward: 0 = the segment split above; 1 = the tiled state
 *             chain (every chunk's start state, then one output workgroup per
 *             chunk), used where it can run (2 .. 64 chunks); 256-token chunks
 *             always run in the chain form (two output workgroups per chunk)
 *   psub      1 = one prologue workgroup per segment (the library may run the
 *             bf16 prologue over half-length sub-segments instead)
 *   scan      -1 = the library's choice; 0 = a scan launch turns the segments'
 *             local states into start states; 1 = (bf16, at most 2 local states
 *             before the last segment) no scan launch: each segment folds them
 *             into its start state in the scan's order, with the same bits
 * Out-of-range fields give GLA_ERR_INVALID_ARG (size queries: 0).
 */
typedef struct {
    int segments;
    int chain;
    int psub;
    int scan;
} gla_plan;

/*
 * The plan a forward over these sizes runs with hint `hint` (NULL = none):
 * out->segments = segments used, out->chain = 0/1, out->psub = prologue
 * sub-segments per segment (1 or 2), out->scan = 1 if the segment scan is
 * folded into the segments (0 if launched or not needed).  The backward splits its state chains
 * into the same segments.  Errors as gla_fwd_workspace_bytes' sizes, plus a
 * NULL out.
 */
gla_status gla_plan_resolve(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk,
                            const gla_plan* hint, gla_plan* out);

/* Workspace of the planned calls below (bytes; 0 for invalid sizes or plans).
 * saved_states != 0: the backward reads states saved by the forward. */
size_t gla_fwd_workspace_bytes_planned(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk,
                                       const gla_plan* plan);
size_t gla_bwd_workspace_bytes_planned(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk,
                                       int saved_states, const gla_plan* plan);

/*
 * gla_fwd_chunked with every option: `states` != NULL saves every chunk's
 * start state (gla_fwd_chunked_states); `ep` != NULL applies the mixer
 * epilogue with gate `g`, o then receiving y (gla_fwd_chunked_epilogue); the
 * two options do not combine (GLA_ERR_UNSUPPORTED).
 */
gla_status gla_fwd_chunked_planned(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk,
                                   const void* q, const void* k, const void* v,
                                   const float* lambda, const float* S0, float scale,
                                   void* o, float* S_final, void* states,
                                   const void* g, const gla_epilogue_params* ep,
                                   const gla_strides* st, const gla_plan* plan,
                                   void* ws, size_t ws_bytes, void* stream);

/* gla_bwd_chunked, or gla_bwd_chunked_states when `states` != NULL. */
gla_status gla_bwd_chunked_planned(gla_dtype dtype, int B, int T, int H, int dk, int dv, int chunk,
                                   const void* q, const void* k, const void* v,
                                   const float* lambda, const float* S0, float scale,
                                   const void* d_o, const float* dS_final, const void* states,
                                   void* dq, void* dk_out, void* dv_out,
                                   float* dlambda, float* dS0, const gla_strides* st,
                                   const gla_plan* plan, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GLA_PLAN_H */
