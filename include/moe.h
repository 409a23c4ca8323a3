/*
 * moe.h -- C ABI of the MI355X (gfx950) sparse-MoE FFN forward of GLM-4.5 / GLM-5.
 *
 * What the layer computes (pages as titled):
 *  - "Group Router" (GLM-4.5), How it works: s = sigmoid(x W_g^T), a bias-free
 *    gate evaluated in float32; s' = s + b, the correction bias used only to
 *    choose experts; G contiguous groups scored by the sum of their two largest
 *    s'; the topk_group best groups kept; the top-k experts by s' inside them;
 *    weights w = alpha * s / (sum over the chosen of s + eps) from the raw s
 *    (w = alpha * s without norm_topk_prob).
 *  - "MoE Forward" (GLM-4.5), How it works: each routed expert is a bias-free
 *    SwiGLU, E_i(x) = W_down (SiLU(W_gate x) * W_up x), with gate and up packed
 *    as one (2 d, D) matrix; y_n = sum over the chosen of w E_i(x_n) + E_sh(x_n);
 *    alpha scales only the routed sum; every token uses exactly k routed
 *    experts plus the shared one.
 *  - "GLM-5 . Mixture of experts" and "Shared output": the module layout (router,
 *    routed experts, one shared MLP of width n_shared * d) and the per-expert
 *    token lists that dispatch builds; the expert loop skips the id E, which
 *    marks an empty slot in routing given by the caller.
 *  - "Module 02 -- MoE: Capacity, Work, and Traffic", section 3: the clamped
 *    SwiGLU of that checkpoint (swiglu_limit below).
 *
 * Conventions for every call:
 *  - Buffers: all tensor pointers are device pointers (HBM), row-major and
 *    contiguous, 16-byte aligned, owned by the caller. The library allocates
 *    nothing and frees nothing on these calls; scratch space is the caller's
 *    `workspace` of at least moe_workspace_size() bytes. Calls that may run at
 *    the same time (on different streams) need separate workspaces.
 *  - Streams: `stream` is a hipStream_t (NULL = the null stream). Every call
 *    enqueues its kernels on it and returns without synchronising.
 *  - Errors: configuration and argument errors are detected on the host before
 *    anything is launched and returned as a status; a failed launch returns
 *    MOE_ERR_HIP. No exception crosses the ABI.
 *  - N = 0 is valid and launches nothing (moe_dispatch: one small kernel that zeroes counts and
 *    offsets).
 *  - Inputs must be finite. Router weight, bias, scores and mixture weights are
 *    float32 whatever `dtype` says; indices are int32.
 *  - Readings where the pages are open: discarded groups are excluded from the
 *    top-k; ties go to the lower expert / group index (IEEE comparison, so +0
 *    equals -0); the k slots are in (s' descending, index ascending) order, and
 *    that order fixes the summation order of the weight denominator; alpha is
 *    applied once, inside the weights unless alpha_on_output moves it to the
 *    routed sum; eps is added to the denominator as a float32 (1e-20 rounds to
 *    9.99999968e-21).
 */
#ifndef SPARSE_MOE_LAYER_GATE_AMD_MOE_H
#define SPARSE_MOE_LAYER_GATE_AMD_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* a config field, size or pointer is invalid */
  MOE_ERR_UNSUPPORTED = 2, /* valid per the pages, not supported by these kernels (see moe_check_config) */
  MOE_ERR_WORKSPACE = 3,   /* workspace missing or smaller than moe_workspace_size() */
  MOE_ERR_HIP = 4          /* a HIP launch or runtime call failed */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* The router / expert fields of the model config ("Group Router": n_group, topk_group,
 * num_experts_per_tok, norm_topk_prob, routed_scaling_factor; "MoE Forward": moe_intermediate_size,
 * n_shared_experts). */
typedef struct {
  int32_t hidden_size;           /* D: multiple of 64 */
  int32_t n_routed_experts;      /* E: 1..512 */
  int32_t n_group;               /* G: divides E, 1..64; E/G >= 2 when G > 1 */
  int32_t topk_group;            /* 1..G */
  int32_t num_experts_per_tok;   /* k: 1..32 and k <= topk_group * E / G */
  int32_t moe_intermediate_size; /* d: multiple of 64 */
  int32_t n_shared_experts;      /* >= 0; the shared MLP has width d * n_shared_experts */
  float routed_scaling_factor;   /* alpha */
  int32_t norm_topk_prob;        /* 0 or 1 */
  float eps;                     /* added to the weight denominator (1e-20 on the pages) */
  int32_t dtype;                 /* moe_dtype of x, the expert weights and y */
  /* Where alpha goes ("MoE Forward", Official code: inside the router or on the routed output, never
   * both). 0: w = alpha * s / (sum s + eps). 1: w = s / (sum s + eps), and the combine multiplies the
   * routed sum by alpha before adding the shared expert. */
  int32_t alpha_on_output;
  /* Clamped SwiGLU ("Module 02 -- MoE: Capacity, Work, and Traffic", section 3), in every expert, routed
   * and shared: with L = swiglu_limit > 0, gate = min(gate, L) (no lower bound) and
   * up = min(max(up, -L), L) before SiLU(gate) * up. 0: plain SwiGLU. Finite and >= 0. */
  float swiglu_limit;
} moe_config;

/* Device pointers to the layer's weights, in the pages' canonical layouts. */
typedef struct {
  const float* w_router; /* [E, D] float32 */
  const float* e_bias;   /* [E] float32 correction bias (selection only) */
  const void* gate_up;   /* [E, 2d, D]: rows [0, d) gate, rows [d, 2d) up */
  const void* down;      /* [E, D, d] */
  const void* sh_gate;   /* [d_sh, D]; NULL iff n_shared_experts == 0 */
  const void* sh_up;     /* [d_sh, D] */
  const void* sh_down;   /* [D, d_sh] */
  /* NULL, or moe_router_prepare's output for w_router (bf16 layers): the forward then reads it and skips
   * splitting w_router on every call; w_router is not read and may be NULL. */
  const void* w_router_prepared;
} moe_weights;

/* moe_route flags. */
#define MOE_ROUTE_SCORES_IN 1u  /* read the float32 scores s [N, E] from `scores`; skip the gate GEMM */
#define MOE_ROUTE_SCORES_OUT 2u /* also write s [N, E] to `scores` (without it `scores` may be NULL) */
#define MOE_ROUTE_PREPARED 4u   /* `w_router` is moe_router_prepare's output, not the float32 weight */

/* Host only. MOE_OK if the config is valid and these kernels support it; otherwise
 * MOE_ERR_INVALID_ARG (not a valid layer) or MOE_ERR_UNSUPPORTED (outside the limits above). */
moe_status moe_check_config(const moe_config* cfg);

/* Host only. Bytes of workspace moe_forward, moe_forward_routed and moe_route need for N tokens (0 for
 * an invalid config): the most any batch of at most N tokens needs, so the size never falls as N grows
 * and a workspace sized for the largest batch serves every smaller one. */
size_t moe_workspace_size(const moe_config* cfg, int64_t N);

/* Host only. Bytes of workspace moe_dispatch needs for N tokens: per-chunk counts for batches of more
 * than 256 tokens, 0 below (one kernel, no scratch). Never falls as N grows. */
size_t moe_dispatch_workspace_size(const moe_config* cfg, int64_t N);

/* Host only. Bytes of the prepared router weight of a bf16 layer: 3 * E * D * 2 (0 for float32 layers,
 * which use w_router as given, or an invalid config). */
size_t moe_router_prepared_size(const moe_config* cfg);

/* Prepare the router weight of a bf16 layer once, for calls that would otherwise split it every time
 * ("Group Router", How it works: the gate is evaluated in float32; the bf16 gate GEMM runs it as three
 * exact bf16 pieces). prepared [3, E, D] bf16 (caller-owned, >= moe_router_prepared_size bytes) receives
 * hi, mid and lo with hi + mid + lo == w_router exactly, each the bf16 rounding of what the pieces before
 * it leave. Pass it as moe_weights.w_router_prepared or to moe_route with MOE_ROUTE_PREPARED; run it
 * again whenever w_router changes. MOE_ERR_INVALID_ARG for float32 layers. Asynchronous on `stream`. */
moe_status moe_router_prepare(const moe_config* cfg, const float* w_router, void* prepared, size_t bytes,
                              void* stream);

/* Router: gate GEMM + sigmoid, then group-restricted top-k and mixture weights ("Group Router").
 *   x        [N, D] of cfg->dtype (ignored with MOE_ROUTE_SCORES_IN)
 *   w_router [E, D] float32, or with MOE_ROUTE_PREPARED the [3, E, D] bf16 output of moe_router_prepare
 *            (ignored with MOE_ROUTE_SCORES_IN)
 *   e_bias   [E] float32
 *   scores   [N, E] float32: read (MOE_ROUTE_SCORES_IN), written (MOE_ROUTE_SCORES_OUT), or unused and
 *            may be NULL (neither flag). SCORES_IN excludes the other two flags.
 *   topk_idx [N, k] int32 out: the chosen experts in slot order
 *   topk_w   [N, k] float32 out: their weights, alpha included (unless alpha_on_output)
 *   workspace, ws_bytes: scratch of at least moe_workspace_size(cfg, N) bytes (unused, may be NULL,
 *            with MOE_ROUTE_SCORES_IN)
 * The logits are float32 dot products (bf16 activations: exact products of x with an exact three-piece
 * bf16 split of w_router, accumulated in float32: on the matrix cores, or with fused multiply-adds for
 * batches of one to four tokens). Given the same float32 scores,
 * indices and weights are bit-identical to a float32 evaluation in the order stated above (correctly
 * rounded add, divide and multiply). */
moe_status moe_route(const moe_config* cfg, int64_t N, const void* x, const void* w_router, const float* e_bias,
                     float* scores, uint32_t flags, int32_t* topk_idx, float* topk_w, void* workspace,
                     size_t ws_bytes, void* stream);

/* Token-choice dispatch: per-expert token lists in the per-expert loop form of "GLM-5 . Mixture of
 * experts", as counts, an exclusive scan and a stable placement (tokens ascending inside each expert).
 *   topk_idx    [N, k] int32 in: expert ids in [0, E); E marks an empty slot
 *   counts      [E] int32 out: (token, slot) pairs per expert
 *   offsets     [E + 1] int32 out: exclusive scan of counts; offsets[E] = N * k less the empty slots
 *   sorted_pair [N * k] int32 out: the flat pair index n * k + slot at each expert-sorted position; the
 *               token is sorted_pair / k (the page's per-expert token index list) and the slot, which
 *               selects the mixture weight, is sorted_pair % k
 *   inv_row     [N * k] int32 out: the position of each pair (inverse of sorted_pair)
 *   workspace, ws_bytes: at least moe_dispatch_workspace_size(cfg, N) bytes (may be NULL when that is 0)
 * Pairs whose id is outside [0, E) are left out of the lists (inv_row = -1); the lists are then
 * shorter than N * k and offsets[E] says so. */
moe_status moe_dispatch(const moe_config* cfg, int64_t N, const int32_t* topk_idx, int32_t* counts,
                        int32_t* offsets, int32_t* sorted_pair, int32_t* inv_row, void* workspace,
                        size_t ws_bytes, void* stream);

/* The whole layer ("MoE Forward", eq. y_n): route, dispatch, the routed SwiGLU experts on bf16 MFMA
 * (float32 accumulation; float32 arithmetic when dtype is MOE_F32), the weighted combine in a fixed
 * order without atomics, and the unscaled shared expert.
 *   x [N, D] and y [N, D] of cfg->dtype; y must not overlap x.
 *   topk_idx_out [N, k], topk_w_out [N, k], counts_out [E]: optional copies of the routing (NULL to skip).
 * Deterministic: the same inputs give bit-identical outputs. */
moe_status moe_forward(const moe_config* cfg, int64_t N, const void* x, const moe_weights* w, void* y,
                       int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out, void* workspace,
                       size_t ws_bytes, void* stream);

/* moe_forward without a workspace argument, for callers that cannot allocate device memory: code being
 * captured into a HIP graph, serving loops that must not call the allocator, harnesses that forbid it.
 * The scratch is a fixed device array of moe_noalloc_scratch_bytes() (32 MiB) inside the library, one
 * per device, taken from the first call on each device until the process ends. The call allocates and
 * frees nothing; it returns MOE_ERR_WORKSPACE, before launching anything, when the batch needs more than
 * that (moe_workspace_size(cfg, N) > moe_noalloc_scratch_bytes(): on the GLM-5 shape batches of up to
 * 146 tokens fit), and MOE_ERR_HIP if the array's device address cannot be found. Every call on a
 * device shares that device's array: calls that may overlap on one device (other streams, other
 * threads) race and must be serialised by the caller. No part of the array has to start at zero: each
 * call writes every region it reads. Arguments and results otherwise as moe_forward. */
moe_status moe_forward_noalloc(const moe_config* cfg, int64_t N, const void* x, const moe_weights* w, void* y,
                               int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out, void* stream);
size_t moe_noalloc_scratch_bytes(void);

/* The layer with routing given by the caller ("MoE Forward", Official code: the experts take x, the
 * top-k indices and the top-k weights; "GLM-5 . Mixture of experts": the expert loop skips id E):
 * dispatch, routed experts, combine and shared expert as in moe_forward, without the router.
 *   topk_idx [N, k] int32 in: expert ids; E (or any id outside [0, E)) marks an empty slot, which
 *            adds nothing
 *   topk_w   [N, k] float32 in: the weights, used as given (alpha is applied on the routed sum only
 *            when cfg->alpha_on_output is 1)
 *   x, y, counts_out, workspace, ws_bytes, stream: as for moe_forward.
 * Deterministic: the same inputs give bit-identical outputs. */
moe_status moe_forward_routed(const moe_config* cfg, int64_t N, const void* x, const moe_weights* w,
                              const int32_t* topk_idx, const float* topk_w, void* y, int32_t* counts_out,
                              void* workspace, size_t ws_bytes, void* stream);

/* The dense SwiGLU FFN of the layers before the MoE ones ("Shared output" (GLM-5), the evidence from the
 * shared expert: the dense feed-forward network is the same bias-free SwiGLU MLP,
 * y = W_down (SiLU(W_gate x) * W_up x), at the model's full intermediate width; "MoE Forward": dense
 * prefix layers never enter the MoE module). Runs on the same GEMM kernels as the shared expert.
 *   N, D, dff: tokens, hidden size, intermediate width (D and dff multiples of 64)
 *   dtype: moe_dtype of x, the weights and y; swiglu_limit as in moe_config (0: plain SwiGLU)
 *   x [N, D], gate [dff, D], up [dff, D], down [D, dff], y [N, D] (y must not overlap x)
 *   workspace, ws_bytes: at least moe_dense_workspace_size(N, D, dff, dtype) bytes.
 * Errors as for the other calls; N = 0 launches nothing. */
size_t moe_dense_workspace_size(int64_t N, int32_t D, int32_t dff, int32_t dtype);
moe_status moe_dense_forward(int64_t N, int32_t D, int32_t dff, int32_t dtype, float swiglu_limit, const void* x,
                             const void* gate, const void* up, const void* down, void* y, void* workspace,
                             size_t ws_bytes, void* stream);

/* Static string naming a status. */
const char* moe_status_str(moe_status status);

/* Per-stage timing for measurement. moe_profile_begin() starts recording a HIP event pair, on the
 * stream each call is given, around every kernel that moe_forward / moe_route / moe_dispatch launch
 * from the calling thread; moe_profile_end() waits for those events, writes the summed milliseconds and
 * launch counts per stage (up to n_stages entries, indexed as moe_stage_name lists them) and stops
 * recording. The recording state is per thread: calls made by other threads are not recorded, and each
 * thread's begin / end pair is independent. A thread's HIP events are reused across its recordings and
 * live until the process ends. Returns MOE_ERR_HIP if event creation or timing fails. For measurement
 * only: recording adds two event records around every launch. */
moe_status moe_profile_begin(void);
/* As moe_profile_begin, recording only the stages whose bit (1 << stage) is set in stage_mask (fewer
 * events in the stream when only some kernels are to be timed). */
moe_status moe_profile_begin_mask(uint32_t stage_mask);
moe_status moe_profile_end(double* ms_per_stage, int32_t* launches_per_stage, int32_t n_stages);
/* Name of stage i (NULL past the last), and the number of stages. */
const char* moe_stage_name(int32_t stage);
int32_t moe_stage_count(void);

#ifdef __cplusplus
}
#endif

#endif
