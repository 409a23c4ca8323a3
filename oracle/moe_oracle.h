/*
 * CPU oracle of the GLM-4.5 / GLM-5 sparse-MoE FFN forward.
 *
 * TEST INFRASTRUCTURE ONLY. This is a plain, slow, obviously correct host
 * implementation of what the pages define, used to check the GPU library.
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load it. The GPU path never calls, links or includes it, and it shares
 * no code with the GPU path (its only common dependency is the seeded input
 * generator, which holds none of the method's arithmetic).
 *
 * Sources (pages as titled):
 *  - "Group Router" (GLM-4.5): How it works -- the fp32 bias-free gate and
 *    sigmoid (eq. s = sigma(x W_g^T)), the selection-only correction bias
 *    (s' = s + b), the group score as the sum of the two largest s' in each
 *    of G contiguous groups, keeping topk_group groups, top-k inside them
 *    (eq. T), and the weights alpha * s / (sum_T s + eps) from the raw s.
 *  - "MoE Forward" (GLM-4.5): How it works -- the SwiGLU expert
 *    E_i(x) = W_down (SiLU(W_gate x) * W_up x), the packed gate_up layout, the
 *    output y_n = sum_T w E_i(x_n) + E_sh(x_n), alpha scaling only the routed
 *    sum, token-choice dispatch.
 *  - "GLM-5 . Mixture of experts": the exact per-instance parameter table and
 *    the per-expert loop form of the routed sum.
 *  - "Shared output" (GLM-5): the shared expert as a bias-free SwiGLU MLP.
 *
 * Precision: dot products accumulate in double over the hidden index in
 * ascending order; the selection arithmetic (s + b, top-2 sums, the weight
 * normalisation) is carried out in float32, one IEEE operation at a time, in
 * the order written below. Expert outputs and the final sum are double,
 * rounded once to float32. Build with -ffp-contract=off.
 *
 * Readings of points the pages leave open (listed with reasons in the design
 * notes): discarded groups are excluded (the "-inf" reading of the group
 * mask); ties go to the lower expert / group index; the k output slots are in
 * (s' descending, index ascending) order and that order fixes the sum in the
 * weight denominator; alpha is applied once, inside the weights unless
 * alpha_on_output asks for it on the routed sum; eps is the float32 nearest
 * 1e-20; the SwiGLU is plain unless limit > 0.
 *
 * Variants ("MoE Forward", Official code: the router and the routed output as
 * separate places alpha may sit; "GLM-5 . Mixture of experts": the loop form
 * that skips the expert id E; "Module 02 -- MoE: Capacity, Work, and Traffic",
 * section 3: the clamped SwiGLU of that checkpoint):
 *  - alpha_on_output = 1: the weights are s / (sum s + eps) and the routed sum
 *    is multiplied by alpha (the shared expert still enters at scale 1);
 *  - limit > 0: every expert, routed or shared, clamps its gate projection
 *    from above at limit (no lower bound) and its up projection to
 *    [-limit, limit] before SiLU(gate) * up;
 *  - routing given by the caller may hold the id E in a slot: that slot adds
 *    nothing (an empty slot).
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of x and of the expert weights. */
enum { ORACLE_F32 = 0, ORACLE_BF16 = 1 };

typedef struct {
  int32_t D;        /* hidden size */
  int32_t E;        /* routed experts */
  int32_t G;        /* n_group */
  int32_t TG;       /* topk_group */
  int32_t k;        /* num_experts_per_tok */
  int32_t d;        /* moe_intermediate_size */
  int32_t n_shared; /* shared experts; the shared MLP width is d * n_shared */
  float alpha;      /* routed_scaling_factor */
  int32_t norm;     /* norm_topk_prob */
  float eps;        /* added to the weight denominator */
  float limit;      /* SwiGLU clamp bound; 0 = plain SwiGLU */
  int32_t alpha_on_output; /* 1: alpha scales the routed sum instead of the weights */
} oracle_cfg;

/* 0 if the configuration is one the oracle can evaluate, else -1. */
int oracle_check_cfg(const oracle_cfg* c);

/* r[n,e] = sum_t x[n,t] W_g[e,t] in double, rounded once to float. x [N,D] of type xdt, W_g [E,D] float. */
int oracle_logits(const oracle_cfg* c, int64_t N, const void* x, int xdt, const float* wg, float* r);

/* s = float(1 / (1 + exp(-r))) evaluated in double. */
void oracle_sigmoid(int64_t count, const float* r, float* s);

/* Selection and weights for N tokens from scores s [N,E] and bias b [E].
 * idx [N,k] (slot order), w [N,k]. kept [N,G] (nullable) receives 1 for kept groups. */
int oracle_select(const oracle_cfg* c, int64_t N, const float* s, const float* b, int32_t* idx, float* w,
                  uint8_t* kept);

/* Smallest decision gap per token: the least difference between consecutive entries of the
 * k+1 largest eligible s' values, and (group stage live) between the topk_group-th and the
 * next group score. A token whose gap exceeds the score error cannot change its routing. */
int oracle_select_margin(const oracle_cfg* c, int64_t N, const float* s, const float* b, double* margin);

/* counts[E], offsets[E+1] (exclusive scan), sorted_pair[offsets[E]] (flat n*k+slot, tokens ascending inside
 * each expert), inv_row[N*k] (position of each (n, slot) in that order; -1 for an empty slot, id E). */
int oracle_dispatch(const oracle_cfg* c, int64_t N, const int32_t* idx, int32_t* counts, int32_t* offsets,
                    int32_t* sorted_pair, int32_t* inv_row);

/* One SwiGLU MLP on one token, in double: out[D] = down (SiLU(a) * u) with a = gate x, u = up x, clamped
 * as a = min(a, limit), u = min(max(u, -limit), limit) when limit > 0.
 * gate, up: [dff, D]; down: [D, dff]; element type wdt. */
void oracle_swiglu(int32_t D, int32_t dff, const void* gate, const void* up, const void* down, int wdt,
                   double limit, const double* x, double* out);

/* Per-token form of the layer output for the listed tokens, given routing (idx, w for all N tokens):
 * y[i] = float( A * sum_slot w * E_idx(x_n) + E_sh(x_n) ), n = tokens[i], A = alpha if alpha_on_output
 * else 1; slots holding id E are empty.
 * gate_up[e] -> [2d, D], down[e] -> [D, d] (entries may be NULL for experts no listed token uses). */
int oracle_forward_tokens(const oracle_cfg* c, int64_t ntok, const int64_t* tokens, const void* x, int xdt,
                          const void* const* gate_up, const void* const* down, const void* sh_gate,
                          const void* sh_up, const void* sh_down, int wdt, const int32_t* idx, const float* w,
                          float* y);

/* Per-expert loop form over all N tokens: for each expert with at least one token, add w * E_e(x_n)
 * into a double accumulator, expert by expert; scale it by A (as above), add the shared expert; round
 * once. Slots holding id E are skipped. */
int oracle_forward_expert_loop(const oracle_cfg* c, int64_t N, const void* x, int xdt,
                               const void* const* gate_up, const void* const* down, const void* sh_gate,
                               const void* sh_up, const void* sh_down, int wdt, const int32_t* idx,
                               const float* w, float* y);

/* Threads the oracle's parallel loops use (OpenMP's maximum). */
int oracle_num_threads(void);

/* Parameter accounting of one MoE block: out = {router (W_g + bias), one routed expert, all routed
 * experts, shared expert, total, used per token (router + k routed + shared)}. */
void oracle_param_count(const oracle_cfg* c, int64_t out[6]);

#ifdef __cplusplus
}
#endif

#endif
