/*
 * CPU oracle of the GLM-4.5 / GLM-5 sparse-MoE FFN forward.
 * TEST INFRASTRUCTURE ONLY -- see moe_oracle.h for scope, sources and readings.
 */
#include "moe_oracle.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

int oracle_num_threads(void) { return omp_get_max_threads(); }

static double widen(const void* p, int dt, int64_t i) {
  if (dt == ORACLE_F32) return (double)((const float*)p)[i];
  uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

int oracle_check_cfg(const oracle_cfg* c) {
  if (c->D < 1 || c->E < 1 || c->d < 1 || c->k < 1 || c->n_shared < 0) return -1;
  if (c->G < 1 || c->E % c->G != 0) return -1;
  if (c->TG < 1 || c->TG > c->G) return -1;
  if (c->G > 1 && c->E / c->G < 2) return -1; /* a group needs two members for its top-2 score */
  if (c->k > c->TG * (c->E / c->G)) return -1; /* kept groups must hold at least k experts */
  if (!(c->limit >= 0.0f) || isinf(c->limit)) return -1;
  if (c->alpha_on_output != 0 && c->alpha_on_output != 1) return -1;
  return 0;
}

/* "Group Router", How it works: the gate is a bias-free linear map evaluated in float32. The oracle
 * forms each logit exactly as a double dot product over the hidden index and rounds once. */
int oracle_logits(const oracle_cfg* c, int64_t N, const void* x, int xdt, const float* wg, float* r) {
  if (oracle_check_cfg(c)) return -1;
  const int64_t D = c->D, E = c->E;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int64_t t = 0; t < D; ++t) acc += widen(x, xdt, n * D + t) * (double)wg[e * D + t];
      r[n * E + e] = (float)acc;
    }
  }
  return 0;
}

/* "Group Router", eq. s = sigma(x W_g^T): a sigmoid, not a softmax. */
void oracle_sigmoid(int64_t count, const float* r, float* s) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) s[i] = (float)(1.0 / (1.0 + exp(-(double)r[i])));
}

/* The routing of one token. sp = s + b (selection scores). */
typedef struct {
  float sp[1024];
  uint8_t eligible[1024];
  float gscore[1024];
  uint8_t kept[1024];
} token_work;

/* "Group Router", How it works: a group's score is the sum of its two largest bias-adjusted entries
 * (duplicates count twice); the topk_group best groups survive, ties to the lower group index. With
 * G = 1, or topk_group = G, every expert stays eligible (the stage is a no-op). */
static void group_stage(const oracle_cfg* c, token_work* tw) {
  const int E = c->E, G = c->G, TG = c->TG, gs = c->E / c->G;
  for (int e = 0; e < E; ++e) tw->eligible[e] = 1;
  for (int g = 0; g < G; ++g) tw->kept[g] = 1;
  if (G == 1 || TG == G) return;
  for (int g = 0; g < G; ++g) {
    float m1 = -INFINITY, m2 = -INFINITY;
    for (int e = g * gs; e < (g + 1) * gs; ++e) {
      float v = tw->sp[e];
      if (v > m1) {
        m2 = m1;
        m1 = v;
      } else if (v > m2) {
        m2 = v;
      }
    }
    tw->gscore[g] = m1 + m2;
  }
  for (int g = 0; g < G; ++g) {
    int ahead = 0; /* groups ranked before g */
    for (int h = 0; h < G; ++h)
      if (tw->gscore[h] > tw->gscore[g] || (tw->gscore[h] == tw->gscore[g] && h < g)) ++ahead;
    tw->kept[g] = (uint8_t)(ahead < TG);
  }
  for (int e = 0; e < E; ++e) tw->eligible[e] = tw->kept[e / gs];
}

/* "Group Router", eq. T: the k largest s' among the eligible experts, taken one at a time, the lower
 * index winning a tie; the order taken is the slot order. */
static void take_topk(const oracle_cfg* c, const token_work* tw, int32_t* idx) {
  uint8_t taken[1024];
  memset(taken, 0, sizeof taken);
  for (int slot = 0; slot < c->k; ++slot) {
    int best = -1;
    for (int e = 0; e < c->E; ++e) {
      if (!tw->eligible[e] || taken[e]) continue;
      if (best < 0 || tw->sp[e] > tw->sp[best]) best = e;
    }
    taken[best] = 1;
    idx[slot] = best;
  }
}

/* "Group Router", eq. s-bar / w, and "MoE Forward", eq. w_{n,i}: the weights use the raw s of the
 * chosen experts (never s'), renormalised over the chosen set with eps in the denominator when
 * norm_topk_prob is set, then multiplied by alpha -- unless alpha goes on the routed output instead
 * ("MoE Forward", Official code: one place or the other, never both). */
static void weights(const oracle_cfg* c, const float* s_row, const int32_t* idx, float* w) {
  const float a = c->alpha_on_output ? 1.0f : c->alpha;
  if (c->norm) {
    float sum = 0.0f;
    for (int slot = 0; slot < c->k; ++slot) sum = sum + s_row[idx[slot]];
    float den = sum + c->eps;
    for (int slot = 0; slot < c->k; ++slot) {
      float q = s_row[idx[slot]] / den;
      w[slot] = a * q;
    }
  } else {
    for (int slot = 0; slot < c->k; ++slot) w[slot] = a * s_row[idx[slot]];
  }
}

int oracle_select(const oracle_cfg* c, int64_t N, const float* s, const float* b, int32_t* idx, float* w,
                  uint8_t* kept) {
  if (oracle_check_cfg(c) || c->E > 1024) return -1;
  const int E = c->E, k = c->k;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    token_work* tw = (token_work*)malloc(sizeof(token_work));
    const float* s_row = s + n * E;
    for (int e = 0; e < E; ++e) tw->sp[e] = s_row[e] + b[e]; /* "Group Router": s' = s + b */
    group_stage(c, tw);
    take_topk(c, tw, idx + n * k);
    weights(c, s_row, idx + n * k, w + n * k);
    if (kept)
      for (int g = 0; g < c->G; ++g) kept[n * c->G + g] = tw->kept[g];
    free(tw);
  }
  return 0;
}

int oracle_select_margin(const oracle_cfg* c, int64_t N, const float* s, const float* b, double* margin) {
  if (oracle_check_cfg(c) || c->E > 1024) return -1;
  const int E = c->E, k = c->k;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < N; ++n) {
    token_work* tw = (token_work*)malloc(sizeof(token_work));
    const float* s_row = s + n * E;
    for (int e = 0; e < E; ++e) tw->sp[e] = s_row[e] + b[e];
    group_stage(c, tw);
    double m = INFINITY;
    /* the k+1 largest eligible s' values, in selection order */
    uint8_t taken[1024];
    memset(taken, 0, sizeof taken);
    double prev = 0.0;
    for (int slot = 0; slot <= k; ++slot) {
      int best = -1;
      for (int e = 0; e < E; ++e) {
        if (!tw->eligible[e] || taken[e]) continue;
        if (best < 0 || tw->sp[e] > tw->sp[best]) best = e;
      }
      if (best < 0) break;
      taken[best] = 1;
      if (slot > 0 && prev - (double)tw->sp[best] < m) m = prev - (double)tw->sp[best];
      prev = (double)tw->sp[best];
    }
    if (c->G > 1 && c->TG < c->G) {
      /* the weakest kept group against the strongest discarded one */
      double weakest_kept = INFINITY, best_dropped = -INFINITY;
      for (int g = 0; g < c->G; ++g) {
        if (tw->kept[g] && tw->gscore[g] < weakest_kept) weakest_kept = tw->gscore[g];
        if (!tw->kept[g] && tw->gscore[g] > best_dropped) best_dropped = tw->gscore[g];
      }
      if (weakest_kept - best_dropped < m) m = weakest_kept - best_dropped;
    }
    margin[n] = m;
    free(tw);
  }
  return 0;
}

/* Token-choice dispatch ("MoE Forward", two facts, #2): each (token, slot) pair goes to one expert.
 * The per-expert token list of the "GLM-5 . Mixture of experts" loop form, written as counts, an
 * exclusive scan and a stable placement in ascending token order. */
int oracle_dispatch(const oracle_cfg* c, int64_t N, const int32_t* idx, int32_t* counts, int32_t* offsets,
                    int32_t* sorted_pair, int32_t* inv_row) {
  const int E = c->E, k = c->k;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int64_t i = 0; i < N * k; ++i) {
    if (idx[i] < 0 || idx[i] > E) return -1;
    if (idx[i] < E) counts[idx[i]]++;
  }
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  int32_t* cursor = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  for (int e = 0; e < E; ++e) cursor[e] = offsets[e];
  for (int64_t n = 0; n < N; ++n) {
    for (int slot = 0; slot < k; ++slot) {
      int64_t p = n * k + slot;
      if (idx[p] == E) {  /* empty slot ("GLM-5 . Mixture of experts": id E is skipped) */
        inv_row[p] = -1;
        continue;
      }
      int32_t pos = cursor[idx[p]]++;
      sorted_pair[pos] = (int32_t)p;
      inv_row[p] = pos;
    }
  }
  free(cursor);
  return 0;
}

/* SiLU(a) * u of one intermediate column; with limit > 0 the gate value is capped from above only and
 * the up value clipped on both sides first ("Module 02 -- MoE: Capacity, Work, and Traffic", section 3). */
static double swiglu_act(double g, double u, double limit) {
  if (limit > 0.0) {
    if (g > limit) g = limit;
    if (u > limit) u = limit;
    if (u < -limit) u = -limit;
  }
  return g / (1.0 + exp(-g)) * u;
}

/* "MoE Forward", eq. E_i: W_down (SiLU(W_gate x) (.) W_up x), bias-free; SiLU(z) = z / (1 + e^-z).
 * "Shared output": the shared expert is the same MLP with its own gate / up / down matrices. */
void oracle_swiglu(int32_t D, int32_t dff, const void* gate, const void* up, const void* down, int wdt,
                   double limit, const double* x, double* out) {
  double* h = (double*)malloc(sizeof(double) * (size_t)dff);
  for (int64_t j = 0; j < dff; ++j) {
    double g = 0.0, u = 0.0;
    for (int64_t t = 0; t < D; ++t) {
      g += widen(gate, wdt, j * D + t) * x[t];
      u += widen(up, wdt, j * D + t) * x[t];
    }
    h[j] = swiglu_act(g, u, limit);
  }
  for (int64_t i = 0; i < D; ++i) {
    double o = 0.0;
    for (int64_t j = 0; j < dff; ++j) o += widen(down, wdt, i * dff + j) * h[j];
    out[i] = o;
  }
  free(h);
}

static size_t elem_size(int dt) { return dt == ORACLE_F32 ? 4 : 2; }

/* Routed expert e: the packed gate_up matrix holds the gate rows first and the up rows after them
 * ("MoE Forward", the packed gate_up_proj layout of shape (2 d_moe, D)). */
static void routed_expert(const oracle_cfg* c, const void* gu, const void* dn, int wdt, const double* x,
                          double* out) {
  const char* base = (const char*)gu;
  const void* up = base + (size_t)c->d * (size_t)c->D * elem_size(wdt);
  oracle_swiglu(c->D, c->d, gu, up, dn, wdt, (double)c->limit, x, out);
}

/* "MoE Forward", eq. y_n: the alpha-scaled routed sum over the chosen experts in slot order, plus the
 * shared expert at scale 1 on the same input. */
int oracle_forward_tokens(const oracle_cfg* c, int64_t ntok, const int64_t* tokens, const void* x, int xdt,
                          const void* const* gate_up, const void* const* down, const void* sh_gate,
                          const void* sh_up, const void* sh_down, int wdt, const int32_t* idx, const float* w,
                          float* y) {
  if (oracle_check_cfg(c)) return -1;
  const int64_t D = c->D, k = c->k;
  for (int64_t i = 0; i < ntok; ++i)
    for (int64_t slot = 0; slot < k; ++slot) {
      int32_t e = idx[tokens[i] * k + slot];
      if (e < 0 || e > c->E || (e < c->E && (!gate_up[e] || !down[e]))) return -1;
    }
  if (c->n_shared > 0 && (!sh_gate || !sh_up || !sh_down)) return -1;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < ntok; ++i) {
    const int64_t n = tokens[i];
    double* xd = (double*)malloc(sizeof(double) * (size_t)D);
    double* o = (double*)malloc(sizeof(double) * (size_t)D);
    double* acc = (double*)calloc((size_t)D, sizeof(double));
    for (int64_t t = 0; t < D; ++t) xd[t] = widen(x, xdt, n * D + t);
    for (int64_t slot = 0; slot < k; ++slot) {
      int32_t e = idx[n * k + slot];
      if (e == c->E) continue; /* empty slot */
      routed_expert(c, gate_up[e], down[e], wdt, xd, o);
      double ws = (double)w[n * k + slot];
      for (int64_t t = 0; t < D; ++t) acc[t] += ws * o[t];
    }
    if (c->alpha_on_output)
      for (int64_t t = 0; t < D; ++t) acc[t] *= (double)c->alpha;
    if (c->n_shared > 0) {
      oracle_swiglu(c->D, c->d * c->n_shared, sh_gate, sh_up, sh_down, wdt, (double)c->limit, xd, o);
      for (int64_t t = 0; t < D; ++t) acc[t] += o[t];
    }
    for (int64_t t = 0; t < D; ++t) y[i * D + t] = (float)acc[t];
    free(xd);
    free(o);
    free(acc);
  }
  return 0;
}

/* The same sum written as the "GLM-5 . Mixture of experts" loop over experts: each expert with at
 * least one token evaluates its MLP on those tokens and adds the weighted result into the output. The
 * weight rows are read once per expert and reused across its tokens. */
int oracle_forward_expert_loop(const oracle_cfg* c, int64_t N, const void* x, int xdt,
                               const void* const* gate_up, const void* const* down, const void* sh_gate,
                               const void* sh_up, const void* sh_down, int wdt, const int32_t* idx,
                               const float* w, float* y) {
  if (oracle_check_cfg(c)) return -1;
  const int64_t D = c->D, k = c->k, E = c->E, d = c->d;
  for (int64_t p = 0; p < N * k; ++p)
    if (idx[p] < 0 || idx[p] > E || (idx[p] < E && (!gate_up[idx[p]] || !down[idx[p]]))) return -1;
  if (c->n_shared > 0 && (!sh_gate || !sh_up || !sh_down)) return -1;
  double* acc = (double*)calloc((size_t)(N * D), sizeof(double));
  double* xd = (double*)malloc(sizeof(double) * (size_t)(N * D));
  for (int64_t i = 0; i < N * D; ++i) xd[i] = widen(x, xdt, i);
  int64_t* tok = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
  double* tw = (double*)malloc(sizeof(double) * (size_t)N);
  for (int64_t e = 0; e <= E; ++e) {
    /* e == E is the shared expert: every token, weight 1, width d * n_shared */
    int64_t m = 0;
    const void *g_ptr, *u_ptr, *dn_ptr;
    int64_t dff;
    if (e < E) {
      for (int64_t n = 0; n < N; ++n)
        for (int64_t slot = 0; slot < k; ++slot)
          if (idx[n * k + slot] == e) {
            tok[m] = n;
            tw[m] = (double)w[n * k + slot];
            ++m;
          }
      if (m == 0) continue;
      dff = d;
      g_ptr = gate_up[e];
      u_ptr = (const char*)gate_up[e] + (size_t)d * (size_t)D * elem_size(wdt);
      dn_ptr = down[e];
    } else {
      if (c->alpha_on_output)
        for (int64_t i = 0; i < N * D; ++i) acc[i] *= (double)c->alpha;
      if (c->n_shared == 0) break;
      for (int64_t n = 0; n < N; ++n) {
        tok[m] = n;
        tw[m] = 1.0;
        ++m;
      }
      dff = d * c->n_shared;
      g_ptr = sh_gate;
      u_ptr = sh_up;
      dn_ptr = sh_down;
    }
    double* h = (double*)malloc(sizeof(double) * (size_t)(m * dff));
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < dff; ++j) {
      for (int64_t i = 0; i < m; ++i) {
        const double* xr = xd + tok[i] * D;
        double g = 0.0, u = 0.0;
        for (int64_t t = 0; t < D; ++t) {
          g += widen(g_ptr, wdt, j * D + t) * xr[t];
          u += widen(u_ptr, wdt, j * D + t) * xr[t];
        }
        h[i * dff + j] = swiglu_act(g, u, (double)c->limit);
      }
    }
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < D; ++t) {
      for (int64_t i = 0; i < m; ++i) {
        double o = 0.0;
        for (int64_t j = 0; j < dff; ++j) o += widen(dn_ptr, wdt, t * dff + j) * h[i * dff + j];
        acc[tok[i] * D + t] += tw[i] * o;
      }
    }
    free(h);
  }
  for (int64_t i = 0; i < N * D; ++i) y[i] = (float)acc[i];
  free(acc);
  free(xd);
  free(tok);
  free(tw);
  return 0;
}

/* "GLM-5 . Mixture of experts", exact per-instance accounting: router = W_g (E x D) plus its E bias
 * values; each expert (routed or shared) = gate + up + down = 3 D d; used per token = router + k routed
 * experts + the shared expert. */
void oracle_param_count(const oracle_cfg* c, int64_t out[6]) {
  const int64_t D = c->D, E = c->E, d = c->d;
  const int64_t router = E * D + E;
  const int64_t expert = 3 * D * d;
  const int64_t routed = E * expert;
  const int64_t shared = 3 * D * d * c->n_shared;
  out[0] = router;
  out[1] = expert;
  out[2] = routed;
  out[3] = shared;
  out[4] = router + routed + shared;
  out[5] = router + (int64_t)c->k * expert + shared;
}
