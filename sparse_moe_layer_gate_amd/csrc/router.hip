// Router kernels: the gate GEMM with its sigmoid, and the selection / weight kernel.
//
// "Group Router" (GLM-4.5), How it works: s = sigmoid(x W_g^T) with a bias-free float32 gate;
// s' = s + b chooses the experts; groups are scored by their two largest s'; topk_group groups
// survive; the top-k by s' inside them are taken; w = alpha * s / (sum s + eps) from the raw s.
#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace moe {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ inline float load_as_f32(const float* p, int64_t i) { return p[i]; }
__device__ inline float load_as_f32(const uint16_t* p, int64_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);  // bf16 -> f32 is exact
}

// ---------------------------------------------------------------------------------------------
// Gate GEMM: scores[n, e] = sigmoid(sum_t x[n, t] * W_g[e, t]) in float32 on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32: exact float32 products, float32 accumulation).
// Block tile: 64 tokens x 64 experts, K step 32; 4 waves in 2 x 2, each 32 x 32 (2 x 2 MFMA tiles).
// LDS holds both tiles k-major with a row pitch of 80 floats: a wave's MFMA operand read touches
// 4 k-rows x 16 consecutive columns, i.e. 64 distinct banks.
constexpr int LG_BM = 64, LG_BN = 64, LG_BK = 32, LG_PITCH = 80;

template <typename XT>
__global__ __launch_bounds__(256) void logits_kernel(const XT* __restrict__ x, const float* __restrict__ wg,
                                                     float* __restrict__ scores, int64_t N, int D, int E) {
  __shared__ float As[LG_BK][LG_PITCH];
  __shared__ float Bs[LG_BK][LG_PITCH];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t n0 = (int64_t)blockIdx.x * LG_BM;
  const int e0 = blockIdx.y * LG_BN;

  // loader coordinates: 8 consecutive k of one row per thread
  const int lr = t >> 2, lk = (t & 3) * 8;
  const int64_t xrow = n0 + lr;
  const int erow = e0 + lr;
  const bool xok = xrow < N, eok = erow < E;

  f32x4 acc[2][2];
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < D; k0 += LG_BK) {
    float av[8], bv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      av[i] = xok ? load_as_f32(x, xrow * D + k0 + lk + i) : 0.f;
      bv[i] = eok ? wg[(int64_t)erow * D + k0 + lk + i] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      As[lk + i][lr] = av[i];
      Bs[lk + i][lr] = bv[i];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < LG_BK; kk += 4) {
      const int kr = kk + (lane >> 4);
      float a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = As[kr][wm * 32 + i * 16 + (lane & 15)];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = Bs[kr][wn * 32 + j * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
  // C layout of the 16x16 tile: lane holds column lane % 16, rows 4 * (lane / 16) + r.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t n = n0 + wm * 32 + i * 16 + 4 * (lane >> 4) + r;
        const int e = e0 + wn * 32 + j * 16 + (lane & 15);
        if (n < N && e < E) {
          const float logit = acc[i][j][r];
          scores[n * E + e] = 1.0f / (1.0f + expf(-logit));
        }
      }
}

// ---------------------------------------------------------------------------------------------
// Selection: one wavefront per token, four tokens per block. Lane l holds experts l, l + 64, ...
// (up to 8). Every float operation below is one correctly rounded IEEE operation in the order the
// header states, so given the same scores the result is bit-identical to a plain float32 evaluation.
constexpr int SEL_MAX_E = 512, SEL_MAX_P = SEL_MAX_E / 64, SEL_MAX_G = 64, SEL_MAX_K = 32;

__device__ inline bool beats(float av, int ai, float bv, int bi) { return av > bv || (av == bv && ai < bi); }

__global__ __launch_bounds__(256) void select_kernel(const float* __restrict__ scores, const float* __restrict__ bias,
                                                     int64_t N, int E, int G, int TG, int k, float alpha, int norm,
                                                     float eps, int32_t* __restrict__ idx_out,
                                                     float* __restrict__ w_out) {
  __shared__ float s_raw[4][SEL_MAX_E];
  __shared__ float s_sel[4][SEL_MAX_E];
  __shared__ float gscore[4][SEL_MAX_G];
  __shared__ int kept[4][SEL_MAX_G];
  __shared__ int chosen[4][SEL_MAX_K];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n = (int64_t)blockIdx.x * 4 + wave;
  const bool live = n < N;
  const int P = (E + 63) >> 6;
  const int gs = E / G;
  const bool group_stage = G > 1 && TG < G;

  float sp[SEL_MAX_P];
  bool elig[SEL_MAX_P];
#pragma unroll
  for (int p = 0; p < SEL_MAX_P; ++p) {
    const int e = lane + 64 * p;
    float sv = 0.f, bv = 0.f;
    if (p < P && e < E && live) {
      sv = scores[n * E + e];
      bv = bias[e];
    }
    sp[p] = __fadd_rn(sv, bv);  // s' = s + b
    elig[p] = p < P && e < E;
    if (p < P && e < E) {
      s_raw[wave][e] = sv;
      s_sel[wave][e] = sp[p];
    }
  }
  __syncthreads();

  if (group_stage) {
    // group score: sum of the two largest s' of the group (a repeated value counts twice)
    if (lane < G) {
      float m1 = -INFINITY, m2 = -INFINITY;
      for (int e = lane * gs; e < (lane + 1) * gs; ++e) {
        const float v = s_sel[wave][e];
        if (v > m1) {
          m2 = m1;
          m1 = v;
        } else if (v > m2) {
          m2 = v;
        }
      }
      gscore[wave][lane] = __fadd_rn(m1, m2);
    }
    __syncthreads();
    if (lane < G) {
      const float mine = gscore[wave][lane];
      int ahead = 0;
      for (int h = 0; h < G; ++h) ahead += beats(gscore[wave][h], h, mine, lane) ? 1 : 0;
      kept[wave][lane] = ahead < TG;
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < SEL_MAX_P; ++p) {
      const int e = lane + 64 * p;
      if (elig[p]) elig[p] = kept[wave][e / gs] != 0;
    }
  }

  // k rounds of a wave-wide arg-max under (s' descending, index ascending)
  for (int slot = 0; slot < k; ++slot) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int p = 0; p < SEL_MAX_P; ++p) {
      const int e = lane + 64 * p;
      if (elig[p] && beats(sp[p], e, bv, bi)) {
        bv = sp[p];
        bi = e;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      if (beats(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
#pragma unroll
    for (int p = 0; p < SEL_MAX_P; ++p)
      if (lane + 64 * p == bi) elig[p] = false;  // k <= eligible count is checked on the host
    if (lane == 0) chosen[wave][slot] = min(bi, E - 1);  // stays in range even for NaN scores
  }
  __syncthreads();

  if (live && lane < k) {
    const int e = chosen[wave][lane];
    const float s_mine = s_raw[wave][e];
    float w;
    if (norm) {
      float sum = 0.f;
      for (int j = 0; j < k; ++j) sum = __fadd_rn(sum, s_raw[wave][chosen[wave][j]]);
      const float den = __fadd_rn(sum, eps);
      w = __fmul_rn(alpha, __fdiv_rn(s_mine, den));
    } else {
      w = __fmul_rn(alpha, s_mine);
    }
    idx_out[n * k + lane] = e;
    w_out[n * k + lane] = w;
  }
}

}  // namespace

hipError_t launch_logits(int dtype, const void* x, const float* wg, const uint16_t* /*wsplit*/, int64_t N, int D,
                         int E, float* scores, hipStream_t s) {
  dim3 grid((unsigned)((N + LG_BM - 1) / LG_BM), (unsigned)((E + LG_BN - 1) / LG_BN));
  if (dtype == MOE_F32)
    hipLaunchKernelGGL(logits_kernel<float>, grid, dim3(256), 0, s, (const float*)x, wg, scores, N, D, E);
  else
    hipLaunchKernelGGL(logits_kernel<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)x, wg, scores, N, D, E);
  return hipGetLastError();
}

hipError_t launch_router_split(const float*, int, int, uint16_t*, hipStream_t) { return hipSuccess; }

hipError_t launch_select(const float* scores, const float* bias, int64_t N, int E, int G, int TG, int k, float alpha,
                         int norm, float eps, int32_t* idx, float* w, hipStream_t s) {
  dim3 grid((unsigned)((N + 3) / 4));
  hipLaunchKernelGGL(select_kernel, grid, dim3(256), 0, s, scores, bias, N, E, G, TG, k, alpha, norm, eps, idx, w);
  return hipGetLastError();
}

}  // namespace moe
