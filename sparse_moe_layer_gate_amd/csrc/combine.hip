// Combine ("MoE Forward", eq. y_n): y_n = sum over the k slots of the weighted expert rows (already
// scaled by w in the down GEMM) + the shared expert's row, accumulated in float32 in slot order and
// then the shared term, rounded once to the output type. When alpha sits on the routed output
// ("MoE Forward", Official code) the slot sum is multiplied by it before the shared term is added.
// Empty slots (inv_row < 0) add nothing. No atomics: the same inputs always give the same bits.
#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int MAX_K = 32;

// 8 consecutive elements of a row, as loaded
template <typename T>
struct V8;
template <>
struct V8<uint16_t> {
  uint4 v;
};
template <>
struct V8<float> {
  float4 a, b;
};
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ inline V8<uint16_t> load8(const uint16_t* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);  // each expert row is read once
  return V8<uint16_t>{make_uint4(v.x, v.y, v.z, v.w)};
}
__device__ inline V8<float> load8(const float* p) { return V8<float>{*(const float4*)p, *(const float4*)(p + 4)}; }
__device__ inline void add8(float* acc, const V8<uint16_t>& x) {
  const uint32_t w[4] = {x.v.x, x.v.y, x.v.z, x.v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    acc[2 * i] += __uint_as_float(w[i] << 16);
    acc[2 * i + 1] += __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ inline void add8(float* acc, const V8<float>& x) {
  acc[0] += x.a.x; acc[1] += x.a.y; acc[2] += x.a.z; acc[3] += x.a.w;
  acc[4] += x.b.x; acc[5] += x.b.y; acc[6] += x.b.z; acc[7] += x.b.w;
}
template <typename T>
__device__ inline void add8(float* acc, const T* p) {
  add8(acc, load8(p));
}
__device__ inline void store8(uint16_t* p, const float* acc) {
  uint4 v;
  v.x = (uint32_t)bf16_rne(acc[0]) | ((uint32_t)bf16_rne(acc[1]) << 16);
  v.y = (uint32_t)bf16_rne(acc[2]) | ((uint32_t)bf16_rne(acc[3]) << 16);
  v.z = (uint32_t)bf16_rne(acc[4]) | ((uint32_t)bf16_rne(acc[5]) << 16);
  v.w = (uint32_t)bf16_rne(acc[6]) | ((uint32_t)bf16_rne(acc[7]) << 16);
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, (u32x4*)p);
}
__device__ inline void store8(float* p, const float* acc) {
  *(float4*)p = make_float4(acc[0], acc[1], acc[2], acc[3]);
  *(float4*)(p + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

// One block per token; each thread owns 8 consecutive features per pass (the launch sizes the block so
// that a row of up to 8192 features takes one pass).
template <typename T>
__global__ __launch_bounds__(1024) void combine_kernel(const T* __restrict__ Y, const T* __restrict__ Ysh,
                                                      const int32_t* __restrict__ inv_row, int k, int D,
                                                      float alpha_out, T* __restrict__ y) {
  __shared__ int rows[MAX_K];
  const int64_t n = blockIdx.x;
  if (threadIdx.x < k) rows[threadIdx.x] = inv_row[n * k + threadIdx.x];
  __syncthreads();
  for (int c = threadIdx.x * 8; c < D; c += blockDim.x * 8) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    V8<T> vsh;
    if (Ysh) vsh = load8(Ysh + n * D + c);  // in flight with the slot rows
    // slots in groups of 8: the group's row loads are all issued before the first add (a loop of
    // load-then-add waited out one memory latency per slot); the adds keep slot order
    for (int s0 = 0; s0 < k; s0 += 8) {
      V8<T> v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int r = s0 + u < k ? rows[s0 + u] : -1;
        if (r >= 0) v[u] = load8(Y + (int64_t)r * D + c);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (s0 + u < k && rows[s0 + u] >= 0) add8(acc, v[u]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = __fmul_rn(acc[i], alpha_out);  // exact when alpha_out == 1
    if (Ysh) add8(acc, vsh);
    store8(y + n * D + c, acc);
  }
}

}  // namespace

hipError_t launch_combine(int dtype, const void* Y, const void* Ysh, const int32_t* inv_row, int64_t N, int k, int D,
                          float alpha_out, void* y, hipStream_t s) {
  // one thread per 8 features, whole waves, at most 1024 (D is a multiple of 64)
  int threads = (D / 8 + 63) / 64 * 64;
  if (threads > 1024) threads = 1024;
  if (dtype == MOE_F32)
    hipLaunchKernelGGL(combine_kernel<float>, dim3((unsigned)N), dim3(threads), 0, s, (const float*)Y,
                       (const float*)Ysh, inv_row, k, D, alpha_out, (float*)y);
  else
    hipLaunchKernelGGL(combine_kernel<uint16_t>, dim3((unsigned)N), dim3(threads), 0, s, (const uint16_t*)Y,
                       (const uint16_t*)Ysh, inv_row, k, D, alpha_out, (uint16_t*)y);
  return hipGetLastError();
}

}  // namespace moe
