// Device build of the seeded generator (see synth_core.h): fills device
// buffers with exactly the values the host build produces. Used to place the
// multi-GB expert weight tensors in HBM without a host round trip.
#include <hip/hip_runtime.h>
#include "synth_core.h"

namespace {

__global__ void normal_bf16_kernel(uint32_t seed, uint32_t id, uint64_t offset, int64_t count, double std,
                                   uint16_t* __restrict__ out) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
    out[i] = synth_f32_to_bf16((float)synth_normal(seed, id, offset + (uint64_t)i, std));
}

__global__ void normal_f32_kernel(uint32_t seed, uint32_t id, uint64_t offset, int64_t count, double std,
                                  float* __restrict__ out) {
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
    out[i] = (float)synth_normal(seed, id, offset + (uint64_t)i, std);
}

int grid_for(int64_t count) {
  int64_t blocks = (count + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  return (int)blocks;
}

}  // namespace

extern "C" {

// Fills out[0..count) with bf16 values of elements offset..offset+count of
// stream (seed, id). Asynchronous on `stream`; returns the launch status.
int synth_dev_normal_bf16(uint32_t seed, uint32_t id, uint64_t offset, int64_t count, double std, void* out,
                          void* stream) {
  if (count <= 0) return 0;
  hipLaunchKernelGGL(normal_bf16_kernel, dim3(grid_for(count)), dim3(256), 0, (hipStream_t)stream, seed, id,
                     offset, count, std, (uint16_t*)out);
  return (int)hipGetLastError();
}

int synth_dev_normal_f32(uint32_t seed, uint32_t id, uint64_t offset, int64_t count, double std, void* out,
                         void* stream) {
  if (count <= 0) return 0;
  hipLaunchKernelGGL(normal_f32_kernel, dim3(grid_for(count)), dim3(256), 0, (hipStream_t)stream, seed, id,
                     offset, count, std, (float*)out);
  return (int)hipGetLastError();
}

}  // extern "C"
