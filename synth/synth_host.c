/* Host build of the seeded generator (see synth_core.h). OpenMP over elements. */
#include "synth_core.h"
#include <stddef.h>

void synth_philox_block(uint32_t k0, uint32_t k1, const uint32_t ctr[4], uint32_t out[4]) {
  synth_block c;
  for (int i = 0; i < 4; ++i) c.v[i] = ctr[i];
  c = synth_philox4x32_10(c, k0, k1);
  for (int i = 0; i < 4; ++i) out[i] = c.v[i];
}

void synth_normal_f64(uint32_t seed, uint32_t id, uint64_t offset, int64_t count, double std, double* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = synth_normal(seed, id, offset + (uint64_t)i, std);
}

void synth_normal_f32(uint32_t seed, uint32_t id, uint64_t offset, int64_t count, double std, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = (float)synth_normal(seed, id, offset + (uint64_t)i, std);
}

void synth_normal_bf16(uint32_t seed, uint32_t id, uint64_t offset, int64_t count, double std, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i)
    out[i] = synth_f32_to_bf16((float)synth_normal(seed, id, offset + (uint64_t)i, std));
}

void synth_uniform_f32(uint32_t seed, uint32_t id, uint64_t offset, int64_t count, double lo, double hi, float* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = (float)synth_uniform(seed, id, offset + (uint64_t)i, lo, hi);
}

void synth_f32_to_bf16_array(const float* in, int64_t count, uint16_t* out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) out[i] = synth_f32_to_bf16(in[i]);
}
