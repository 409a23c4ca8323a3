/*
 * Seeded synthetic inputs: one counter-based stream per tensor.
 *
 * This header is the whole generator. It is compiled twice: by gcc into the
 * host library (synth_host.c) and by hipcc into the device library
 * (synth_dev.hip). Both builds use -ffp-contract=off, and every floating-point
 * step below is a single IEEE operation (exact integer sums, correctly rounded
 * double multiplies, a double->float conversion, an integer bf16 rounding), so
 * the two builds produce bit-identical values for the same (seed, tensor id,
 * element index).
 *
 * The generator holds none of the MoE method's arithmetic; it only produces
 * the input tensors (activations, router weights, correction bias, expert
 * weights) that the oracle and the GPU path both consume.
 *
 * Bit source: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC'11), keyed by (seed, tensor id), with the
 * 128-bit counter set to (element index low word, high word, 0, 0). Each
 * element consumes one block of four 32-bit words.
 *
 * Normal stand-in: the Irwin-Hall sum of the eight 16-bit halves of that
 * block, centred and scaled to unit variance. Its support is about +-4.9 and
 * its excess kurtosis -0.15; it replaces Box-Muller because it needs no
 * transcendental function, so host and device agree bit for bit.
 */
#ifndef SYNTH_CORE_H
#define SYNTH_CORE_H

#include <stdint.h>

#ifdef __HIPCC__
#define SYNTH_FN static inline __host__ __device__
#else
#define SYNTH_FN static inline
#endif

#define SYNTH_PHILOX_M0 0xD2511F53u
#define SYNTH_PHILOX_M1 0xCD9E8D57u
#define SYNTH_PHILOX_W0 0x9E3779B9u
#define SYNTH_PHILOX_W1 0xBB67AE85u

typedef struct { uint32_t v[4]; } synth_block;

/* One Philox4x32 round: two 32x32->64 multiplies, the high halves xored with
 * the other counter words and the key. */
SYNTH_FN synth_block synth_philox_round(synth_block c, uint32_t k0, uint32_t k1) {
  uint64_t p0 = (uint64_t)SYNTH_PHILOX_M0 * (uint64_t)c.v[0];
  uint64_t p1 = (uint64_t)SYNTH_PHILOX_M1 * (uint64_t)c.v[2];
  synth_block o;
  o.v[0] = (uint32_t)(p1 >> 32) ^ c.v[1] ^ k0;
  o.v[1] = (uint32_t)p1;
  o.v[2] = (uint32_t)(p0 >> 32) ^ c.v[3] ^ k1;
  o.v[3] = (uint32_t)p0;
  return o;
}

/* Philox4x32-10: ten rounds, the key advanced by the Weyl constants between
 * consecutive rounds. */
SYNTH_FN synth_block synth_philox4x32_10(synth_block c, uint32_t k0, uint32_t k1) {
  for (int r = 0; r < 10; ++r) {
    if (r > 0) { k0 += SYNTH_PHILOX_W0; k1 += SYNTH_PHILOX_W1; }
    c = synth_philox_round(c, k0, k1);
  }
  return c;
}

SYNTH_FN synth_block synth_element_block(uint32_t seed, uint32_t tensor_id, uint64_t index) {
  synth_block c;
  c.v[0] = (uint32_t)index;
  c.v[1] = (uint32_t)(index >> 32);
  c.v[2] = 0u;
  c.v[3] = 0u;
  return synth_philox4x32_10(c, seed, tensor_id);
}

/* sqrt(3/2) * 2^-17, correctly rounded: maps the centred half-sum c = 2S - 8*65535
 * (S = sum of the eight 16-bit halves) to a unit-variance value. */
#define SYNTH_IH8_SCALE 0x1.3988e1409212ep-17

/* Approximately N(0, std^2) as a double: centred Irwin-Hall(8) times std. */
SYNTH_FN double synth_normal(uint32_t seed, uint32_t tensor_id, uint64_t index, double std) {
  synth_block b = synth_element_block(seed, tensor_id, index);
  int32_t s = 0;
  for (int j = 0; j < 4; ++j) s += (int32_t)(b.v[j] & 0xFFFFu) + (int32_t)(b.v[j] >> 16);
  int32_t c = 2 * s - 8 * 65535;
  double z = (double)c * SYNTH_IH8_SCALE;
  return z * std;
}

/* U(lo, hi) from the first word: lo + (hi - lo) * (w + 1/2) 2^-32, three rounded steps. */
SYNTH_FN double synth_uniform(uint32_t seed, uint32_t tensor_id, uint64_t index, double lo, double hi) {
  synth_block b = synth_element_block(seed, tensor_id, index);
  double u = ((double)b.v[0] + 0.5) * 0x1p-32;
  double span = hi - lo;
  double t = span * u;
  return lo + t;
}

/* float -> bfloat16 bits, round to nearest even (inputs here are finite). */
SYNTH_FN uint16_t synth_f32_to_bf16(float f) {
  union { float f; uint32_t u; } cv;
  cv.f = f;
  uint32_t u = cv.u;
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

#endif
