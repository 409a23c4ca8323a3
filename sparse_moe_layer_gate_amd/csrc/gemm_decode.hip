// Grouped bf16 expert GEMMs for token-poor (decode) batches.
//
// With one or two tokens per expert the layer is a weight stream ("Module 02 -- MoE: Capacity, Work,
// and Traffic", section 1: traffic, not arithmetic, governs decode), so this kernel is built to keep
// as many weight bytes in flight as possible and to touch each weight byte once:
//  - row tiles of at most 16 rows (the tile list is built with 16 rows per tile);
//  - no LDS and no barriers: each wave streams its own weight rows (16 output columns per
//    v_mfma_f32_16x16x32_bf16 tile) straight from HBM into registers, U K-slices per iteration, and
//    reads the few activation rows from L2; many independent waves per CU hide the HBM latency;
//  - gate_up: each wave owns 32 intermediate columns as two gate and two up tiles and applies the
//    SwiGLU in registers; down: each wave owns 64 output columns and scales each row by its weight.
#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#ifndef MOE_DC_U
#define MOE_DC_U 16
#endif
#ifndef MOE_DC_NT
#define MOE_DC_NT 2
#endif
constexpr int DC_U = MOE_DC_U;    // K-slices of 32 per loop iteration
constexpr int DC_NT = MOE_DC_NT;  // 16-column MFMA tiles per wave (gate_up: half gate, half up)

__device__ inline uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ inline float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

template <bool GATE_UP>
__global__ __launch_bounds__(256) void grouped_bf16_decode(GroupedArgs a, int ncol_max) {
  constexpr int NT = DC_NT;
  constexpr int WAVE_COLS = GATE_UP ? NT / 2 * 16 : NT * 16;  // output columns per wave
  constexpr int BLOCK_COLS = 4 * WAVE_COLS;
  static_assert(NT % 2 == 0, "gate_up pairs gate and up tiles");

  const int64_t L = xcd_logical_block((int64_t)*a.n_tiles * ncol_max);
  if (L < 0) return;
  const int64_t tile_id = L / ncol_max;
  const int ct = (int)(L % ncol_max);
  const Tile tile = a.tiles[tile_id];
  const ExpertProblem P = pick_problem(a, tile.problem);
  const int col0 = ct * BLOCK_COLS;
  if (col0 >= P.ncols) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wcol0 = col0 + wave * WAVE_COLS;
  const int r16 = lane & 15, kq = lane >> 4;  // operand row / column within a tile, 8-element k group

  // activation row of this lane (A operand: row r16, k 8 kq .. 8 kq + 7 of each 32-slice)
  const bool arow_ok = r16 < tile.rows;
  int64_t g = (int64_t)tile.row_start + min(r16, tile.rows - 1);
  if (P.gather) g = a.sorted_pair[g] / a.k;
  const uint16_t* aptr = (const uint16_t*)P.A + g * P.lda + 8 * kq;

  // weight rows (B operand: output column r16 of each 16-column tile)
  const uint16_t* bptr[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const uint16_t* base;
    int col;
    if (GATE_UP) {
      base = (const uint16_t*)(j < NT / 2 ? P.B0 : P.B1);
      col = wcol0 + (j % (NT / 2)) * 16 + r16;
    } else {
      base = (const uint16_t*)P.B0;
      col = wcol0 + j * 16 + r16;
    }
    col = min(col, P.ncols - 1);
    bptr[j] = base + (int64_t)tile.expert * P.b_stride + (int64_t)col * P.K + 8 * kq;
  }

  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const bf16x8 zero8 = {};
  int k0 = 0;
  for (; k0 + 32 * DC_U <= P.K; k0 += 32 * DC_U) {
    bf16x8 av[DC_U], bv[DC_U][NT];
#pragma unroll
    for (int u = 0; u < DC_U; ++u) {
#pragma unroll
      for (int j = 0; j < NT; ++j) bv[u][j] = *(const bf16x8*)(bptr[j] + k0 + 32 * u);
      av[u] = arow_ok ? *(const bf16x8*)(aptr + k0 + 32 * u) : zero8;
    }
#pragma unroll
    for (int u = 0; u < DC_U; ++u)
#pragma unroll
      for (int j = 0; j < NT; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u], bv[u][j], acc[j], 0, 0, 0);
  }
  for (; k0 < P.K; k0 += 32) {  // K is a multiple of 64: at most one short iteration
    bf16x8 bv[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) bv[j] = *(const bf16x8*)(bptr[j] + k0);
    const bf16x8 av = arow_ok ? *(const bf16x8*)(aptr + k0) : zero8;
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv[j], acc[j], 0, 0, 0);
  }

  // 16x16 C layout: lane holds column lane % 16, rows 4 (lane / 16) + i.
  uint16_t* out = (uint16_t*)P.out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * kq + i;
    if (row >= tile.rows) continue;
    const int64_t orow = (int64_t)tile.row_start + row;
    if (GATE_UP) {
#pragma unroll
      for (int j = 0; j < NT / 2; ++j) {
        const int col = wcol0 + j * 16 + r16;
        if (col < P.ncols) out[orow * P.ldo + col] = bf16_rne(silu_mul(acc[j][i], acc[j + NT / 2][i]));
      }
    } else {
      const float sc = P.scale_rows ? a.topk_w[a.sorted_pair[orow]] : 1.0f;
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int col = wcol0 + j * 16 + r16;
        if (col < P.ncols) out[orow * P.ldo + col] = bf16_rne(acc[j][i] * sc);
      }
    }
  }
}

template <bool GATE_UP>
hipError_t launch(const GroupedArgs& a, int64_t max_tile_count, hipStream_t s) {
  constexpr int BLOCK_COLS = 4 * (GATE_UP ? DC_NT / 2 * 16 : DC_NT * 16);
  int nc = 0;
  for (int p = 0; p < 2; ++p)
    if (a.prob[p].out) nc = max(nc, (a.prob[p].ncols + BLOCK_COLS - 1) / BLOCK_COLS);
  const int64_t blocks = (max_tile_count * nc + 7) / 8 * 8;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(grouped_bf16_decode<GATE_UP>, dim3((unsigned)blocks), dim3(256), 0, s, a, nc);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bf16_decode(bool gate_up, const GroupedArgs& a, int64_t max_tile_count, hipStream_t s) {
  return gate_up ? launch<true>(a, max_tile_count, s) : launch<false>(a, max_tile_count, s);
}

}  // namespace moe
