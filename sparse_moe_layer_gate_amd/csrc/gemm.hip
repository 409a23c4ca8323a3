// Grouped expert GEMMs on the matrix cores.
//
// "MoE Forward" (GLM-4.5), eq. E_i: E_i(x) = W_down (SiLU(W_gate x) * W_up x), bias-free, with gate and
// up packed as gate_up[i] of shape (2 d, D) (rows [0, d) gate, [d, 2d) up). The routed experts and the
// shared expert (same MLP, width d * n_shared, its own matrices; "Shared output") run in one launch
// per GEMM: a device-built tile list names, for each row tile, its problem (routed / shared), expert,
// first row and row count.
//
//   gate_up launch: H[r, c] = SiLU(sum_t A[r, t] Wg[c, t]) * (sum_t A[r, t] Wu[c, t])
//                   A rows are rows of x gathered through sorted_pair (routed) or x itself (shared).
//   down launch:    Y[r, c] = s_r * sum_j H[r, j] Wd[c, j], with s_r = w[sorted_pair[r]] for routed
//                   rows (the mixture weight, alpha included) and 1 for the shared expert.
//
// Both operands are K-contiguous (an "NT" product). This file holds the float32 kernels
// (v_mfma_f32_16x16x4_f32 straight from memory) and the launch choice; the bf16 kernels are in
// gemm_bf16.hip.
#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int F_BM = 64, F_BN = 64;                      // fp32 path

// fp32 layers: 64 x 64 block tile, 4 waves in 2 x 2, each 32 x 32 as 2 x 2 tiles of
// v_mfma_f32_16x16x4_f32 (A: row lane % 16, k lane / 16; C: column lane % 16, rows 4 (lane / 16) + r).
// For gate_up a wave's j = 0 / j = 1 tiles are the gate / up projections of 16 intermediate columns.
template <bool GATE_UP>
__global__ __launch_bounds__(256) void grouped_f32(GroupedArgs a, int ncol_max) {
  const int64_t L = xcd_logical_block((int64_t)*a.n_tiles * ncol_max);
  if (L < 0) return;
  const int64_t tile_id = L / ncol_max;
  const int ct = (int)(L % ncol_max);
  const Tile tile = a.tiles[tile_id];
  const ExpertProblem P = pick_problem(a, tile.problem);
  constexpr int COLS = GATE_UP ? F_BN / 2 : F_BN;
  const int col0 = ct * COLS;
  if (col0 >= P.ncols) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const float* ap[2];
  const float* bp[2];
  float sc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = min(wm * 32 + i * 16 + (lane & 15), tile.rows - 1);
    int64_t g = (int64_t)tile.row_start + r;
    if (P.gather) g = a.sorted_pair[g] / a.k;
    ap[i] = (const float*)P.A + g * P.lda + (lane >> 4);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int rr = min(wm * 32 + i * 16 + 4 * (lane >> 4) + q, tile.rows - 1);
      sc[i][q] = (!GATE_UP && P.scale_rows) ? a.topk_w[a.sorted_pair[tile.row_start + rr]] : 1.0f;
    }
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const float* base;
    int c;
    if (GATE_UP) {
      base = (const float*)(j == 0 ? P.B0 : P.B1);
      c = min(col0 + wn * 16 + (lane & 15), P.ncols - 1);
    } else {
      base = (const float*)P.B0;
      c = min(col0 + wn * 32 + j * 16 + (lane & 15), P.ncols - 1);
    }
    bp[j] = base + (int64_t)tile.expert * P.b_stride + (int64_t)c * P.K + (lane >> 4);
  }
  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < P.K; k0 += 4) {
    float av[2], bv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) av[i] = ap[i][k0];
#pragma unroll
    for (int j = 0; j < 2; ++j) bv[j] = bp[j][k0];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[i], bv[j], acc[i][j], 0, 0, 0);
  }
  float* out = (float*)P.out;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = wm * 32 + i * 16 + 4 * (lane >> 4) + q;
      if (row >= tile.rows) continue;
      const int64_t orow = (int64_t)tile.row_start + row;
      if (GATE_UP) {
        const int col = col0 + wn * 16 + (lane & 15);
        if (col < P.ncols) out[orow * P.ldo + col] = swiglu(acc[i][0][q], acc[i][1][q], a.swiglu_limit);
      } else {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = col0 + wn * 32 + j * 16 + (lane & 15);
          if (col < P.ncols) out[orow * P.ldo + col] = acc[i][j][q] * sc[i][q];
        }
      }
    }
}

int ncol_tiles(const GroupedArgs& a, int cols_per_tile) {
  int m = 0;
  for (int p = 0; p < 2; ++p) {
    if (!a.prob[p].out) continue;
    const int n = (a.prob[p].ncols + cols_per_tile - 1) / cols_per_tile;
    m = n > m ? n : m;
  }
  return m;
}

template <typename Kern>
hipError_t launch_grouped(Kern kern, const GroupedArgs& a, int64_t max_tile_count, int cols_per_tile, hipStream_t s) {
  const int nc = ncol_tiles(a, cols_per_tile);
  int64_t blocks = max_tile_count * nc;
  blocks = (blocks + 7) / 8 * 8;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, s, a, nc);
  return hipGetLastError();
}

}  // namespace

int64_t max_tiles(int64_t N, int k, int E, int n_shared_problem, int bm) {
  const int64_t pairs = N * k;
  int64_t routed = pairs / bm + (pairs < E ? pairs : E);
  // padding of the 256-row lists (MOE_TILE_ALIGN, MOE_HOT_ALIGN): at most that many empty tiles less one
  // per expert
  const int pad = (MOE_HOT_TILES > 0 && MOE_HOT_ALIGN > MOE_TILE_ALIGN) ? MOE_HOT_ALIGN : MOE_TILE_ALIGN;
  if (bm == 256 && pad > 1) routed += (int64_t)(pad - 1) * (pairs < E ? pairs : E);
  const int64_t shared = n_shared_problem ? (N + bm - 1) / bm : 0;
  return routed + shared;
}

#ifndef MOE_DECODE_ROWS
#define MOE_DECODE_ROWS 4  // average rows per expert below which the decode kernels run
#endif

int gemm_bm(int dtype, int64_t N, int k, int E) {
  if (dtype == MOE_F32) return F_BM;
  // Measured (layer ms, decode kernel against the persistent prefill kernel): with uniform routing
  // (GLM-5 weights) they are within ~3% of each other from 3 to 6 rows per expert and the prefill
  // kernel leads from 7 on (N = 224: 3.30 -> 3.14); with skewed routing (GLM-4.5 weights) the decode
  // kernel's 16-row tiles re-stream a hot expert's weights once per 16 rows and lose 30-43% already at
  // 4.8-6.4 rows per expert (N = 96: 0.61 against 0.47 ms, N = 128: 0.74 against 0.52 ms).
  if (N * k < (int64_t)MOE_DECODE_ROWS * E) return 16;  // weight-streaming decode kernel, 16-row tiles
  return 256;                                           // prefill kernels, 256-row tiles
}

#ifndef MOE_PICK_BAND_ROWS
#define MOE_PICK_BAND_ROWS 12  // average rows per expert below which the kernel choice is left to the device
#endif
#ifndef MOE_PICK_MAX_ROWS
#define MOE_PICK_MAX_ROWS 24  // largest expert's rows up to which such a batch runs the decode kernels
#endif

// Between MOE_DECODE_ROWS and MOE_PICK_BAND_ROWS rows per expert on average the better kernel depends on
// how the rows spread over the experts, which only the device knows: the forward builds both a 16-row
// and a 256-row tile list, and the scan kernel empties the one not taken (the decode list when the
// largest expert has more than MOE_PICK_MAX_ROWS rows). Measured (layer ms, prefill against decode
// kernels): uniform routing, GLM-5 weights N = 128 / 192 / 256: 3.00 / 3.18 / 3.24 against 2.70 / 2.93 /
// 3.16 (largest expert 13 / 17 / 23 rows), the 288-expert shape N = 192 / 256: 2.65 / 2.80 against
// 2.24 / 2.42 (20 / 24 rows); skewed GLM-4.5 routing N = 96 / 128 (largest expert 51 / 66 rows): 0.47 /
// 0.51 against 0.65 / 0.82; and from ~12 rows per expert the prefill kernels lead under uniform routing
// too (GLM-5 N = 384, 28 rows: 3.39 against 3.98).
int device_pick_rows(int dtype, int64_t N, int k, int E) {
  if (dtype != MOE_BF16) return 0;
  const int64_t pairs = N * k;
  if (pairs < (int64_t)MOE_DECODE_ROWS * E || pairs >= (int64_t)MOE_PICK_BAND_ROWS * E) return 0;
  return MOE_PICK_MAX_ROWS;
}

int tile_plan_rows(int i) { return i == 0 ? MOE_DECODE_ROWS : MOE_PICK_BAND_ROWS; }

#ifndef MOE_SMALL_EXPERT_ROWS
#define MOE_SMALL_EXPERT_ROWS 128  // 256-row tiles: experts with at most half a tile of rows
#endif

// Tile order (see build_tiles): the single tiles of experts with at most half a tile of rows, which
// mostly stream their expert's weights, go after the other tiles, so that the rasterization rectangles
// of the prefill kernels hold the large experts' tiles together. (An earlier order merged them evenly
// among the others to balance the XCDs' runs before the kernels claimed work per XCD; with the claiming
// kernels and 2 x 16 rectangles the separated order is 2-4% faster on GLM-5 and Air and equal on the
// skewed GLM-4.5 layer.) Each large expert's tiles are padded to an even number of list slots
// (MOE_TILE_ALIGN), so that its tiles share a rectangle.
int small_expert_rows(int dtype, int bm) { return (dtype == MOE_BF16 && bm == 256) ? MOE_SMALL_EXPERT_ROWS : 0; }

hipError_t launch_gate_up(int dtype, const GroupedArgs& a, int64_t max_tile_count, hipStream_t s) {
  if (dtype == MOE_F32) return launch_grouped(grouped_f32<true>, a, max_tile_count, F_BN / 2, s);
  if (a.bm == 16) return launch_bf16_decode(true, a, max_tile_count, s);
  return launch_bf16_prefill(true, a.bm, a, max_tile_count, s);
}

hipError_t launch_down(int dtype, const GroupedArgs& a, int64_t max_tile_count, hipStream_t s) {
  if (dtype == MOE_F32) return launch_grouped(grouped_f32<false>, a, max_tile_count, F_BN, s);
  if (a.bm == 16) return launch_bf16_decode(false, a, max_tile_count, s);
  return launch_bf16_prefill(false, a.bm, a, max_tile_count, s);
}

}  // namespace moe
