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
// Both operands are K-contiguous (an "NT" product), so each lane feeds v_mfma_f32_32x32x16_bf16 from
// 16-byte LDS reads. bf16 path: 128 x 128 block tile, K step 64, LDS double-buffered (one barrier per
// K step), 4 waves in 2 x 2 each owning 64 x 64 outputs (2 x 2 MFMA tiles). For gate_up a wave's two
// column tiles are the gate and the up projection of the same 32 intermediate columns, so the SwiGLU
// is applied in registers. fp32 path (float32 layers): v_mfma_f32_16x16x4_f32 straight from memory.
#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int BM = 128, BN = 128, BK = 64, PITCH = 72;  // PITCH: bf16 per LDS row (64 + 8 pad)
static_assert(BM == 128 && BN == 128 && BK == 64, "the loader below moves 4 rows of A and B per thread");
constexpr int F_BM = 64, F_BN = 64;                      // fp32 path

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ inline float silu_mul(float g, float u) { return g / (1.0f + expf(-g)) * u; }

// Block id -> logical work id. The hardware deals workgroups to the 8 XCDs round-robin; this remap
// gives each XCD a contiguous run of logical ids, so the column tiles of one row tile (which share
// the gathered A rows) and neighbouring row tiles of one expert (which share B) meet in one L2.
__device__ inline int64_t logical_block() {
  const int64_t b = blockIdx.x, nb = gridDim.x;  // nb is a multiple of 8
  return (b & 7) * (nb >> 3) + (b >> 3);
}

// Field-wise select keeps the problem descriptor in scalar registers (a dynamically indexed
// kernel-argument array would be copied to scratch).
__device__ inline ExpertProblem pick(const GroupedArgs& a, int p) {
  ExpertProblem r;
  const ExpertProblem& x = a.prob[0];
  const ExpertProblem& y = a.prob[1];
  r.A = p ? y.A : x.A;
  r.lda = p ? y.lda : x.lda;
  r.gather = p ? y.gather : x.gather;
  r.B0 = p ? y.B0 : x.B0;
  r.B1 = p ? y.B1 : x.B1;
  r.b_stride = p ? y.b_stride : x.b_stride;
  r.K = p ? y.K : x.K;
  r.ncols = p ? y.ncols : x.ncols;
  r.out = p ? y.out : x.out;
  r.ldo = p ? y.ldo : x.ldo;
  r.scale_rows = p ? y.scale_rows : x.scale_rows;
  return r;
}

template <bool GATE_UP>
__global__ __launch_bounds__(256) void grouped_bf16(GroupedArgs a, int ncol_max) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][(BM + BN) * PITCH];
  __shared__ float wrow[BM];

  const int64_t L = logical_block();
  const int64_t tile_id = L / ncol_max;
  const int ct = (int)(L % ncol_max);
  if (tile_id >= *a.n_tiles) return;
  const Tile tile = a.tiles[tile_id];
  const ExpertProblem P = pick(a, tile.problem);
  constexpr int COLS = GATE_UP ? BN / 2 : BN;
  const int col0 = ct * COLS;
  if (col0 >= P.ncols) return;

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lrow = t >> 3, kc = (t & 7) * 8;  // loader: row lrow + 32 i, 8 bf16 at kc

  const uint16_t* arow[4];
  const uint16_t* brow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = min(lrow + 32 * i, tile.rows - 1);
    int64_t g = (int64_t)tile.row_start + r;
    if (P.gather) g = a.sorted_pair[g] / a.k;
    arow[i] = (const uint16_t*)P.A + g * P.lda + kc;
    const int j = lrow + 32 * i;
    const uint16_t* base;
    int c;
    if (GATE_UP) {
      base = (const uint16_t*)(j < BN / 2 ? P.B0 : P.B1);
      c = min(col0 + (j & (BN / 2 - 1)), P.ncols - 1);
    } else {
      base = (const uint16_t*)P.B0;
      c = min(col0 + j, P.ncols - 1);
    }
    brow[i] = base + (int64_t)tile.expert * P.b_stride + (int64_t)c * P.K + kc;
  }
  if (!GATE_UP && t < BM) {
    const int r = min(t, tile.rows - 1);
    wrow[t] = P.scale_rows ? a.topk_w[a.sorted_pair[tile.row_start + r]] : 1.0f;
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  uint4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;  // the next K step, in flight during the MFMAs
#define MOE_GLOAD(k0)                       \
  ra0 = *(const uint4*)(arow[0] + (k0));    \
  ra1 = *(const uint4*)(arow[1] + (k0));    \
  ra2 = *(const uint4*)(arow[2] + (k0));    \
  ra3 = *(const uint4*)(arow[3] + (k0));    \
  rb0 = *(const uint4*)(brow[0] + (k0));    \
  rb1 = *(const uint4*)(brow[1] + (k0));    \
  rb2 = *(const uint4*)(brow[2] + (k0));    \
  rb3 = *(const uint4*)(brow[3] + (k0));
#define MOE_LSTORE(buf)                                                \
  {                                                                    \
    uint16_t* As_ = lds[(buf)] + lrow * PITCH + kc;                    \
    uint16_t* Bs_ = lds[(buf)] + (BM + lrow) * PITCH + kc;             \
    *(uint4*)(As_) = ra0;                                              \
    *(uint4*)(As_ + 32 * PITCH) = ra1;                                 \
    *(uint4*)(As_ + 64 * PITCH) = ra2;                                 \
    *(uint4*)(As_ + 96 * PITCH) = ra3;                                 \
    *(uint4*)(Bs_) = rb0;                                              \
    *(uint4*)(Bs_ + 32 * PITCH) = rb1;                                 \
    *(uint4*)(Bs_ + 64 * PITCH) = rb2;                                 \
    *(uint4*)(Bs_ + 96 * PITCH) = rb3;                                 \
  }

  const int nk = P.K / BK;
  MOE_GLOAD(0)
  MOE_LSTORE(0)
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) {
      MOE_GLOAD((kt + 1) * BK)
    }
    const uint16_t* As = lds[kt & 1];
    const uint16_t* Bs = lds[kt & 1] + BM * PITCH;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      const int ko = kk + 8 * (lane >> 5);
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = *(const bf16x8*)(As + (wm * 64 + i * 32 + (lane & 31)) * PITCH + ko);
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int br = GATE_UP ? (j * (BN / 2) + wn * 32) : (wn * 64 + j * 32);
        bfr[j] = *(const bf16x8*)(Bs + (br + (lane & 31)) * PITCH + ko);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) {
      MOE_LSTORE((kt + 1) & 1)
    }
    __syncthreads();
  }
#undef MOE_GLOAD
#undef MOE_LSTORE

  // 32x32 C layout: lane holds column lane % 32, rows 8 (r / 4) + 4 (lane / 32) + r % 4.
  uint16_t* out = (uint16_t*)P.out;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (row >= tile.rows) continue;
      const int64_t orow = (int64_t)tile.row_start + row;
      if (GATE_UP) {
        const int col = col0 + wn * 32 + (lane & 31);
        if (col < P.ncols) out[orow * P.ldo + col] = f32_to_bf16_rne(silu_mul(acc[i][0][r], acc[i][1][r]));
      } else {
        const float sc = wrow[row];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int col = col0 + wn * 64 + j * 32 + (lane & 31);
          if (col < P.ncols) out[orow * P.ldo + col] = f32_to_bf16_rne(acc[i][j][r] * sc);
        }
      }
    }
}

// fp32 layers: 64 x 64 block tile, 4 waves in 2 x 2, each 32 x 32 as 2 x 2 tiles of
// v_mfma_f32_16x16x4_f32 (A: row lane % 16, k lane / 16; C: column lane % 16, rows 4 (lane / 16) + r).
// For gate_up a wave's j = 0 / j = 1 tiles are the gate / up projections of 16 intermediate columns.
template <bool GATE_UP>
__global__ __launch_bounds__(256) void grouped_f32(GroupedArgs a, int ncol_max) {
  const int64_t L = logical_block();
  const int64_t tile_id = L / ncol_max;
  const int ct = (int)(L % ncol_max);
  if (tile_id >= *a.n_tiles) return;
  const Tile tile = a.tiles[tile_id];
  const ExpertProblem P = pick(a, tile.problem);
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
        if (col < P.ncols) out[orow * P.ldo + col] = silu_mul(acc[i][0][q], acc[i][1][q]);
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
  const int64_t routed = pairs / bm + (pairs < E ? pairs : E);
  const int64_t shared = n_shared_problem ? (N + bm - 1) / bm : 0;
  return routed + shared;
}

int gemm_bm(int dtype, int64_t, int, int) { return dtype == MOE_F32 ? F_BM : BM; }

hipError_t launch_gate_up(int dtype, const GroupedArgs& a, int64_t max_tile_count, hipStream_t s) {
  if (dtype == MOE_F32) return launch_grouped(grouped_f32<true>, a, max_tile_count, F_BN / 2, s);
  return launch_grouped(grouped_bf16<true>, a, max_tile_count, BN / 2, s);
}

hipError_t launch_down(int dtype, const GroupedArgs& a, int64_t max_tile_count, hipStream_t s) {
  if (dtype == MOE_F32) return launch_grouped(grouped_f32<false>, a, max_tile_count, F_BN, s);
  return launch_grouped(grouped_bf16<false>, a, max_tile_count, BN, s);
}

}  // namespace moe
