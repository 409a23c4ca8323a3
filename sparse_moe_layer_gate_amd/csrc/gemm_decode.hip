// Grouped bf16 expert GEMMs for token-poor (decode) batches.
//
// With one or two tokens per expert the layer is a weight stream ("Module 02 -- MoE: Capacity, Work,
// and Traffic", section 1: traffic, not arithmetic, governs decode), so this kernel is built to keep
// many weight bytes in flight and to move each weight byte once, in whole cache lines:
//  - row tiles of at most 16 rows (the tile list is built with 16 rows per tile);
//  - each wave owns NT 16-column tiles of one expert (gate_up: NT/2 gate and NT/2 up tiles, SwiGLU in
//    registers; down: NT tiles, each row scaled by its weight) and works alone: no block barriers;
//  - loaded straight into registers, the MFMA operand layout (v_mfma_f32_16x16x32_bf16: a lane holds
//    8 k of one row) makes every load touch 16 rows x 64 bytes, half of each 128-byte line, which
//    costs about a fifth of the stream rate. Instead each wave copies its rows into a private LDS ring
//    with global_load_lds_dwordx4, CPR 16-byte chunks per row and stage (whole lines), S stages deep,
//    and reads them back in MFMA layout. The ring also holds the wave's activation rows, so every
//    stage is the same fixed number of DMA instructions and one vmcnt wait orders the ring.
#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#ifndef MOE_DC_U
#define MOE_DC_U 4
#endif
#ifndef MOE_DC_S
#define MOE_DC_S 2
#endif
#ifndef MOE_DC_NT
#define MOE_DC_NT 2
#endif
// Cache policy of the weight loads: non-temporal (the NT bit, 2 on gfx950). Each weight byte is read
// once per launch, and the hint keeps the stream from allocating in the caches: GLM-5 decode gate_up
// 1.28-1.33 -> 1.17 ms (6.6 TB/s), down 0.62 -> 0.57 ms; the activation rows, re-read by every wave
// of a tile, keep the default policy.
#ifndef MOE_DC_WEIGHT_CPOL
#define MOE_DC_WEIGHT_CPOL 2
#endif

template <bool GATE_UP, int WPB>
struct DecodeTile {
  static constexpr int NT = MOE_DC_NT;  // 16-column weight tiles per wave
  static constexpr int U = MOE_DC_U;    // 32-wide K slices per stage
  static constexpr int S = MOE_DC_S;    // ring depth (stages)
  static constexpr int SK = 32 * U;     // K elements per stage
  static constexpr int CPR = SK / 8;    // 16-byte chunks per row and stage
  static constexpr int RPI = 64 / CPR;  // rows per DMA instruction
  static constexpr int QPT = 16 / RPI;  // DMA instructions per 16-row tile and stage
  static constexpr int TILE_BYTES = 16 * SK * 2;
  static constexpr int STAGE_BYTES = (NT + 1) * TILE_BYTES;  // activation tile, then NT weight tiles
  static constexpr int WAVE_BYTES = S * STAGE_BYTES;
  static constexpr int NDMA = (NT + 1) * QPT;  // DMA instructions per stage
  static constexpr int WAVE_COLS = GATE_UP ? NT / 2 * 16 : NT * 16;  // output columns per wave
  static constexpr int BLOCK_COLS = WPB * WAVE_COLS;  // WPB waves per block
  static_assert(!GATE_UP || NT % 2 == 0, "gate_up pairs gate and up tiles");
  static_assert(CPR >= 8 && CPR <= 64 && 64 % CPR == 0, "a DMA instruction covers whole 128-byte lines");
  static_assert((S - 1) * NDMA < 64, "vmcnt is 6 bits");
  static_assert(4 * WAVE_BYTES <= 160 * 1024, "LDS per CU");

  // Chunk swizzle: chunk c of row r sits in slot c ^ sig(r). For each MFMA operand read (16 lanes of
  // one k group over rows 0..15) the 16 slots then fall in distinct 16-byte bank groups.
  __device__ static int sig(int r) { return CPR >= 16 ? r : r / (16 / CPR); }
};

template <bool GATE_UP, int WPB>
__global__ __launch_bounds__(64 * WPB) void grouped_bf16_decode(GroupedArgs a, int ncol_max) {
  using T = DecodeTile<GATE_UP, WPB>;
  constexpr int NT = T::NT, U = T::U, S = T::S, SK = T::SK, CPR = T::CPR, RPI = T::RPI, QPT = T::QPT;
  __shared__ __attribute__((aligned(1024))) char lds[WPB * T::WAVE_BYTES];

  const int64_t L = xcd_logical_block((int64_t)*a.n_tiles * ncol_max);
  if (L < 0) return;
  const int64_t tile_id = L / ncol_max;
  const int ct = (int)(L % ncol_max);
  const Tile tile = a.tiles[tile_id];
  const ExpertProblem P = pick_problem(a, tile.problem);
  const int col0 = ct * T::BLOCK_COLS;
  if (col0 >= P.ncols) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wcol0 = col0 + wave * T::WAVE_COLS;
  char* const ring = lds + wave * T::WAVE_BYTES;

  // DMA sources of this lane: in instruction q of a tile it moves chunk chunk[q] of tile row
  // q * RPI + lane / CPR into slot lane % CPR of that row. Every lane of every instruction is active:
  // activation rows past tile.rows repeat the last valid row and weight rows past ncols repeat the
  // last column (neither reaches a stored output), so each stage is exactly NDMA instructions.
  const uint16_t* src[NT + 1][QPT];
  int chunk[QPT];
#pragma unroll
  for (int q = 0; q < QPT; ++q) {
    const int r = q * RPI + lane / CPR;
    chunk[q] = (lane % CPR) ^ T::sig(r);
    int64_t g = (int64_t)tile.row_start + min(r, tile.rows - 1);
    if (P.gather) g = a.sorted_pair[g] / a.k;
    src[0][q] = (const uint16_t*)P.A + g * P.lda;
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const uint16_t* base;
      int col;
      if (GATE_UP) {
        base = (const uint16_t*)(j < NT / 2 ? P.B0 : P.B1);
        col = wcol0 + (j % (NT / 2)) * 16 + r;
      } else {
        base = (const uint16_t*)P.B0;
        col = wcol0 + j * 16 + r;
      }
      col = min(col, P.ncols - 1);
      src[1 + j][q] = base + (int64_t)tile.expert * P.b_stride + (int64_t)col * P.K;
    }
  }

  const int nst = (P.K + SK - 1) / SK;
  const int ktail = P.K - (nst - 1) * SK;  // K elements of the last stage (a multiple of 32)

  // Stage t -> ring slot t % S. In a short last stage, chunks past K load the last chunk in K instead
  // (their slots are never read), keeping every address inside its row.
  auto issue = [&](int t) {
    char* st = ring + (t % S) * T::STAGE_BYTES;
    const int kmax = t == nst - 1 ? ktail : SK;
#pragma unroll
    for (int q = 0; q < QPT; ++q) {
      const int64_t ke = (int64_t)t * SK + 8 * min(chunk[q], kmax / 8 - 1);
      __builtin_amdgcn_global_load_lds((const void*)(src[0][q] + ke), (lds_void*)(st + q * 1024), 16, 0, 0);
#pragma unroll
      for (int j = 1; j <= NT; ++j)
        __builtin_amdgcn_global_load_lds((const void*)(src[j][q] + ke), (lds_void*)(st + j * T::TILE_BYTES + q * 1024),
                                         16, 0, MOE_DC_WEIGHT_CPOL);
    }
  };

  const int r16 = lane & 15, kq = lane >> 4;  // MFMA operand row and 8-element k group of this lane
  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int t = 0; t < S - 1; ++t)
    if (t < nst) issue(t);
  for (int t = 0; t < nst; ++t) {
    // The refill of slot (t - 1) % S follows the reads of stage t - 1, which have completed: their
    // values fed that stage's MFMAs.
    if (t + S - 1 < nst) {
      issue(t + S - 1);
      wait_vmcnt<(S - 1) * T::NDMA>();
    } else {
      wait_vmcnt<0>();
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const char* st = ring + (t % S) * T::STAGE_BYTES;
    const int kmax = t == nst - 1 ? ktail : SK;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (32 * u >= kmax) break;
      const int off = r16 * CPR * 16 + 16 * ((4 * u + kq) ^ T::sig(r16));
      const bf16x8 av = *(const bf16x8*)(st + off);
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const bf16x8 bv = *(const bf16x8*)(st + (1 + j) * T::TILE_BYTES + off);
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[j], 0, 0, 0);
      }
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
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
        if (col < P.ncols) out[orow * P.ldo + col] = bf16_rne(swiglu_bf16(acc[j][i], acc[j + NT / 2][i], a.swiglu_limit));
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

#ifndef MOE_DC_ONE_WAVE_BLOCKS
#define MOE_DC_ONE_WAVE_BLOCKS 1024
#endif

template <bool GATE_UP, int WPB>
int64_t decode_blocks(const GroupedArgs& a, int64_t max_tile_count, int* nc) {
  constexpr int BLOCK_COLS = DecodeTile<GATE_UP, WPB>::BLOCK_COLS;
  *nc = 0;
  for (int p = 0; p < 2; ++p)
    if (a.prob[p].out) *nc = max(*nc, (a.prob[p].ncols + BLOCK_COLS - 1) / BLOCK_COLS);
  return (max_tile_count * *nc + 7) / 8 * 8;
}

// Four-wave blocks, or one-wave blocks when a batch has too few tiles to give every CU several blocks
// (a few tokens: at one token the 9 tiles of GLM-5 make 288 four-wave blocks for 256 CUs, so a quarter
// of the CUs stream twice as long as the rest); the waves work alone either way.
template <bool GATE_UP>
hipError_t launch(const GroupedArgs& a, int64_t max_tile_count, hipStream_t s) {
  int nc = 0;
  int64_t blocks = decode_blocks<GATE_UP, 4>(a, max_tile_count, &nc);
  if (blocks == 0) return hipSuccess;
  if (blocks < MOE_DC_ONE_WAVE_BLOCKS) {
    blocks = decode_blocks<GATE_UP, 1>(a, max_tile_count, &nc);
    hipLaunchKernelGGL((grouped_bf16_decode<GATE_UP, 1>), dim3((unsigned)blocks), dim3(64), 0, s, a, nc);
  } else {
    hipLaunchKernelGGL((grouped_bf16_decode<GATE_UP, 4>), dim3((unsigned)blocks), dim3(256), 0, s, a, nc);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bf16_decode(bool gate_up, const GroupedArgs& a, int64_t max_tile_count, hipStream_t s) {
  return gate_up ? launch<true>(a, max_tile_count, s) : launch<false>(a, max_tile_count, s);
}

}  // namespace moe
