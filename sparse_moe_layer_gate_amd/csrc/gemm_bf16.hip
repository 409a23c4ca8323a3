// Grouped bf16 expert GEMMs for token-rich (prefill) batches: 256-row tiles.
//
// Same products as the generic grouped kernels ("MoE Forward", eq. E_i: the gate_up GEMM with the
// SwiGLU applied in registers, and the down GEMM scaled by the mixture weight w_{n,i}), laid out for
// gfx950. Two kernels:
//  - grouped_bf16_w8 (the one the forward runs): eight waves, two per SIMD, each wave computing a
//    64 x 128 share of a 256 x 256 tile and issuing an eighth of every step's loads (described where
//    it is defined); persistent, one block per CU claiming tiles per XCD;
//  - grouped_bf16_lds (fallback when x spans 4 GiB or more, where the eight-wave kernel's 32-bit
//    buffer offsets do not reach): four waves, each 128 x 128 of the tile.
// Common to both:
//  - operands go global -> LDS directly (lane l of a wave writes bytes [16 l, 16 l + 16) of a 1 KiB
//    run), no register staging;
//  - LDS rows are BK bf16 long, unpadded; the 16-byte chunks of a row are XOR-swizzled by the row's
//    position so that the MFMA operand reads (32 rows at one k offset) hit distinct banks;
//  - v_mfma_f32_32x32x16_bf16 tiles; 32-row MFMA sub-tiles past a tile's valid rows are skipped, so a
//    sparsely filled tile (a rarely chosen expert) costs little MFMA time;
//  - blocks follow an XCD-aware order over the valid tiles with a row-tile-major rasterization.
#include <hip/hip_runtime.h>

#include <atomic>

#include "moe_internal.h"

namespace moe {
namespace {

// Rasterization: row tiles per column sweep (see grouped_bf16_lds), for gate_up and down.
#ifndef MOE_PF_GROUP_ROWS_GU
#define MOE_PF_GROUP_ROWS_GU 32
#endif
#ifndef MOE_PF_GROUP_ROWS_DN
#define MOE_PF_GROUP_ROWS_DN 16
#endif
// L2 line touches ahead of the ring (see PrefillTile::TOUCH): distance in K steps (0: off) for the
// gate_up and down GEMMs, the smallest routed-expert row count that turns them on, and which operands
// (bit 0: A, bit 1: B) are touched.
#ifndef MOE_PF_TOUCH_GU
#define MOE_PF_TOUCH_GU 0
#endif
#ifndef MOE_PF_TOUCH_DN
#define MOE_PF_TOUCH_DN 2
#endif
#ifndef MOE_PF_TOUCH_MIN_ROWS
#define MOE_PF_TOUCH_MIN_ROWS 1024
#endif
#ifndef MOE_PF_TOUCH_GU_OPS
#define MOE_PF_TOUCH_GU_OPS 3
#endif
#ifndef MOE_PF_TOUCH_DN_OPS
#define MOE_PF_TOUCH_DN_OPS 1
#endif

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
template <int V>
struct IntC {
  static constexpr int value = V;
};
template <bool V>
struct BoolC {
  static constexpr bool value = V;
};

template <int BM, int BK, int STAGES, bool GATE_UP>
struct PrefillTile {
  static constexpr int BN = 256;
  static constexpr int WM = BM == 256 ? 2 : 1, WN = 4 / WM;
  static constexpr int WAVE_M = BM / WM, WAVE_N = BN / WN;
  static constexpr int TM = WAVE_M / 32, TN = WAVE_N / 32;
  static constexpr int ROWB = BK * 2;        // bytes per LDS row
  static constexpr int CPR = BK / 8;         // 16-byte chunks per row
  static constexpr int NA = BM * CPR / 256;  // direct loads per thread per K step (A)
  static constexpr int NB = BN * CPR / 256;  // (B)
  static constexpr int LPS = NA + NB;
  static constexpr int STAGE_BYTES = (BM + BN) * ROWB;
  static constexpr int COLS = GATE_UP ? BN / 2 : BN;  // output columns per block
  static_assert(TN % 2 == 0, "gate_up pairs gate and up column tiles inside a wave");
  static_assert(CPR == 8 || CPR == 4, "BK is 64 or 32");
  // L2 warm-up: with a two-stage ring a step's operands have one step of compute to arrive, less
  // than a miss to HBM takes. For tiles of large experts (whose B is shared by many row tiles and stays
  // cached, so the A rows are what misses) each lane also touches one line of the selected operands
  // TOUCH steps ahead (4-byte direct loads into a scratch word), so the later full loads hit L2.
  // Measured: it pays for down on row-heavy experts; elsewhere the extra requests cost more.
  static constexpr int TOUCH = STAGES == 2 ? (GATE_UP ? MOE_PF_TOUCH_GU : MOE_PF_TOUCH_DN) : 0;
  static constexpr int TOUCH_OPS = GATE_UP ? MOE_PF_TOUCH_GU_OPS : MOE_PF_TOUCH_DN_OPS;  // bit 0: A, bit 1: B
  static constexpr int NTOUCH = (TOUCH_OPS & 1) + ((TOUCH_OPS >> 1) & 1);

  // Chunk swizzle: the 16-byte chunk c of LDS row r is stored in slot c ^ swz(r). swz depends on
  // r mod 32 only, and any 8 (and any aligned 16) consecutive rows get distinct slots, so the MFMA
  // operand reads (32 rows x one chunk) are free of bank conflicts for 8- or 16-lane LDS passes.
  __device__ static int swz(int r) {
    r &= 31;
    if (CPR == 8) return (r ^ (r >> 3)) & 7;
    return ((r >> 1) ^ (r >> 3)) & 3;
  }

  // One K step's direct loads: load q of wave w fills the operand's chunks [(4 q + w) 64, + 64).
  __device__ static void issue(char* lds, const uint16_t* const (&srcA)[NA], const uint16_t* const (&srcB)[NB],
                               int kstep, int wave) {
    char* st = lds + (kstep % STAGES) * STAGE_BYTES;
    const int k0 = kstep * BK;
#pragma unroll
    for (int q = 0; q < NA; ++q)
      if (srcA[q])  // rows past the tile's valid rows are not loaded (their MFMA outputs are not stored)
        __builtin_amdgcn_global_load_lds((const void*)(srcA[q] + k0), (lds_void*)(st + (q * 4 + wave) * 1024), 16, 0,
                                         0);
#pragma unroll
    for (int q = 0; q < NB; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(srcB[q] + k0), (lds_void*)(st + BM * ROWB + (q * 4 + wave) * 1024),
                                       16, 0, 0);
  }

  __device__ static int b_row(int j, int wn) {
    if (GATE_UP) return (j < TN / 2 ? 0 : BN / 2) + wn * (WAVE_N / 2) + (j % (TN / 2)) * 32;
    return wn * WAVE_N + j * 32;
  }

  // The K loop for a wave whose first MI 32-row sub-tiles hold valid rows (MI = 0: loads only).
  template <int MI, bool TOUCHING>
  __device__ static __attribute__((always_inline)) void run(char* lds, const uint16_t* const (&srcA)[NA],
                                                            const uint16_t* const (&srcB)[NB], f32x16 (&acc)[TM][TN],
                                                            int nk, int wave, int lane, int wm, int wn,
                                                            const uint16_t* touchA, const uint16_t* touchB,
                                                            int* sink) {
    auto touch = [&](int kstep) {
      if (TOUCH_OPS & 1) __builtin_amdgcn_global_load_lds((const void*)(touchA + kstep * BK), (lds_void*)sink, 4, 0, 0);
      if (TOUCH_OPS & 2) __builtin_amdgcn_global_load_lds((const void*)(touchB + kstep * BK), (lds_void*)sink, 4, 0, 0);
    };
    const int sw = swz(lane & 31);
    const int a_off = (wm * WAVE_M + (lane & 31)) * ROWB;
    int b_off[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) b_off[j] = BM * ROWB + (b_row(j, wn) + (lane & 31)) * ROWB;
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s)
      if (s < nk) issue(lds, srcA, srcB, s, wave);
    if (TOUCHING && TOUCH < nk) touch(TOUCH);
    for (int kt = 0; kt < nk; ++kt) {
      // Step kt's direct loads are this wave's oldest outstanding VMEM ops (only the two touches of
      // step kt + TOUCH, issued right after them, may be newer); once every wave has waited for its
      // own and met at the barrier, step kt is in LDS. The barrier also ends every wave's reads of the
      // stage that the next issue() refills (they fed MFMAs of step kt - 1). A plain s_barrier:
      // __syncthreads() would add a vmcnt(0) wait and drain the prefetches of later steps.
      if (TOUCHING && kt + TOUCH < nk)
        wait_vmcnt<NTOUCH>();
      else if (kt + STAGES - 2 < nk)
        wait_vmcnt<(STAGES - 2) * LPS>();
      else
        wait_vmcnt<0>();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      __builtin_amdgcn_s_barrier();
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      if (kt + STAGES - 1 < nk) {
        issue(lds, srcA, srcB, kt + STAGES - 1, wave);
        if (TOUCHING && kt + 1 + TOUCH < nk) touch(kt + 1 + TOUCH);
      }
      if (MI == 0) continue;
      const char* st = lds + (kt % STAGES) * STAGE_BYTES;
      bf16x8 af[2][MI > 0 ? MI : 1], bfr[2][TN];
      auto load_frags = [&](int kk, int buf) {
        const int coff = ((2 * kk + (lane >> 5)) ^ sw) * 16;
#pragma unroll
        for (int j = 0; j < TN; ++j) bfr[buf][j] = *(const bf16x8*)(st + b_off[j] + coff);
#pragma unroll
        for (int i = 0; i < MI; ++i) af[buf][i] = *(const bf16x8*)(st + a_off + i * 32 * ROWB + coff);
      };
      load_frags(0, 0);
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        if (kk + 1 < BK / 16) load_frags(kk + 1, (kk + 1) & 1);
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk & 1][i], bfr[kk & 1][j], acc[i][j], 0, 0, 0);
      }
      schedule<MI>();
    }
  }

  // Instruction order of one K step: the first slice's operand reads, then each slice's MFMAs with the
  // next slice's reads spread between them, so LDS latency hides under MFMA work.
  template <int MI>
  __device__ static __attribute__((always_inline)) void schedule() {
#ifndef MOE_PF_NO_SCHED
    constexpr int R = MI + TN;   // LDS reads per slice
    constexpr int M = MI * TN;   // MFMAs per slice
    constexpr int PER = M / R > 0 ? M / R : 1;
    __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
#pragma unroll
    for (int kk = 0; kk + 1 < BK / 16; ++kk) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      if (M > PER * R) __builtin_amdgcn_sched_group_barrier(0x008, M - PER * R, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, M, 0);
#endif
  }
};

template <int BM, int BK, int STAGES, bool GATE_UP>
__global__ __launch_bounds__(256, 1) void grouped_bf16_lds(GroupedArgs a, int ncol_max) {
  using T = PrefillTile<BM, BK, STAGES, GATE_UP>;
  constexpr int BN = T::BN, CPR = T::CPR, NA = T::NA, NB = T::NB, TM = T::TM, TN = T::TN;
  constexpr int WAVE_M = T::WAVE_M, WAVE_N = T::WAVE_N;

  constexpr int OUT_BYTES = 4 * WAVE_M * ((GATE_UP ? WAVE_N / 2 : WAVE_N) + 8) * 2;
  constexpr int LDS_BYTES = STAGES * T::STAGE_BYTES > OUT_BYTES ? STAGES * T::STAGE_BYTES : OUT_BYTES;
  __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];
  __shared__ float wrow[BM];
  __shared__ int touch_sink[64];

  // Rasterization: logical ids walk GR row tiles down a column before moving right, so the blocks
  // one XCD runs together share GR-fold the B slices and (32 / GR)-fold the A slices.
  const int64_t n_tiles = *a.n_tiles;
  const int64_t L = xcd_logical_block(n_tiles * ncol_max);
  if (L < 0) return;
  constexpr int GR = GATE_UP ? MOE_PF_GROUP_ROWS_GU : MOE_PF_GROUP_ROWS_DN;
  const int64_t sg = L / ((int64_t)GR * ncol_max), within = L % ((int64_t)GR * ncol_max);
  // the last group may hold fewer than GR row tiles
  const int64_t gr = min((int64_t)GR, n_tiles - sg * GR);
  const int64_t tile_id = sg * GR + within % gr;
  const int ct = (int)(within / gr);
  const Tile tile = a.tiles[tile_id];
  const ExpertProblem P = pick_problem(a, tile.problem);
  const int col0 = ct * T::COLS;
  if (col0 >= P.ncols) return;

  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave / T::WN, wn = wave % T::WN;

  // Global source of each direct load: LDS chunk p is row p / CPR, slot p % CPR, which holds the
  // row's logical chunk slot ^ swz(row).
  const uint16_t* srcA[NA];
  const uint16_t* srcB[NB];
#pragma unroll
  for (int q = 0; q < NA; ++q) {
    const int p = (q * 4 + wave) * 64 + lane;
    const int r = p / CPR, c = (p % CPR) ^ T::swz(r);
    int64_t g = (int64_t)tile.row_start + min(r, tile.rows - 1);
    if (P.gather) g = a.sorted_pair[g] / a.k;
    srcA[q] = (const uint16_t*)P.A + g * P.lda + 8 * c;
    // Skipping a load leaves fewer VMEM ops in flight than the vmcnt thresholds of a deeper ring
    // assume, so only the two-stage ring (which waits for all of them) skips.
    if (STAGES == 2 && r >= tile.rows) srcA[q] = nullptr;
  }
#pragma unroll
  for (int q = 0; q < NB; ++q) {
    const int p = (q * 4 + wave) * 64 + lane;
    const int r = p / CPR, c = (p % CPR) ^ T::swz(r);
    const uint16_t* base;
    int col;
    if (GATE_UP) {
      base = (const uint16_t*)(r < BN / 2 ? P.B0 : P.B1);
      col = min(col0 + (r % (BN / 2)), P.ncols - 1);
    } else {
      base = (const uint16_t*)P.B0;
      col = min(col0 + r, P.ncols - 1);
    }
    srcB[q] = base + (int64_t)tile.expert * P.b_stride + (int64_t)col * P.K + 8 * c;
  }
  // The shared expert's down GEMM (every token) counts as large.
  const bool touch_on = T::TOUCH > 0 && (tile.problem == 1 || !a.offsets ||
                                         a.offsets[tile.expert + 1] - a.offsets[tile.expert] >= MOE_PF_TOUCH_MIN_ROWS);
  // Line-touch sources: A row t (clamped to the tile) and B row t, at chunk 0.
  const uint16_t* touchA;
  const uint16_t* touchB;
  {
    int64_t g = (int64_t)tile.row_start + min(t, tile.rows - 1);
    if (P.gather) g = a.sorted_pair[g] / a.k;
    touchA = (const uint16_t*)P.A + g * P.lda;
    const uint16_t* base;
    int col;
    if (GATE_UP) {
      base = (const uint16_t*)(t % BN < BN / 2 ? P.B0 : P.B1);
      col = min(col0 + t % (BN / 2), P.ncols - 1);
    } else {
      base = (const uint16_t*)P.B0;
      col = min(col0 + t % BN, P.ncols - 1);
    }
    touchB = base + (int64_t)tile.expert * P.b_stride + (int64_t)col * P.K;
  }
  if (!GATE_UP && t < BM) {
    const int r = min(t, tile.rows - 1);
    wrow[t] = P.scale_rows ? a.topk_w[a.sorted_pair[tile.row_start + r]] : 1.0f;
  }

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = P.K / BK;
  const int live_m = tile.rows - wm * WAVE_M;  // valid rows of this wave's slab
  const int mi = live_m <= 0 ? 0 : min(TM, (live_m + 31) / 32);
  auto run = [&](auto mi_tag, auto touch_tag) {
    T::template run<decltype(mi_tag)::value, decltype(touch_tag)::value>(lds, srcA, srcB, acc, nk, wave, lane, wm, wn,
                                                                         touchA, touchB, touch_sink);
  };
  auto run_mi = [&](auto touch_tag) {
    switch (mi) {
      case 0: run(IntC<0>{}, touch_tag); break;
      case 1: run(IntC<1>{}, touch_tag); break;
      case 2: run(IntC<(TM >= 2 ? 2 : 1)>{}, touch_tag); break;
      case 3: run(IntC<(TM >= 3 ? 3 : 1)>{}, touch_tag); break;
      default: run(IntC<TM>{}, touch_tag); break;
    }
  };
  if (T::TOUCH > 0 && touch_on)
    run_mi(BoolC<true>{});
  else
    run_mi(BoolC<false>{});

  // Epilogue through LDS: each wave writes its bf16 results (SwiGLU / weight scale applied) into its
  // own padded region, then stores whole 16-byte row chunks, so a store instruction covers
  // contiguous runs of the output rows instead of 2-byte scatters.
  constexpr int OC = GATE_UP ? WAVE_N / 2 : WAVE_N;  // output columns per wave
  constexpr int OPITCH = OC + 8;                      // bf16 per staged row (16-byte pad: the two
                                                      // half-waves' rows land on disjoint banks)
  __syncthreads();  // every wave is done reading the operand ring
  uint16_t* stage_out = (uint16_t*)lds + wave * (WAVE_M * OPITCH);
  // 32x32 C layout: lane holds column lane % 32, rows 8 (r / 4) + 4 (lane / 32) + r % 4.
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    if (i >= mi) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);  // within the wave slab
      if (GATE_UP) {
#pragma unroll
        for (int j = 0; j < TN / 2; ++j)
          stage_out[row * OPITCH + j * 32 + (lane & 31)] = bf16_rne(swiglu_bf16(acc[i][j][r], acc[i][j + TN / 2][r], a.swiglu_limit));
      } else {
        const float sc = wrow[min(wm * WAVE_M + row, BM - 1)];
#pragma unroll
        for (int j = 0; j < TN; ++j) stage_out[row * OPITCH + j * 32 + (lane & 31)] = bf16_rne(acc[i][j][r] * sc);
      }
    }
  }
  __syncthreads();
  uint16_t* out = (uint16_t*)P.out;
  const int ocol0 = col0 + wn * OC;
  constexpr int CH = OC / 8;  // 16-byte chunks per staged row
  const int rows_here = min(WAVE_M, tile.rows - wm * WAVE_M);
  for (int c = lane; c < rows_here * CH; c += 64) {
    const int row = c / CH, ch = c % CH;
    const int col = ocol0 + ch * 8;
    if (col < P.ncols) {  // ncols is a multiple of 64: a chunk is wholly in or out
      const uint4 v = *(const uint4*)(stage_out + row * OPITCH + ch * 8);
      *(uint4*)(out + ((int64_t)tile.row_start + wm * WAVE_M + row) * P.ldo + col) = v;
    }
  }
}

// ---- eight-wave kernel for 256-row tiles ----
//
// With one wave per SIMD, the wave that issues a K step's direct loads stalls while the texture path
// accepts them (measured: a CU takes 1 KiB global_load_lds_dwordx4 instructions at ~26-30 bytes per
// clock, so the 64 KiB of operands of a 256 x 256 x 64 step hold a wave about as long as the step's
// MFMAs run), and its SIMD's matrix core idles meanwhile. Here each SIMD runs two waves (w and w + 4),
// each with its own 64 x 128 share of the tile, its own fragment reads and an eighth of every step's
// loads: while one of them waits on the load path, the other keeps the matrix core busy.
//  - block tile 256 x 256, BK = 64 (whole 128-byte lines per row and load); A in a two-stage ring, B
//    in a three-stage ring, together all 160 KiB of LDS; rows chunk-swizzled as in PrefillTile;
//  - half g = w / 4 owns tile rows [128 g, 128 g + 128); wave w % 4 = 2 wn + mh owns 64 rows (mh) of
//    that half and 128 B rows (wn), as 2 x 4 tiles of v_mfma_f32_32x32x16_bf16 (gate_up: 64 gate rows
//    and the matching 64 up rows, so SwiGLU pairs stay in one wave);
//  - the waves of half g load rows [128 g, 128 g + 128) of both operands, four direct loads per lane
//    of each per step (buffer_load_dwordx4 ... lds through raw buffer descriptors);
//  - per K step t a wave issues its A loads of step t + 1, reads the fragments of the step's first 32
//    K values, reads the second half's fragments while the first half's MFMAs run, issues its B loads
//    of step t + 2, runs the second half's MFMAs, waits for its loads of step t + 1 and meets the
//    others at a barrier. A stage is refilled only after every wave has passed the barrier that
//    follows its last read; A loads get about one step to land and B loads two.
template <bool GATE_UP>
struct Wave8Tile {
  static constexpr int BM = 256, BN = 256, BK = 64;
  static constexpr int ROWB = BK * 2;          // bytes per LDS row
  static constexpr int OPB = 256 * ROWB;       // one operand's bytes per stage (32 KiB)
  static constexpr int A_STAGES = 2, B_STAGES = 3;
  static constexpr int B_BASE = A_STAGES * OPB;
  static constexpr int RING = (A_STAGES + B_STAGES) * OPB;
  static constexpr int NL = 4;                 // direct loads per lane and quarter (128 rows of one operand)
  static constexpr int COLS = GATE_UP ? BN / 2 : BN;  // output columns per block
  static constexpr int OC = GATE_UP ? 64 : 128;       // output columns per wave
  __device__ static int swz(int r) {
    r &= 31;
    return (r ^ (r >> 3)) & 7;
  }
  // LDS row (within a B stage) of the wave's column tile j
  __device__ static int b_row(int j, int wn) {
    if (GATE_UP) return (j < 2 ? 0 : BN / 2) + wn * 64 + (j & 1) * 32;
    return wn * 128 + j * 32;
  }
};

// Word 3 of a raw (untyped, stride 0) buffer descriptor on gfx9-family parts: 32-bit data format, no
// swizzle, no index stride.
constexpr int kRawBufferWord3 = 0x00020000;
constexpr uint32_t kNoRow = 0xffffffffu;  // marks a direct-load lane that loads nothing

// s_waitcnt lgkmcnt(0), other counters at their maximum
__device__ inline void wait_lgkm0() { __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8)); }
// Workgroup barrier without the memory-counter waits __syncthreads() adds (callers wait for exactly
// what they need first); the signal fences keep the compiler from moving memory accesses across it.
__device__ inline void bare_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// The K loop of one wave. offA / offB: byte offsets of this wave's direct-load sources in its half's
// rows (A lanes of rows past the tile's valid rows load nothing; B is never skipped, so a wave's newest
// NL loads are always B loads, which is what the vmcnt(NL) waits rely on).
template <bool GATE_UP, int MI>
__device__ __attribute__((always_inline)) inline void wave8_loop(char* lds, __amdgpu_buffer_rsrc_t rsrcA,
                                                                 const uint32_t (&offA)[4], __amdgpu_buffer_rsrc_t rsrcB,
                                                                 const uint32_t (&offB)[4], f32x16 (&acc)[2][4], int nk,
                                                                 int grp, int q, int lane, int m0, int wn) {
  using T = Wave8Tile<GATE_UP>;
  constexpr int NL = T::NL, TN = 4, ROWB = T::ROWB;
  const int sw = T::swz(lane & 31);
  const int a_off = (m0 + (lane & 31)) * ROWB;
  int b_off[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) b_off[j] = (T::b_row(j, wn) + (lane & 31)) * ROWB;
  // fragments of the lo and hi K halves in separate registers
  bf16x8 af[2][2][MI > 0 ? MI : 1], bfr[2][2][TN];
  const int half_off = grp * (T::OPB / 2) + q * 1024;  // this wave's first LDS chunk run in a stage

  // this wave's loads of step kstep: load i fills chunks [(4 i + q) 64, + 64) of its half's rows; the K
  // offset rides in the scalar offset
  auto issue_a = [&](int kstep) {
    char* dst = lds + (kstep % T::A_STAGES) * T::OPB + half_off;
#pragma unroll
    for (int i = 0; i < NL; ++i)
      if (offA[i] != kNoRow)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrcA, (lds_void*)(dst + i * 4096), 16, (int)offA[i], kstep * T::BK * 2,
                                                 0, 0);
  };
  auto issue_b = [&](int kstep) {
    char* dst = lds + T::B_BASE + (kstep % T::B_STAGES) * T::OPB + half_off;
#pragma unroll
    for (int i = 0; i < NL; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrcB, (lds_void*)(dst + i * 4096), 16, (int)offB[i], kstep * T::BK * 2,
                                               0, 0);
  };
  // operand fragments of K slices 2h, 2h + 1 of step kstep (issued only; wait_lgkm0 waits for them)
  auto read_frags = [&](int kstep, int h) {
    const char* sa = lds + (kstep % T::A_STAGES) * T::OPB;
    const char* sb = lds + T::B_BASE + (kstep % T::B_STAGES) * T::OPB;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int coff = ((2 * (2 * h + s) + (lane >> 5)) ^ sw) * 16;
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[h][s][j] = *(const bf16x8*)(sb + b_off[j] + coff);
#pragma unroll
      for (int i = 0; i < MI; ++i) af[h][s][i] = *(const bf16x8*)(sa + a_off + i * 32 * ROWB + coff);
    }
  };
  auto compute = [&](int h) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[h][s][i], bfr[h][s][j], acc[i][j], 0, 0, 0);
  };

  // prologue: this wave's rows of A(0), B(0), B(1); wait for step 0
  issue_a(0);
  issue_b(0);
  if (nk > 1) {
    issue_b(1);
    wait_vmcnt<NL>();  // B loads are never skipped: the newest NL are step 1's
  } else {
    wait_vmcnt<0>();
  }
  bare_barrier();
  for (int kt = 0; kt < nk; ++kt) {
    // step kt is in LDS: A stage kt % 2, B stage kt % 3
    if (kt + 1 < nk) issue_a(kt + 1);  // into the A stage step kt - 1 used (every wave is done with it)
    read_frags(kt, 0);
    wait_lgkm0();
    read_frags(kt, 1);                 // lands while the lo half's MFMAs run
    compute(0);
    if (kt + 2 < nk) issue_b(kt + 2);  // into the B stage step kt - 1 used
    wait_lgkm0();
    compute(1);
    // step kt + 1 has landed (only this wave's B loads of step kt + 2 may still be in flight)
    if (kt + 1 < nk) {
      if (kt + 2 < nk)
        wait_vmcnt<NL>();
      else
        wait_vmcnt<0>();
    }
    bare_barrier();
  }
}

// The K loop of one wave for a tile of at most 64 valid rows. Such a block is a stream of its expert's
// weights, and its speed is set by how many bytes are in flight, so the 160 KiB are laid out for that:
// four stages of the tile's 64 A rows (8 KiB each) and four of B (32 KiB each), with three steps of
// loads in flight where the large-tile ring has two. Every wave issues one A load (its 8 of the 64
// rows; rows past the tile repeat its last row) and NL B loads per step, so a fixed count of loads
// per step orders the ring through vmcnt. Waves 0-3 compute 32 rows each (m0 = 0 or 32, MI <= 1).
template <bool GATE_UP>
struct SmallRing {
  static constexpr int S = 4;                                  // stages of A and of B
  static constexpr int A_STAGE = 64 * Wave8Tile<GATE_UP>::ROWB;  // 8 KiB
  static constexpr int B_BASE = S * A_STAGE;
  static_assert(B_BASE + S * Wave8Tile<GATE_UP>::OPB == Wave8Tile<GATE_UP>::RING, "the small ring fills the LDS");
};

template <bool GATE_UP, int MI>
__device__ __attribute__((always_inline)) inline void wave8_loop_small(char* lds, __amdgpu_buffer_rsrc_t rsrcA,
                                                                       uint32_t offA1, __amdgpu_buffer_rsrc_t rsrcB,
                                                                       const uint32_t (&offB)[4], f32x16 (&acc)[2][4],
                                                                       int nk, int grp, int q, int wave, int lane,
                                                                       int m0, int wn) {
  using T = Wave8Tile<GATE_UP>;
  using R = SmallRing<GATE_UP>;
  constexpr int NL = T::NL, TN = 4, ROWB = T::ROWB, S = R::S;
  constexpr int PER = NL + 1;  // loads per wave and step
  const int sw = T::swz(lane & 31);
  const int a_off = (m0 + (lane & 31)) * ROWB;
  int b_off[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) b_off[j] = (T::b_row(j, wn) + (lane & 31)) * ROWB;
  bf16x8 af[2][2][MI > 0 ? MI : 1], bfr[2][2][TN];
  const int half_off = grp * (T::OPB / 2) + q * 1024;

  // step kstep's loads into stage kstep % S: this wave's 8 A rows (chunks [64 wave, + 64)) and its B
  // chunks as in the large-tile ring
  auto issue = [&](int kstep) {
    char* da = lds + (kstep % S) * R::A_STAGE + wave * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrcA, (lds_void*)da, 16, (int)offA1, kstep * T::BK * 2, 0, 0);
    char* db = lds + R::B_BASE + (kstep % S) * T::OPB + half_off;
#pragma unroll
    for (int i = 0; i < NL; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrcB, (lds_void*)(db + i * 4096), 16, (int)offB[i], kstep * T::BK * 2,
                                               0, 0);
  };
  auto read_frags = [&](int kstep, int h) {
    const char* sa = lds + (kstep % S) * R::A_STAGE;
    const char* sb = lds + R::B_BASE + (kstep % S) * T::OPB;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int coff = ((2 * (2 * h + s) + (lane >> 5)) ^ sw) * 16;
#pragma unroll
      for (int j = 0; j < TN; ++j) bfr[h][s][j] = *(const bf16x8*)(sb + b_off[j] + coff);
#pragma unroll
      for (int i = 0; i < MI; ++i) af[h][s][i] = *(const bf16x8*)(sa + a_off + i * 32 * ROWB + coff);
    }
  };
  auto compute = [&](int h) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[h][s][i], bfr[h][s][j], acc[i][j], 0, 0, 0);
  };

  // prologue: steps 0-2; wait for step 0
  issue(0);
  if (nk > 1) issue(1);
  if (nk > 2) issue(2);
  if (nk > 2)
    wait_vmcnt<2 * PER>();
  else if (nk > 1)
    wait_vmcnt<PER>();
  else
    wait_vmcnt<0>();
  bare_barrier();
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 3 < nk) issue(kt + 3);  // into the stage step kt - 1 used (every wave is done with it)
    read_frags(kt, 0);
    wait_lgkm0();
    read_frags(kt, 1);
    compute(0);
    wait_lgkm0();
    compute(1);
    // step kt + 1 has landed (steps kt + 2 and kt + 3 may still be in flight)
    if (kt + 1 < nk) {
      if (kt + 3 < nk)
        wait_vmcnt<2 * PER>();
      else if (kt + 2 < nk)
        wait_vmcnt<PER>();
      else
        wait_vmcnt<0>();
    }
    bare_barrier();
  }
}

// One logical block of the eight-wave kernel: row tile and column tile from the logical id L, K loop,
// epilogue. Every wave of the block calls it with the same arguments.
template <bool GATE_UP>
__device__ __forceinline__ void w8_block(const GroupedArgs& a, int ncol_max, int64_t n_tiles, int64_t L, char* lds) {
  using T = Wave8Tile<GATE_UP>;
  constexpr int NL = T::NL, OC = T::OC;
  constexpr int OPITCH = OC + 8;  // bf16 per staged output row (16-byte pad)
  constexpr int OUT_BYTES = 8 * 64 * OPITCH * 2;
  constexpr int WROW_OFF = OUT_BYTES;  // row scales (down), after the staged outputs
  static_assert(T::RING <= 160 * 1024 && WROW_OFF + 256 * 4 <= T::RING, "LDS budget");

  constexpr int GR = GATE_UP ? MOE_PF_GROUP_ROWS_GU : MOE_PF_GROUP_ROWS_DN;
  const int64_t sg = L / ((int64_t)GR * ncol_max), within = L % ((int64_t)GR * ncol_max);
  const int64_t gr = min((int64_t)GR, n_tiles - sg * GR);
  const int64_t tile_id = sg * GR + within % gr;
  const int ct = (int)(within / gr);
  const Tile tile = a.tiles[tile_id];
  const ExpertProblem P = pick_problem(a, tile.problem);
  const int col0 = ct * T::COLS;
  if (col0 >= P.ncols) return;

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int grp = wave >> 2, q = wave & 3;
  // gate_up tiles of at most 64 rows run the weight-streaming ring (wave8_loop_small): waves 0-3
  // compute 32 rows each; otherwise each wave computes 64 of the 256 rows. (The down GEMM's short K
  // loop did not gain from it: 1.37 -> 1.41 ms on the skewed GLM-4.5 layer.)
  const bool small = GATE_UP && tile.rows <= 64;
  const int m0 = small && grp == 0 ? (q & 1) * 32 : grp * 128 + (q & 1) * 64, wn = q >> 1;

  // Direct-load sources: chunk p of this half's 128 rows is row 128 g + p / 8, slot p % 8, which holds
  // the row's logical chunk slot ^ swz(row). Both operands are read through raw buffer descriptors
  // with 32-bit byte offsets: B over the expert's matrix (the rows of one half come from one matrix:
  // gate_up's half 0 loads gate rows, half 1 up rows), A over the tile's rows, or over all of x when
  // rows are gathered (the launcher checks that x spans less than 4 GiB). No range clamping: every
  // offset is in bounds.
  const uint16_t* bbase =
      (const uint16_t*)(GATE_UP && grp == 1 ? P.B1 : P.B0) + (int64_t)tile.expert * P.b_stride;
  const uint16_t* abase = (const uint16_t*)P.A + (P.gather ? 0 : (int64_t)tile.row_start * P.lda);
  const __amdgpu_buffer_rsrc_t rsrcB = __builtin_amdgcn_make_buffer_rsrc((void*)bbase, (short)0, -1, kRawBufferWord3);
  const __amdgpu_buffer_rsrc_t rsrcA = __builtin_amdgcn_make_buffer_rsrc((void*)abase, (short)0, -1, kRawBufferWord3);
  uint32_t offA[4], offB[4];
#pragma unroll
  for (int i = 0; i < NL; ++i) {
    const int p = (i * 4 + q) * 64 + lane;
    const int r = grp * 128 + (p >> 3), c = (p & 7) ^ T::swz(r);
    const int col = min(col0 + (GATE_UP ? r % (T::BN / 2) : r), P.ncols - 1);
    offB[i] = ((uint32_t)col * (uint32_t)P.K + 8 * c) * 2;
    if (r < tile.rows) {
      const int64_t g = P.gather ? a.sorted_pair[(int64_t)tile.row_start + r] / a.k : r;
      offA[i] = (uint32_t)(g * P.lda + 8 * c) * 2;
    } else {
      offA[i] = kNoRow;  // past the tile's valid rows: not loaded
    }
  }
  // small ring: this lane's A chunk is row 8 wave + lane / 8 (past the tile: its last row), slot lane % 8
  uint32_t offA1 = 0;
  if (small) {
    const int r = 8 * wave + (lane >> 3), c = (lane & 7) ^ T::swz(r);
    const int rr = min(r, tile.rows - 1);
    const int64_t g = P.gather ? a.sorted_pair[(int64_t)tile.row_start + rr] / a.k : rr;
    offA1 = (uint32_t)(g * P.lda + 8 * c) * 2;
  }
  // down: this thread's row scale, read now so its latency hides under the K loop
  float wscale = 1.0f;
  if (!GATE_UP && t < 256 && P.scale_rows) wscale = a.topk_w[a.sorted_pair[tile.row_start + min(t, tile.rows - 1)]];

  f32x16 acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int nk = P.K / T::BK;
  const int live_m = tile.rows - m0;
  const int mi = live_m <= 0 || (small && grp == 1) ? 0 : min(small ? 1 : 2, (live_m + 31) / 32);
  if (small) {
    if (mi == 1)
      wave8_loop_small<GATE_UP, 1>(lds, rsrcA, offA1, rsrcB, offB, acc, nk, grp, q, wave, lane, m0, wn);
    else
      wave8_loop_small<GATE_UP, 0>(lds, rsrcA, offA1, rsrcB, offB, acc, nk, grp, q, wave, lane, m0, wn);
  } else if (mi == 2) {
    wave8_loop<GATE_UP, 2>(lds, rsrcA, offA, rsrcB, offB, acc, nk, grp, q, lane, m0, wn);
  } else if (mi == 1) {
    wave8_loop<GATE_UP, 1>(lds, rsrcA, offA, rsrcB, offB, acc, nk, grp, q, lane, m0, wn);
  } else {
    wave8_loop<GATE_UP, 0>(lds, rsrcA, offA, rsrcB, offB, acc, nk, grp, q, lane, m0, wn);
  }

  // Epilogue through LDS (the loop ended on a barrier after the last operand read): each wave stages
  // its 64 x OC bf16 results (SwiGLU / weight scale applied) in its own padded region, then stores
  // whole 16-byte row chunks.
  float* wrow = (float*)(lds + WROW_OFF);
  if (!GATE_UP) {
    if (t < 256) wrow[t] = wscale;
    __syncthreads();
  }
  uint16_t* stage_out = (uint16_t*)lds + wave * (64 * OPITCH);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (i >= mi) continue;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);  // within the wave's 64 rows
      if (GATE_UP) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
          stage_out[row * OPITCH + j * 32 + (lane & 31)] = bf16_rne(swiglu_bf16(acc[i][j][r], acc[i][j + 2][r], a.swiglu_limit));
      } else {
        const float sc = wrow[m0 + row];
#pragma unroll
        for (int j = 0; j < 4; ++j) stage_out[row * OPITCH + j * 32 + (lane & 31)] = bf16_rne(acc[i][j][r] * sc);
      }
    }
  }
  __syncthreads();
  uint16_t* out = (uint16_t*)P.out;
  const int ocol0 = col0 + wn * OC;
  constexpr int CH = OC / 8;  // 16-byte chunks per staged row
  const int rows_here = min(32 * mi, tile.rows - m0);  // the rows this wave computed and staged
  for (int c = lane; c < rows_here * CH; c += 64) {
    const int row = c / CH, ch = c % CH;
    const int col = ocol0 + ch * 8;
    if (col < P.ncols) {  // ncols is a multiple of 64: a chunk is wholly in or out
      const uint4 v = *(const uint4*)(stage_out + row * OPITCH + ch * 8);
      *(uint4*)(out + ((int64_t)tile.row_start + m0 + row) * P.ldo + col) = v;
    }
  }
}

// Persistent form: one block per CU. The logical blocks are split into 8 contiguous runs of nearly equal
// length, one per XCD (the run the hardware's round-robin deal of a full grid would give that XCD,
// xcd_logical_block), and a block claims the next logical block of its XCD's run from that run's
// counter; when the run is empty it claims from the other runs in turn, and it exits once all eight
// are empty. Compared with one launched block per logical block this removes the gaps between
// consecutive blocks on a CU (the dispatcher deals workgroups in order, so a busy XCD holds up the
// next workgroup of every other XCD) and lets the XCDs that finish early take the others' last blocks.
template <bool GATE_UP>
__global__ __launch_bounds__(512, 1) void grouped_bf16_w8(GroupedArgs a, int ncol_max) {
  constexpr int RING = Wave8Tile<GATE_UP>::RING;
  __shared__ __attribute__((aligned(1024))) char lds[RING];
  // The claimed index passes through the ring's last word: the K loop is over when it is written (the
  // epilogue's barrier) and the epilogue stages below it; the next K loop starts after every wave read it.
  static_assert(8 * 64 * (Wave8Tile<GATE_UP>::OC + 8) * 2 + 256 * 4 <= RING - 4, "claim word overlaps the epilogue");
  int* claim_word = (int*)(lds + RING - 4);
  const int64_t n_tiles = *a.n_tiles, nvalid = n_tiles * ncol_max;
  const int64_t q = nvalid >> 3, r = nvalid & 7;
  const int x = blockIdx.x & 7;  // the XCD the hardware dealt this block to
  for (int v = 0; v < 8; ++v) {
    const int y = (x + v) & 7;
    const int64_t start = y * q + min((int64_t)y, r), len = q + (y < r ? 1 : 0);
    for (;;) {
      if (threadIdx.x == 0) *claim_word = atomicAdd(&a.work_ctr[y], 1);
      __syncthreads();  // also: the previous logical block's epilogue is done with the LDS
      const int64_t j = *claim_word;
      __syncthreads();  // every wave has read claim before it is overwritten
      if (j >= len) break;
      w8_block<GATE_UP>(a, ncol_max, n_tiles, start + j, lds);
    }
  }
}

#ifndef MOE_PF_EIGHT_WAVES
#define MOE_PF_EIGHT_WAVES 1
#endif

#ifndef MOE_PF_BK
#define MOE_PF_BK 64
#endif
#ifndef MOE_PF_STAGES
#define MOE_PF_STAGES 2
#endif

// The eight-wave kernel addresses its operands with 32-bit byte offsets: from x for gathered rows,
// from a tile's first row otherwise, and from an expert's matrix for B.
bool wave8_fits(const GroupedArgs& a) {
  constexpr int64_t LIM = int64_t(1) << 32;
  for (int p = 0; p < 2; ++p) {
    const ExpertProblem& P = a.prob[p];
    if (!P.out) continue;
    const int64_t a_rows = P.gather ? a.gather_rows : 256;
    if (a_rows <= 0 || a_rows * P.lda * 2 >= LIM) return false;
    if ((int64_t)P.ncols * P.K * 2 >= LIM) return false;
  }
  return true;
}

// Blocks of the persistent kernel: one per CU of the current device (a multiple of 8: every XCD gets
// the same number), queried once per device.
int64_t persistent_grid() {
  static std::atomic<int> cached[64];  // 0 until queried; callers on several threads may race to fill it
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8) n = 256;
    n = n / 8 * 8;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <bool GATE_UP>
hipError_t launch_bm(int bm, const GroupedArgs& a, int64_t max_tile_count, hipStream_t s) {
  constexpr int COLS = GATE_UP ? 128 : 256;
  int nc = 0;
  for (int p = 0; p < 2; ++p)
    if (a.prob[p].out) nc = max(nc, (a.prob[p].ncols + COLS - 1) / COLS);
  int64_t blocks = (max_tile_count * nc + 7) / 8 * 8;
  if (blocks == 0) return hipSuccess;
  if (bm != 256) return hipErrorInvalidValue;  // the forward builds 256-row tile lists for these kernels
  if (MOE_PF_EIGHT_WAVES && wave8_fits(a)) {
    if (!a.work_ctr) return hipErrorInvalidValue;
    const int64_t grid = min(blocks, persistent_grid());
    hipLaunchKernelGGL((grouped_bf16_w8<GATE_UP>), dim3((unsigned)grid), dim3(512), 0, s, a, nc);
  } else
    hipLaunchKernelGGL((grouped_bf16_lds<256, MOE_PF_BK, MOE_PF_STAGES, GATE_UP>), dim3((unsigned)blocks), dim3(256),
                       0, s, a, nc);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bf16_prefill(bool gate_up, int bm, const GroupedArgs& a, int64_t max_tile_count, hipStream_t s) {
  return gate_up ? launch_bm<true>(bm, a, max_tile_count, s) : launch_bm<false>(bm, a, max_tile_count, s);
}

}  // namespace moe
