// Internal declarations shared by the library's translation units (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// Stages of the forward, in launch order; each has its own timing slot.
enum Stage {
  ST_ROUTER_SPLIT = 0,  // float32 router weight -> three bfloat16 pieces
  ST_LOGITS,            // gate GEMM + sigmoid -> scores
  ST_SELECT,            // bias, group stage, top-k, weights
  ST_COUNT,             // per-chunk expert histogram (batches of one chunk: the whole dispatch)
  ST_SCAN,              // offsets, chunk bases, tile lists
  ST_PLACE,             // stable placement -> sorted_pair / inv_row
  ST_GATE_UP,           // grouped gate_up GEMM + SwiGLU (routed and shared)
  ST_DOWN,              // grouped down GEMM + weight scale (routed and shared)
  ST_COMBINE,           // y = sum of weighted rows + shared row
  ST_COUNT_STAGES
};

// One row tile of a grouped GEMM: problem 0 = routed experts, 1 = shared expert.
struct Tile {
  int32_t problem;
  int32_t expert;
  int32_t row_start;  // first row in the problem's row space
  int32_t rows;       // valid rows in this tile (1..BM; 0 for the padding of the 256-row lists)
};

// ---- device helpers shared by the kernels ----
typedef __attribute__((address_space(3))) void lds_void;

// float -> bfloat16 bits, round to nearest even (finite inputs).
__device__ inline uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ inline float bf16_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// SwiGLU of one intermediate column: SiLU(gate) * up, clamped first when lim > 0 (gate from above only,
// up on both sides: "Module 02 -- MoE: Capacity, Work, and Traffic", section 3).
__device__ inline float swiglu(float g, float u, float lim) {
  if (lim > 0.f) {
    g = fminf(g, lim);
    u = fminf(fmaxf(u, -lim), lim);
  }
  return g / (1.0f + expf(-g)) * u;
}
// The same for results rounded to bfloat16: the hardware exponential and reciprocal (a few float32 ulp,
// far below the bfloat16 rounding that follows) instead of the full-precision library sequence.
__device__ inline float swiglu_bf16(float g, float u, float lim) {
  if (lim > 0.f) {
    g = fminf(g, lim);
    u = fminf(fmaxf(u, -lim), lim);
  }
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

// s_waitcnt with vmcnt = N and the other counters left at their maximum (gfx9 encoding).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Profiling hooks (no-ops unless moe_profile_begin() was called).
void prof_before(int stage, hipStream_t s);
void prof_after(int stage, hipStream_t s);

constexpr int kDispatchChunk = 256;  // tokens per dispatch block
// 256-row tile lists: each large expert's tiles take a multiple of this many list slots (padded with
// empty tiles), so that they start a row group of the prefill kernels' 2-row rasterization rectangles
// and an expert's two tiles share its weights in L2 instead of straddling two rectangles. Measured
// against no padding (layer ms): GLM-5 prefill 6.73 -> 6.51, Air 1.63 -> 1.58, the 288-expert prefill
// 4.82 -> 4.59, mild-skew GLM-4.5 3.99 -> 3.89, skewed GLM-4.5 4.14 -> 4.09; padding to 4 with 4-row
// rectangles was 1-2% slower than this except on the skewed GLM-4.5 layer.
#ifndef MOE_TILE_ALIGN
#define MOE_TILE_ALIGN 2
#endif
// Experts with at least MOE_HOT_TILES tiles ("hot") go first in the 256-row lists, padded to a multiple
// of MOE_HOT_ALIGN slots, and the prefill gate_up kernel walks that region in MOE_HOT_ALIGN-row
// rectangles, so that four row tiles of a hot expert share each of its weight panels in L2 (0: no hot
// region). Same box, layer ms (mean of two runs): skewed GLM-4.5 4.01 -> 3.96, mild-skew GLM-4.5
// 3.84 -> 3.80, GLM-5, Air and the 288-expert prefill unchanged; the same rectangles in the down GEMM
// as well were no better, and a threshold of 5 tiles was between the two.
#ifndef MOE_HOT_TILES
#define MOE_HOT_TILES 3
#endif
#ifndef MOE_HOT_ALIGN
#define MOE_HOT_ALIGN 4
#endif

// ---- router ----
struct RouterPlan {
  bool split;  // bf16 activations: the router weight runs as three bf16 pieces on the bf16 matrix cores
  bool gemv;   // split, and few enough tokens for the one-wave-per-expert kernel (ks = 1)
  int ks;      // partial sums per logit (split of the hidden dimension)
  int kchunk;  // hidden elements per split (a multiple of 32)
};
RouterPlan router_plan(int dtype, int64_t N, int D, int E);
int router_rows_per_block(int dtype);  // token rows of one logits block (the plan changes at multiples)
hipError_t launch_router_split(const float* wg, int E, int D, uint16_t* w3, hipStream_t s);
hipError_t launch_logits(int dtype, const RouterPlan& p, const void* x, const float* wg, const uint16_t* w3, int64_t N,
                         int D, int E, float* part, hipStream_t s);
// part == nullptr: scores are an input; otherwise scores are formed from the KS partials and written
// (unless scores == nullptr).
hipError_t launch_select(float* scores, const float* part, int KS, const float* bias, int64_t N, int E, int G, int TG,
                         int k, float alpha, int norm, float eps, int32_t* idx, float* w, hipStream_t s);

// ---- dispatch ----
struct TileSpec {
  int bm;            // rows per tile
  Tile* tiles;       // output list (nullptr: no list is built)
  int32_t* n_tiles;  // output count
  int small_max;     // > 0: tiles of experts with 1..small_max rows go after all the others, and
                     // the other experts' tiles are padded to MOE_TILE_ALIGN slots
  int32_t* work_ctr;  // the list's 8 work counters (persistent kernels), zeroed with the list; or nullptr
  int32_t* n_hot;     // output: slots of the hot region at the list's start (or nullptr)
};
hipError_t launch_count(const int32_t* idx, int64_t N, int k, int E, int32_t* chunk_counts, hipStream_t s);
hipError_t launch_scan(const int32_t* chunk_counts, int nchunks, int64_t N, int k, int E, int n_shared_problem,
                       int32_t* counts, int32_t* offsets, int32_t* chunk_base, TileSpec t0, TileSpec t1,
                       int pick_rows, hipStream_t s);
// Tile lists of a single dense problem over N rows (the dense FFN).
hipError_t launch_dense_tiles(int64_t N, TileSpec t0, TileSpec t1, hipStream_t s);
hipError_t launch_place(const int32_t* idx, int64_t N, int k, int E, const int32_t* chunk_base, int32_t* sorted_pair,
                        int32_t* inv_row, hipStream_t s);
// count + scan + place in one block for N <= kDispatchChunk (same results as the three kernels)
hipError_t launch_dispatch_small(const int32_t* idx, int64_t N, int k, int E, int n_shared_problem, int32_t* counts,
                                 int32_t* offsets, int32_t* sorted_pair, int32_t* inv_row, TileSpec t0, TileSpec t1,
                                 int pick_rows, hipStream_t s);

// ---- grouped expert GEMMs ----
struct ExpertProblem {
  const void* A;       // activation rows
  int64_t lda;         // elements between rows of A
  int gather;          // 1: A row = sorted_pair[row] / k (rows of x in expert order); 0: A row = row
  const void* B0;      // gate rows (gate_up) or down rows, expert 0
  const void* B1;      // up rows (gate_up), expert 0
  int64_t b_stride;    // elements between consecutive experts' B
  int K;               // reduction length
  int ncols;           // output columns
  void* out;           // [rows, ncols]
  int64_t ldo;
  int scale_rows;      // 1: multiply row r by topk_w[sorted_pair[r]]
};
struct GroupedArgs {
  ExpertProblem prob[2];
  int bm;  // rows per tile of the tile list this launch walks
  const Tile* tiles;
  const int32_t* n_tiles;
  const int32_t* sorted_pair;
  const float* topk_w;
  int k;
  float swiglu_limit;      // gate_up epilogue clamp bound (0: plain SwiGLU)
  int64_t gather_rows;     // rows of the matrix that gathered A rows index (x); 0 when unknown
  int32_t* work_ctr;       // 8 counters, zero at launch: per-XCD work claims of the persistent kernels
  const int32_t* n_hot;    // slots of the list's hot region (MOE_HOT_TILES), or nullptr: none
};
// Field-wise select keeps a problem descriptor in scalar registers (a dynamically indexed
// kernel-argument array would be copied to scratch).
__device__ inline ExpertProblem pick_problem(const GroupedArgs& a, int p) {
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

// Block id -> logical work id over the nvalid blocks that have work (the grid is sized for the
// largest possible tile count; the rest return at once). The hardware deals workgroups to the 8 XCDs
// round-robin (block b to XCD b % 8); this bijection on [0, nvalid) gives each XCD a contiguous run of
// logical ids of nearly equal length, so the column tiles of one row tile (which share the A rows) and
// neighbouring row tiles of one expert (which share B) meet in one L2, and all XCDs share the work.
// Returns -1 for blocks past nvalid.
__device__ inline int64_t xcd_logical_block(int64_t nvalid) {
  const int64_t b = blockIdx.x;
  if (b >= nvalid) return -1;
  const int64_t x = b & 7, j = b >> 3, q = nvalid >> 3, r = nvalid & 7;
  return x * q + (x < r ? x : r) + j;
}

// Upper bound on tiles for a tile list with bm rows per tile.
int64_t max_tiles(int64_t N, int k, int E, int n_shared_problem, int bm);
int gemm_bm(int dtype, int64_t N, int k, int E);  // rows per tile the forward will use
int small_expert_rows(int dtype, int bm);         // TileSpec::small_max for a list of bm-row tiles
int device_pick_rows(int dtype, int64_t N, int k, int E);  // > 0: both tile lists, the scan picks
int tile_plan_rows(int i);  // i = 0, 1: rows per expert (pairs / E) where the tile lists change form
hipError_t launch_gate_up(int dtype, const GroupedArgs& a, int64_t max_tile_count, hipStream_t s);
hipError_t launch_down(int dtype, const GroupedArgs& a, int64_t max_tile_count, hipStream_t s);
hipError_t launch_bf16_prefill(bool gate_up, int bm, const GroupedArgs& a, int64_t max_tile_count, hipStream_t s);
hipError_t launch_bf16_decode(bool gate_up, const GroupedArgs& a, int64_t max_tile_count, hipStream_t s);

// ---- combine ----
// y = alpha_out * (routed rows in slot order) + shared row
hipError_t launch_combine(int dtype, const void* Y, const void* Ysh, const int32_t* inv_row, int64_t N, int k, int D,
                          float alpha_out, void* y, hipStream_t s);
// p[0 .. n) = v and q[0 .. m) = v in one launch (a kernel rather than memset nodes, so the call may sit
// in a captured graph)
hipError_t launch_fill2_i32(int32_t* p, int64_t n, int32_t* q, int64_t m, int32_t v, hipStream_t s);

}  // namespace moe
