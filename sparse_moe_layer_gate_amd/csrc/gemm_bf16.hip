// Grouped bf16 expert GEMMs for token-rich (prefill) batches: 256-row tiles.
//
// Same products as the generic grouped kernels ("MoE Forward", eq. E_i: the gate_up GEMM with the
// SwiGLU applied in registers, and the down GEMM scaled by the mixture weight w_{n,i}), laid out for
// gfx950: grouped_bf16_w8, eight waves, two per SIMD, each wave computing a 64 x 128 share of a
// 256 x 256 tile and issuing an eighth of every step's loads (described where it is defined);
// persistent, one block per CU claiming tiles per XCD.
//  - operands go global -> LDS directly (lane l of a wave writes bytes [16 l, 16 l + 16) of a 1 KiB
//    run), no register staging;
//  - LDS rows are 64 bf16 long, unpadded; the 16-byte chunks of a row are XOR-swizzled by the row's
//    position so that the MFMA operand reads (32 rows at one k offset) hit distinct banks;
//  - v_mfma_f32_32x32x16_bf16 tiles; 32-row MFMA sub-tiles past a tile's valid rows are skipped, so a
//    sparsely filled tile (a rarely chosen expert) costs little MFMA time;
//  - blocks follow an XCD-aware order over the valid tiles, rasterized in rectangles of row tiles x
//    column tiles so that the blocks one XCD runs together share both operands in its L2.
//  - operands are addressed with 32-bit byte offsets from x (gathered rows), from a tile's first row,
//    or from an expert's matrix; the host rejects layers whose x or expert matrices reach 4 GiB.
#include <hip/hip_runtime.h>

#include <atomic>

#include "moe_internal.h"

namespace moe {
namespace {

// Rasterization rectangles (see w8_block): row tiles x column tiles, for gate_up and down. Measured
// (layer ms; 1-D groups of 32 / 16 row tiles down whole columns -> 2 x 16 rectangles, with the small
// experts' tiles after the others, see build_tiles): GLM-5 prefill 6.95 -> 6.77, Air 1.71 -> 1.65,
// skewed GLM-4.5 4.17 -> 4.16; 8 x 4, 4 x 12 and 16 x 2 rectangles were within 1% of 2 x 16 or slower.
#ifndef MOE_PF_GROUP_ROWS_GU
#define MOE_PF_GROUP_ROWS_GU 2
#endif
#ifndef MOE_PF_GROUP_COLS_GU
#define MOE_PF_GROUP_COLS_GU 16
#endif
#ifndef MOE_PF_GROUP_ROWS_DN
#define MOE_PF_GROUP_ROWS_DN 2
#endif
#ifndef MOE_PF_GROUP_COLS_DN
#define MOE_PF_GROUP_COLS_DN 16
#endif
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---- eight-wave kernel for 256-row tiles ----
//
// With one wave per SIMD, the wave that issues a K step's direct loads stalls while the texture path
// accepts them (the CU's waves issue theirs within a short window of the step, so they queue behind
// one another), and its SIMD's matrix core idles meanwhile. Here each SIMD runs two waves (w and w + 4),
// each with its own 64 x 128 share of the tile, its own fragment reads and an eighth of every step's
// loads: while one of them waits on the load path, the other keeps the matrix core busy.
//  - block tile 256 x 256, BK = 64 (whole 128-byte lines per row and load); A in a two-stage ring, B
//    in a three-stage ring, together all 160 KiB of LDS; rows chunk-swizzled (Wave8Tile::swz);
//  - half g = w / 4 owns tile rows [128 g, 128 g + 128); wave w % 4 = 2 wn + mh owns 64 rows (mh) of
//    that half and 128 B rows (wn), as 2 x 4 tiles of v_mfma_f32_32x32x16_bf16 (gate_up: 64 gate rows
//    and the matching 64 up rows, so SwiGLU pairs stay in one wave);
//  - the waves of half g load rows [128 g, 128 g + 128) of both operands, four direct loads per lane
//    of each per step (buffer_load_dwordx4 ... lds through raw buffer descriptors);
//  - per K step t a wave issues its A loads of step t + 1 and works through the step's four 16-wide K
//    slices with the fragments double-buffered by slice: the reads of slice s + 1 are in flight while
//    slice s's MFMAs run. It issues its B loads of step t + 2 with the second slice, waits for its
//    loads of step t + 1, meets the others at a barrier, and then reads step t + 1's first slice while
//    the last slice's MFMAs run. A stage is refilled only after every wave has passed the barrier that
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

template <bool V>
struct BoolC {
  static constexpr bool value = V;
};
template <int V>
struct IntC {
  static constexpr int value = V;
};

// Word 3 of a raw (untyped, stride 0) buffer descriptor on gfx9-family parts: 32-bit data format, no
// swizzle, no index stride.
constexpr int kRawBufferWord3 = 0x00020000;

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
// rows; na: how many of its A loads reach a valid row (the others are not issued; lanes of an issued
// load past the tile repeat its last row). B is never skipped, so a wave's newest NL loads are always
// B loads, which is what the vmcnt(NL) waits rely on.
template <bool GATE_UP, int MI>
__device__ __attribute__((always_inline)) inline void wave8_loop(char* lds, __amdgpu_buffer_rsrc_t rsrcA,
                                                                 const uint32_t (&offA)[4], int na,
                                                                 __amdgpu_buffer_rsrc_t rsrcB, const uint32_t (&offB)[4],
                                                                 f32x16 (&acc)[2][4], int nk, int grp, int q, int lane,
                                                                 int m0, int wn) {
  using T = Wave8Tile<GATE_UP>;
  constexpr int NL = T::NL, TN = 4, ROWB = T::ROWB;
  const int sw = T::swz(lane & 31);
  const int a_off = (m0 + (lane & 31)) * ROWB;
  int b_off[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) b_off[j] = (T::b_row(j, wn) + (lane & 31)) * ROWB;
  const int half_off = grp * (T::OPB / 2) + q * 1024;  // this wave's first LDS chunk run in a stage

  // this wave's loads of step kstep: load i fills chunks [(4 i + q) 64, + 64) of its half's rows; the K
  // offset rides in the scalar offset
  auto issue_a = [&](int kstep) {
    char* dst = lds + (kstep % T::A_STAGES) * T::OPB + half_off;
#pragma unroll
    for (int i = 0; i < NL; ++i)
      if (i < na)  // wave-uniform: loads wholly past the tile's rows are not issued
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
  // Fragments of one 16-wide K slice (kstep's slice sl) into buffer buf; the reads are only issued
  // here, and the waits below order them. A wave with no valid rows reads nothing.
  constexpr int NR = MI > 0 ? MI + TN : 0;  // LDS reads per slice
  bf16x8 af[2][MI > 0 ? MI : 1], bfr[2][TN];
  auto read_slice = [&](int kstep, int sl, int buf) {
    if (MI == 0) return;
    const char* sa = lds + (kstep % T::A_STAGES) * T::OPB;
    const char* sb = lds + T::B_BASE + (kstep % T::B_STAGES) * T::OPB;
    const int coff = ((2 * sl + (lane >> 5)) ^ sw) * 16;
#pragma unroll
    for (int j = 0; j < TN; ++j) bfr[buf][j] = *(const bf16x8*)(sb + b_off[j] + coff);
#pragma unroll
    for (int i = 0; i < MI; ++i) af[buf][i] = *(const bf16x8*)(sa + a_off + i * 32 * ROWB + coff);
  };
  auto compute = [&](int buf) {
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[buf][i], bfr[buf][j], acc[i][j], 0, 0, 0);
  };
  // Scheduling fence: without it the compiler sinks each fragment read next to its first MFMA and
  // waits for it there, so the matrix core idles for an LDS round trip per read.
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
  // s_waitcnt lgkmcnt(NR): all but the newest slice's reads have landed
  auto wait_older_slices = [] { __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (NR << 8)); };

  // prologue: this wave's rows of A(0), B(0), B(1); wait for step 0; read its first slice
  issue_a(0);
  issue_b(0);
  if (nk > 1) {
    issue_b(1);
    wait_vmcnt<NL>();  // B loads are never skipped: the newest NL are step 1's
  } else {
    wait_vmcnt<0>();
  }
  bare_barrier();
  read_slice(0, 0, 0);
  fence();
  // The steps that issue both operands' loads run in a loop of their own, free of the branches and of
  // the variable waits of the last two steps, which are peeled (with the small-tile loop peeled the same
  // way, against one loop with the conditions inside: dense FFN gate_up 1.74 -> 1.65 ms, skewed GLM-4.5
  // layer 4.22 -> 4.08 ms, Air 1.75 -> 1.63 ms; 239 -> 207 VGPRs in gate_up). The slice double buffer
  // against reading whole K halves, which the compiler had interleaved read by read with the MFMAs:
  // gate_up 1-2% faster on every layer (skewed GLM-4.5 2.35 -> 2.34 ms, mild skew 2.23 -> 2.19,
  // GLM-5 3.88 -> 3.83, Air 0.90 -> 0.89).
  auto step = [&](int kt, auto more_a, auto more_b, auto last) {
    constexpr bool MA = decltype(more_a)::value, MB = decltype(more_b)::value, LAST = decltype(last)::value;
    // step kt is in LDS (A stage kt % 2, B stage kt % 3), its slice 0 being read into buffer 0
    if (MA) issue_a(kt + 1);  // into the A stage step kt - 1 used (every wave is done with it)
    read_slice(kt, 1, 1);
    fence();
    wait_older_slices();
    compute(0);
    fence();
    read_slice(kt, 2, 0);
    fence();
    wait_older_slices();
    if (MB) issue_b(kt + 2);  // into the B stage step kt - 1 used
    compute(1);
    fence();
    read_slice(kt, 3, 1);
    fence();
    wait_older_slices();
    compute(0);
    fence();
    wait_lgkm0();
    // step kt + 1 has landed (only this wave's B loads of step kt + 2 may still be in flight)
    if (MB)
      wait_vmcnt<NL>();
    else if (MA)
      wait_vmcnt<0>();
    bare_barrier();
    if (!LAST) read_slice(kt + 1, 0, 0);
    fence();
    compute(1);  // the last slice, while the next step's first reads land
    fence();
  };
  int kt = 0;
  for (; kt + 2 < nk; ++kt) step(kt, BoolC<true>{}, BoolC<true>{}, BoolC<false>{});
  if (kt + 1 < nk) step(kt++, BoolC<true>{}, BoolC<false>{}, BoolC<false>{});
  step(kt, BoolC<false>{}, BoolC<false>{}, BoolC<true>{});
}

// The K loop of one wave for a tile of at most 64 valid rows. Such a block is a stream of its expert's
// weights, and its speed is set by how many bytes are in flight, so the 160 KiB are laid out for that:
// four stages of the tile's 64 A rows (8 KiB each) and four of B (32 KiB each), with three steps of
// loads in flight where the large-tile ring has two. Every wave issues one A load (its 8 of the 64
// rows; rows past the tile repeat its last row) and NL B loads per step, so a fixed count of loads
// per step orders the ring through vmcnt. Waves 0-3 compute 32 rows each (m0 = 0 or 32, MI <= 1).
// Cache policy of the small-tile ring's weight loads: non-temporal (the NT bit, 2 on gfx950). Almost
// every small tile is its expert's only tile (the rest are the last tiles of larger experts), so these
// weight bytes are read once per launch, and the hint keeps that stream from evicting the hot experts'
// weight panels, which several row tiles share in L2:
// skewed GLM-4.5 gate_up 2.35 -> 2.29 ms (124 experts of at most 64 rows, 3.9 GB of their weights),
// the other layers within 1%. (On every B load it costs 1-12%: there the panels are reused.)
constexpr int kStreamPolicy = 2;

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
                                               0, kStreamPolicy);
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
  // AHEAD: steps issued after step kt + 1 when step kt ends (2 in the main loop, then 1, 0); the last
  // step waits for nothing. As in the large-tile loop, the main steps run in a loop of their own.
  auto step = [&](int kt, auto ahead_tag) {
    constexpr int AHEAD = decltype(ahead_tag)::value;
    if (AHEAD == 2) issue(kt + 3);  // into the stage step kt - 1 used (every wave is done with it)
    read_frags(kt, 0);
    wait_lgkm0();
    read_frags(kt, 1);
    compute(0);
    wait_lgkm0();
    compute(1);
    // step kt + 1 has landed (steps kt + 2 and kt + 3 may still be in flight)
    if (AHEAD == 2)
      wait_vmcnt<2 * PER>();
    else if (AHEAD == 1)
      wait_vmcnt<PER>();
    else if (AHEAD == 0)
      wait_vmcnt<0>();
    bare_barrier();
  };
  int kt = 0;
  for (; kt + 3 < nk; ++kt) step(kt, IntC<2>{});
  if (kt + 2 < nk) step(kt++, IntC<1>{});
  if (kt + 1 < nk) step(kt++, IntC<0>{});
  step(kt, IntC<-1>{});
}

// One logical block of the eight-wave kernel: row tile and column tile from the logical id L, K loop,
// epilogue. Every wave of the block calls it with the same arguments.
// Logical block L of a region of n_region row tiles -> (row tile within the region, column tile): walk
// rectangles of GR row tiles x GC column tiles (the last ones of a row group or of the region smaller),
// row tiles fastest.
template <int GR, int GC>
__device__ inline void raster(int64_t L, int ncol_max, int64_t n_region, int64_t& tile_rel, int& ct) {
  const int64_t sg = L / ((int64_t)GR * ncol_max), within = L % ((int64_t)GR * ncol_max);
  const int64_t gr = min((int64_t)GR, n_region - sg * GR);
  const int64_t cg = within / (gr * GC), w2 = within % (gr * GC);
  tile_rel = sg * GR + w2 % gr;
  ct = (int)(cg * GC + w2 / gr);
}

template <bool GATE_UP>
__device__ __forceinline__ void w8_block(const GroupedArgs& a, int ncol_max, int64_t n_tiles, int64_t n_hot, int64_t L,
                                         char* lds) {
  using T = Wave8Tile<GATE_UP>;
  constexpr int NL = T::NL, OC = T::OC;
  constexpr int OPITCH = OC + 8;  // bf16 per staged output row (16-byte pad)
  constexpr int OUT_BYTES = 8 * 64 * OPITCH * 2;
  constexpr int WROW_OFF = OUT_BYTES;  // row scales (down), after the staged outputs
  static_assert(T::RING <= 160 * 1024 && WROW_OFF + 256 * 4 <= T::RING, "LDS budget");

  // Rasterization: logical ids walk rectangles of GR row tiles x GC column tiles (for gate_up,
  // MOE_HOT_ALIGN rows in the hot region at the list's start), row tiles fastest. The blocks an XCD runs at one time are
  // consecutive logical ids, so they cover about one rectangle and read GR A slices and GC B slices
  // per K step between them instead of one of each per block.
  constexpr int GR = GATE_UP ? MOE_PF_GROUP_ROWS_GU : MOE_PF_GROUP_ROWS_DN;
  constexpr int GC = GATE_UP ? MOE_PF_GROUP_COLS_GU : MOE_PF_GROUP_COLS_DN;
  int64_t tile_id;
  int ct;
#ifndef MOE_HOT_DOWN
#define MOE_HOT_DOWN 0  // 1: the down GEMM walks the hot region in MOE_HOT_ALIGN-row rectangles too
#endif
  if ((GATE_UP || MOE_HOT_DOWN) && L < n_hot * ncol_max) {
    raster<MOE_HOT_ALIGN, GC>(L, ncol_max, n_hot, tile_id, ct);
  } else if (GATE_UP || MOE_HOT_DOWN) {
    raster<GR, GC>(L - n_hot * ncol_max, ncol_max, n_tiles - n_hot, tile_id, ct);
    tile_id += n_hot;
  } else {
    raster<GR, GC>(L, ncol_max, n_tiles, tile_id, ct);  // the hot region is a multiple of GR rows
  }
  const Tile tile = a.tiles[tile_id];
  if (tile.rows <= 0) return;  // padding
  const ExpertProblem P = pick_problem(a, tile.problem);
  const int col0 = ct * T::COLS;
  if (col0 >= P.ncols) return;

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int grp = wave >> 2, q = wave & 3;
  // Tiles of at most 64 rows run the weight-streaming ring (wave8_loop_small): waves 0-3 compute 32
  // rows each; otherwise each wave computes 64 of the 256 rows. (The down GEMM, 24 K steps, gains only
  // with the ring's non-temporal weight loads: skewed GLM-4.5 down 1.36 -> 1.33 ms, 1.37 -> 1.41 ms
  // without the hint; the other layers within 0.5%.)
  const bool small = tile.rows <= 64;
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
    const int rr = min(r, tile.rows - 1);  // rows past the tile repeat its last row (never stored)
    const int64_t g = P.gather ? a.sorted_pair[(int64_t)tile.row_start + rr] / a.k : rr;
    offA[i] = (uint32_t)(g * P.lda + 8 * c) * 2;
  }
  // A loads of this wave that reach a valid row: load i covers rows 128 g + 32 i + 8 q + [0, 8)
  const int na = max(0, min(NL, (tile.rows - grp * 128 - 8 * q + 31) / 32));
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
    wave8_loop<GATE_UP, 2>(lds, rsrcA, offA, na, rsrcB, offB, acc, nk, grp, q, lane, m0, wn);
  } else if (mi == 1) {
    wave8_loop<GATE_UP, 1>(lds, rsrcA, offA, na, rsrcB, offB, acc, nk, grp, q, lane, m0, wn);
  } else {
    wave8_loop<GATE_UP, 0>(lds, rsrcA, offA, na, rsrcB, offB, acc, nk, grp, q, lane, m0, wn);
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
  const int64_t n_hot = a.n_hot ? min((int64_t)*a.n_hot, n_tiles) : 0;
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
      w8_block<GATE_UP>(a, ncol_max, n_tiles, n_hot, start + j, lds);
    }
  }
}

}  // namespace

// The eight-wave kernel addresses its operands with 32-bit byte offsets: from x for gathered rows,
// from a tile's first row otherwise (256 rows), and from an expert's matrix for B.
bool bf16_prefill_fits(const GroupedArgs& a) {
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

namespace {

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
  // the host rejects layers beyond the 32-bit offsets before anything is launched
  if (!bf16_prefill_fits(a) || !a.work_ctr) return hipErrorInvalidValue;
  const int64_t grid = min(blocks, persistent_grid());
  hipLaunchKernelGGL((grouped_bf16_w8<GATE_UP>), dim3((unsigned)grid), dim3(512), 0, s, a, nc);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bf16_prefill(bool gate_up, int bm, const GroupedArgs& a, int64_t max_tile_count, hipStream_t s) {
  return gate_up ? launch_bm<true>(bm, a, max_tile_count, s) : launch_bm<false>(bm, a, max_tile_count, s);
}

}  // namespace moe
