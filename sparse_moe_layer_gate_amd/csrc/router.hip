// Router kernels: the gate GEMM, and the selection / weight kernel.
//
// "Group Router" (GLM-4.5), How it works: s = sigmoid(x W_g^T) with a bias-free float32 gate;
// s' = s + b chooses the experts; groups are scored by their two largest s'; topk_group groups
// survive; the top-k by s' inside them are taken; w = alpha * s / (sum s + eps) from the raw s.
//
// The gate GEMM writes float32 logits split along the hidden dimension (KS partial sums per logit);
// the selection kernel adds the partials in a fixed order, applies the sigmoid and writes the scores.
//  - bf16 activations: the float32 router weight is split exactly into three bf16 pieces,
//    W = hi + mid + lo (each piece the bf16 rounding of what the previous ones left), so every product
//    x * piece is exact in float32 and the bf16 matrix cores accumulate x W in float32 at 3x the bf16
//    work instead of running the 16x slower float32 matrix path; batches of one to four tokens take a
//    one-wave-per-expert kernel that adds the same exact products with fused multiply-adds.
//  - float32 activations: v_mfma_f32_16x16x4_f32 (exact float32 products, float32 accumulation).
#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace moe {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ inline float load_as_f32(const float* p, int64_t i) { return p[i]; }
__device__ inline float load_as_f32(const uint16_t* p, int64_t i) {
  return __uint_as_float((uint32_t)p[i] << 16);  // bf16 -> f32 is exact
}

// ---------------------------------------------------------------------------------------------
// W (float32) -> hi, mid, lo (bf16), stored as three [E, D] matrices. Each residual is exact in
// float32, so hi + mid + lo == W.
__global__ __launch_bounds__(256) void split_kernel(const float* __restrict__ wg, int64_t count,
                                                    uint16_t* __restrict__ w3) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256) {
    const float w = wg[i];
    const uint16_t hi = bf16_rne(w);
    const float r1 = __fsub_rn(w, bf16_f32(hi));
    const uint16_t mid = bf16_rne(r1);
    const float r2 = __fsub_rn(r1, bf16_f32(mid));
    w3[i] = hi;
    w3[count + i] = mid;
    w3[2 * count + i] = bf16_rne(r2);
  }
}

// ---------------------------------------------------------------------------------------------
// bf16 gate GEMM: part[ks, n, e] = sum over the ks-th hidden range of x[n, t] (lo + mid + hi)[e, t].
// A block covers 128 tokens and NJ 32-expert column tiles (all of E up to 256, so x is read once per
// K range), K step 32, an S-stage LDS ring fed by global_load_lds_dwordx4 (the swizzled chunk layout of
// the expert GEMMs); each of the 4 waves owns 32 tokens x all NJ column tiles, v_mfma_f32_32x32x16_bf16
// per piece. The gate GEMM is small and wait-bound, so the ring is as deep as the LDS allows (S - 1
// steps of loads in flight).
constexpr int RB_BM = 128, RB_BK = 32, RB_ROWB = RB_BK * 2, RB_CPR = 4;
constexpr int RB_A_BYTES = RB_BM * RB_ROWB;                // 8 KiB
constexpr int RB_A_LOADS = RB_BM * RB_CPR / 256;            // A loads per thread per K step

template <int NJ>
struct RouterTile {
  static constexpr int BN = 32 * NJ;                             // experts per block
  static constexpr int B_CHUNKS = 3 * BN * RB_CPR;               // 16-byte chunks of the three pieces
  static constexpr int B_LOADS = (B_CHUNKS + 255) / 256;         // B loads per thread per K step
  static constexpr int STAGE = RB_A_BYTES + B_LOADS * 256 * 16;  // the last load's spare chunks land at the end
  static constexpr int S = (160 * 1024) / STAGE < 4 ? (160 * 1024) / STAGE : 4;
  static constexpr int LOADS = RB_A_LOADS + B_LOADS;             // loads per thread per K step
  static_assert(S >= 2, "two stages at least");
  static_assert((S - 2) * LOADS < 64, "vmcnt is 6 bits");
};

__device__ inline int rb_swz(int r) {
  r &= 31;
  return ((r >> 1) ^ (r >> 3)) & 3;
}

// Blocks are numbered (K range, column block)-major, token block minor, and dealt to the XCDs in
// contiguous runs (xcd_logical_block), so an XCD works through few K ranges of the weight pieces and
// they stay in its L2 while its token blocks stream x.
template <int NJ>
__global__ __launch_bounds__(256) void logits_bf16x3_kernel(const uint16_t* __restrict__ x,
                                                            const uint16_t* __restrict__ w3, int64_t N, int D, int E,
                                                            int kchunk, int ks_count, float* __restrict__ part) {
  using T = RouterTile<NJ>;
  constexpr int S = T::S;
  __shared__ __attribute__((aligned(1024))) char lds[S * T::STAGE];
  const int64_t row_blocks = (N + RB_BM - 1) / RB_BM;
  const int col_blocks = (E + T::BN - 1) / T::BN;
  const int64_t L = xcd_logical_block(row_blocks * col_blocks * ks_count);
  if (L < 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n0 = (L % row_blocks) * RB_BM;
  const int64_t slice = L / row_blocks;
  const int e0 = (int)(slice % col_blocks) * T::BN;
  const int ks = (int)(slice / col_blocks);
  const int kbeg = ks * kchunk;
  const int nk = min(kchunk, D - kbeg) / RB_BK;

  // direct-load sources (fixed rows; the K offset advances): load q of this thread fills chunk
  // p = (4 q + wave) 64 + lane of its operand, i.e. row p / 4, slot p % 4 holding the row's logical
  // chunk slot ^ swz(row). Every lane loads: B chunks past the three pieces repeat the last one (into
  // spare space at the end of the stage), experts past E repeat expert E - 1 (never stored).
  const uint16_t* srcA[RB_A_LOADS];
#pragma unroll
  for (int q = 0; q < RB_A_LOADS; ++q) {
    const int p = (q * 4 + wave) * 64 + lane, r = p / RB_CPR, c = (p % RB_CPR) ^ rb_swz(r);
    const int64_t n = min(n0 + r, N - 1);
    srcA[q] = x + n * D + kbeg + 8 * c;
  }
  const uint16_t* srcB[T::B_LOADS];
#pragma unroll
  for (int q = 0; q < T::B_LOADS; ++q) {
    const int p = min((q * 4 + wave) * 64 + lane, T::B_CHUNKS - 1);
    const int piece = p / (T::BN * RB_CPR), rr = (p % (T::BN * RB_CPR)) / RB_CPR;
    const int c = (p % RB_CPR) ^ rb_swz(rr);
    const int e = min(e0 + rr, E - 1);
    srcB[q] = w3 + (int64_t)piece * E * D + (int64_t)e * D + kbeg + 8 * c;
  }
  auto issue = [&](int kstep) {
    char* st = lds + (kstep % S) * T::STAGE;
    const int k0 = kstep * RB_BK;
#pragma unroll
    for (int q = 0; q < RB_A_LOADS; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(srcA[q] + k0), (lds_void*)(st + (q * 4 + wave) * 1024), 16, 0, 0);
#pragma unroll
    for (int q = 0; q < T::B_LOADS; ++q)
      __builtin_amdgcn_global_load_lds((const void*)(srcB[q] + k0),
                                       (lds_void*)(st + RB_A_BYTES + (q * 4 + wave) * 1024), 16, 0, 0);
  };

  f32x16 acc[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  const int sw = rb_swz(lane & 31);
  const int a_off = (wave * 32 + (lane & 31)) * RB_ROWB;

#pragma unroll
  for (int t = 0; t < S - 1; ++t)
    if (t < nk) issue(t);
  for (int kt = 0; kt < nk; ++kt) {
    // step kt's loads are complete (later steps' may be in flight; every thread issues T::LOADS per
    // step); after the barrier everyone's are, and every read of the stage refilled next (step kt - 1)
    // is done
    const int ahead = min(S - 2, nk - 1 - kt);  // steps issued after kt
    if (S > 3 && ahead >= 2) {
      wait_vmcnt<(S > 3 ? 2 : 0) * T::LOADS>();
    } else if (S > 2 && ahead >= 1) {
      wait_vmcnt<(S > 2 ? 1 : 0) * T::LOADS>();
    } else {
      wait_vmcnt<0>();
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (kt + S - 1 < nk) issue(kt + S - 1);
    const char* st = lds + (kt % S) * T::STAGE;
#pragma unroll
    for (int kk = 0; kk < RB_BK / 16; ++kk) {
      const int coff = ((2 * kk + (lane >> 5)) ^ sw) * 16;
      const bf16x8 af = *(const bf16x8*)(st + a_off + coff);
#pragma unroll
      for (int piece = 2; piece >= 0; --piece)  // smallest piece first
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
          const int brow = piece * T::BN + j * 32 + (lane & 31);
          const bf16x8 bf = *(const bf16x8*)(st + RB_A_BYTES + brow * RB_ROWB + coff);
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc[j], 0, 0, 0);
        }
    }
  }
  // 32x32 C layout: lane holds column lane % 32, rows 8 (r / 4) + 4 (lane / 32) + r % 4.
  float* out = part + (int64_t)ks * N * E;
#pragma unroll
  for (int j = 0; j < NJ; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t n = n0 + wave * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      const int e = e0 + j * 32 + (lane & 31);
      if (n < N && e < E) out[n * E + e] = acc[j][r];
    }
}

// Column tiles per block: all of E's 32-expert tiles when there are at most 8, else an even split
// into blocks of at most 8; at most 2 for batches of one or two token blocks (more blocks to spread
// over the CUs, shallower per-block work).
int router_nj(int64_t N, int E) {
  const int most = (N + RB_BM - 1) / RB_BM <= 2 ? 2 : 8;
  const int tiles = (E + 31) / 32, blocks = (tiles + most - 1) / most;
  return (tiles + blocks - 1) / blocks;
}

// ---------------------------------------------------------------------------------------------
// Cross-lane steps on the DPP paths (no LDS round trip). dpp<CTRL>(v): lane i reads v of the lane CTRL
// names; the four patterns used are permutations of each 16-lane row, so every lane has a source.
constexpr int DPP_QUAD_XOR1 = 0xB1;     // quad_perm [1, 0, 3, 2]
constexpr int DPP_QUAD_XOR2 = 0x4E;     // quad_perm [2, 3, 0, 1]
constexpr int DPP_ROW_HALF_MIRROR = 0x141;  // lane i <- lane 7 - i within each 8 lanes
constexpr int DPP_ROW_MIRROR = 0x140;       // lane i <- lane 15 - i within each 16 lanes
template <int CTRL>
__device__ inline int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ inline float dpp_f(float v) {
  return __int_as_float(dpp_i<CTRL>(__float_as_int(v)));
}
__device__ inline float readlane_f(float v, int l) { return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l)); }

// Sum of v over the 64 lanes, the same value in every lane. Each step adds a lane's value to its
// partner's within a 16-lane row (a + b == b + a, so both partners hold the same sum), then the four
// row sums are added as (r0 + r1) + (r2 + r3).
__device__ inline float wave_sum(float v) {
  v += dpp_f<DPP_QUAD_XOR1>(v);
  v += dpp_f<DPP_QUAD_XOR2>(v);
  v += dpp_f<DPP_ROW_HALF_MIRROR>(v);
  v += dpp_f<DPP_ROW_MIRROR>(v);
  return (readlane_f(v, 0) + readlane_f(v, 16)) + (readlane_f(v, 32) + readlane_f(v, 48));
}

// ---------------------------------------------------------------------------------------------
// bf16 gate GEMV for batches of at most RG_MAX_N tokens: part[0, n, e] = x[n] (lo + mid + hi)[e]^T
// over the whole hidden dimension (one partial per logit). A one-wave block per expert: lane l takes
// the 16-byte chunks l, l + 64, ... of the expert's three pieces and of every token's row, adds
// x * lo, x * mid, x * hi per element in float32 (each product exact), and the wave sums its lanes. The
// matrix-core kernel spends a 128-token block on a batch of one token and has too few blocks to spread
// the router weight's stream over the CUs.
constexpr int RG_MAX_N = 4;
template <int NT>
__global__ __launch_bounds__(64) void logits_gemv_kernel(const uint16_t* __restrict__ x,
                                                         const uint16_t* __restrict__ w3, int D, int E,
                                                         float* __restrict__ part) {
  const int e = blockIdx.x, lane = threadIdx.x;
  if (e >= E) return;
  const int64_t ED = (int64_t)E * D;
  const uint16_t* wr = w3 + (int64_t)e * D;
  float acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = 0.f;
  const int nch = D / 8;  // D is a multiple of 64
#pragma unroll 4
  for (int c = lane; c < nch; c += 64) {
    uint4 wv[3], xv[NT];
#pragma unroll
    for (int piece = 0; piece < 3; ++piece) wv[piece] = *(const uint4*)(wr + piece * ED + 8 * c);
#pragma unroll
    for (int n = 0; n < NT; ++n) xv[n] = *(const uint4*)(x + (int64_t)n * D + 8 * c);
#pragma unroll
    for (int h = 0; h < 8; ++h) {
      const int word = h >> 1, sh = (h & 1) * 16;
      const float lo = __uint_as_float(((((const uint32_t*)&wv[2])[word] >> sh) & 0xffffu) << 16);
      const float mid = __uint_as_float(((((const uint32_t*)&wv[1])[word] >> sh) & 0xffffu) << 16);
      const float hi = __uint_as_float(((((const uint32_t*)&wv[0])[word] >> sh) & 0xffffu) << 16);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const float xf = __uint_as_float(((((const uint32_t*)&xv[n])[word] >> sh) & 0xffffu) << 16);
        acc[n] = __fmaf_rn(xf, lo, acc[n]);  // exact product: the fma rounds once, as the add would
        acc[n] = __fmaf_rn(xf, mid, acc[n]);
        acc[n] = __fmaf_rn(xf, hi, acc[n]);
      }
    }
  }
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const float sum = wave_sum(acc[n]);
    if (lane == 0) part[(int64_t)n * E + e] = sum;
  }
}

// ---------------------------------------------------------------------------------------------
// float32 gate GEMM on v_mfma_f32_16x16x4_f32: part[ks, n, e] over the ks-th hidden range.
// Block tile: 64 tokens x 64 experts, K step 32; 4 waves in 2 x 2, each 32 x 32 (2 x 2 MFMA tiles).
// LDS holds both tiles k-major with a row pitch of 80 floats: a wave's MFMA operand read touches
// 4 k-rows x 16 consecutive columns, i.e. 64 distinct banks.
constexpr int LG_BM = 64, LG_BN = 64, LG_BK = 32, LG_PITCH = 80;

template <typename XT>
__global__ __launch_bounds__(256) void logits_f32_kernel(const XT* __restrict__ x, const float* __restrict__ wg,
                                                         int64_t N, int D, int E, int kchunk,
                                                         float* __restrict__ part) {
  __shared__ float As[LG_BK][LG_PITCH];
  __shared__ float Bs[LG_BK][LG_PITCH];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t n0 = (int64_t)blockIdx.x * LG_BM;
  const int e0 = blockIdx.y * LG_BN;
  const int ks = blockIdx.z;
  const int kbeg = ks * kchunk, kend = min(kbeg + kchunk, D);

  const int lr = t >> 2, lk = (t & 3) * 8;
  const int64_t xrow = n0 + lr;
  const int erow = e0 + lr;
  const bool xok = xrow < N, eok = erow < E;

  f32x4 acc[2][2];
  for (int i = 0; i < 2; ++i)
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int k0 = kbeg; k0 < kend; k0 += LG_BK) {
    float av[8], bv[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      av[i] = xok ? load_as_f32(x, xrow * D + k0 + lk + i) : 0.f;
      bv[i] = eok ? wg[(int64_t)erow * D + k0 + lk + i] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      As[lk + i][lr] = av[i];
      Bs[lk + i][lr] = bv[i];
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < LG_BK; kk += 4) {
      const int kr = kk + (lane >> 4);
      float a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) a[i] = As[kr][wm * 32 + i * 16 + (lane & 15)];
#pragma unroll
      for (int j = 0; j < 2; ++j) b[j] = Bs[kr][wn * 32 + j * 16 + (lane & 15)];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  }
  // C layout of the 16x16 tile: lane holds column lane % 16, rows 4 * (lane / 16) + r.
  float* out = part + (int64_t)ks * N * E;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t n = n0 + wm * 32 + i * 16 + 4 * (lane >> 4) + r;
        const int e = e0 + wn * 32 + j * 16 + (lane & 15);
        if (n < N && e < E) out[n * E + e] = acc[i][j][r];
      }
}

// ---------------------------------------------------------------------------------------------
// Selection: one wavefront per token, four tokens per block. Lane l holds experts l, l + 64, ...
// (up to 8). With `part` set, the scores are first formed from the KS logit partials (added in
// order) and written out when `scores` is set; otherwise they are read from `scores`. Every float operation of the selection is one
// correctly rounded IEEE operation in the order the header states, so given the same scores the
// result is bit-identical to a plain float32 evaluation.
constexpr int SEL_MAX_E = 512, SEL_MAX_P = SEL_MAX_E / 64, SEL_MAX_G = 64, SEL_MAX_K = 32;
constexpr int SEL_MAX_KS = 16;  // logit partials per score (router_plan keeps KS within this)

__device__ inline bool beats(float av, int ai, float bv, int bi) { return av > bv || (av == bv && ai < bi); }
// (bv, bi) <- the better of this lane's pair and the pair of the lane CTRL names
template <int CTRL>
__device__ inline void argmax_row_step(float& bv, int& bi) {
  const float ov = dpp_f<CTRL>(bv);
  const int oi = dpp_i<CTRL>(bi);
  if (beats(ov, oi, bv, bi)) {
    bv = ov;
    bi = oi;
  }
}

template <int MAXKS>
__global__ __launch_bounds__(256) void select_kernel(float* __restrict__ scores, const float* __restrict__ part,
                                                     int KS, const float* __restrict__ bias, int64_t N, int E, int G,
                                                     int TG, int k, float alpha, int norm, float eps,
                                                     int32_t* __restrict__ idx_out, float* __restrict__ w_out) {
  __shared__ float s_sel[4][SEL_MAX_E];
  __shared__ float gscore[4][SEL_MAX_G];
  __shared__ int kept[4][SEL_MAX_G];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t n = (int64_t)blockIdx.x * 4 + wave;
  const bool live = n < N;
  const int P = (E + 63) >> 6;
  const int gs = E / G;
  const bool group_stage = G > 1 && TG < G;

  float sp[SEL_MAX_P];
  bool elig[SEL_MAX_P];
  float sraw[SEL_MAX_P] = {};
  // Scores: with partials, the KS partials of SEL_PB experts per lane are all loaded before the first
  // add (one memory round trip per group of SEL_PB experts), then added in order q = 0, 1, ... The loads
  // are unconditional, from clamped in-bounds addresses (MAXKS >= KS slots; extra slots repeat partial
  // KS - 1 and are not added), so no load sits behind a branch whose join would wait for it.
  constexpr int SEL_PB = 4;
#pragma unroll
  for (int p0 = 0; p0 < SEL_MAX_P; p0 += SEL_PB) {
    if (p0 >= P) break;
    if (part) {
      float pv[SEL_PB][MAXKS];
      const int64_t nn = live ? n : N - 1;
#pragma unroll
      for (int pp = 0; pp < SEL_PB; ++pp) {
        const int e = min(lane + 64 * (p0 + pp), E - 1);
#pragma unroll
        for (int q = 0; q < MAXKS; ++q) pv[pp][q] = part[(int64_t)min(q, KS - 1) * N * E + nn * E + e];
      }
#pragma unroll
      for (int pp = 0; pp < SEL_PB; ++pp) {
        float r = pv[pp][0];
#pragma unroll
        for (int q = 1; q < MAXKS; ++q)
          if (q < KS) r = __fadd_rn(r, pv[pp][q]);
        sraw[p0 + pp] = 1.0f / (1.0f + expf(-r));  // s = sigmoid(x W_g^T)
      }
    } else {
#pragma unroll
      for (int pp = 0; pp < SEL_PB; ++pp) {
        const int e = lane + 64 * (p0 + pp);
        sraw[p0 + pp] = p0 + pp < P && e < E && live ? scores[n * E + e] : 0.f;
      }
    }
  }
#pragma unroll
  for (int p = 0; p < SEL_MAX_P; ++p) {
    const int e = lane + 64 * p;
    float sv = 0.f, bv = 0.f;
    if (p < P && e < E && live) {
      sv = sraw[p];
      if (part && scores) scores[n * E + e] = sv;  // the forward does not keep them
      bv = bias[e];
    }
    sp[p] = __fadd_rn(sv, bv);  // s' = s + b
    elig[p] = p < P && e < E;
    if (p < P && e < E) s_sel[wave][e] = sp[p];
  }
  __syncthreads();

  if (group_stage) {
    // group score: sum of the two largest s' of the group (a repeated value counts twice)
    if (lane < G) {
      // running top two (m1 >= m2): v above m1 pushes m1 down, v in (m2, m1] replaces m2
      float m1 = -INFINITY, m2 = -INFINITY;
      const float* gv = &s_sel[wave][lane * gs];
#pragma unroll 8
      for (int j = 0; j < gs; ++j) {
        const float v = gv[j];
        m2 = fmaxf(m2, fminf(m1, v));
        m1 = fmaxf(m1, v);
      }
      gscore[wave][lane] = __fadd_rn(m1, m2);
    }
    __syncthreads();
    if (lane < G) {
      const float mine = gscore[wave][lane];
      int ahead = 0;
      for (int h = 0; h < G; ++h) ahead += beats(gscore[wave][h], h, mine, lane) ? 1 : 0;
      kept[wave][lane] = ahead < TG;
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < SEL_MAX_P; ++p) {
      const int e = lane + 64 * p;
      if (elig[p]) elig[p] = kept[wave][e / gs] != 0;
    }
  }

  // k rounds of a wave-wide arg-max under (s' descending, index ascending). beats() is a strict total
  // order on (value, index) pairs with distinct indices, so the winner does not depend on the order in
  // which the lanes' candidates meet. The winner's raw score is read from the lane that holds it and
  // added to the running sum in slot order; lane j keeps slot j.
  float sum = 0.f, my_s = 0.f;
  int my_e = 0;
  for (int slot = 0; slot < k; ++slot) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int p = 0; p < SEL_MAX_P; ++p) {
      const int e = lane + 64 * p;
      if (elig[p] && beats(sp[p], e, bv, bi)) {
        bv = sp[p];
        bi = e;
      }
    }
    argmax_row_step<DPP_QUAD_XOR1>(bv, bi);
    argmax_row_step<DPP_QUAD_XOR2>(bv, bi);
    argmax_row_step<DPP_ROW_HALF_MIRROR>(bv, bi);
    argmax_row_step<DPP_ROW_MIRROR>(bv, bi);
    // every lane of a 16-lane row holds the row's winner; the four rows meet in uniform registers
    float wv = readlane_f(bv, 0);
    int wi = __builtin_amdgcn_readlane(bi, 0);
#pragma unroll
    for (int r = 16; r < 64; r += 16) {
      const float rv = readlane_f(bv, r);
      const int ri = __builtin_amdgcn_readlane(bi, r);
      if (beats(rv, ri, wv, wi)) {
        wv = rv;
        wi = ri;
      }
    }
    const int ce = min(wi, E - 1);  // stays in range even for NaN scores
    float held = 0.f;
#pragma unroll
    for (int p = 0; p < SEL_MAX_P; ++p)
      if (p == (ce >> 6)) held = sraw[p];
    const float s_win = readlane_f(held, ce & 63);
    sum = __fadd_rn(sum, s_win);
    if (lane == slot) {
      my_e = ce;
      my_s = s_win;
    }
#pragma unroll
    for (int p = 0; p < SEL_MAX_P; ++p)
      if (lane + 64 * p == wi) elig[p] = false;  // k <= eligible count is checked on the host
  }

  if (live && lane < k) {
    float w;
    if (norm) {
      const float den = __fadd_rn(sum, eps);
      w = __fmul_rn(alpha, __fdiv_rn(my_s, den));
    } else {
      w = __fmul_rn(alpha, my_s);
    }
    idx_out[n * k + lane] = my_e;
    w_out[n * k + lane] = w;
  }
}

}  // namespace

#ifndef MOE_ROUTER_BLOCKS
#define MOE_ROUTER_BLOCKS 256  // blocks the bf16 gate GEMM aims for (the K range splits until then)
#endif

int router_rows_per_block(int dtype) { return dtype == MOE_BF16 ? RB_BM : LG_BM; }

RouterPlan router_plan(int dtype, int64_t N, int D, int E) {
  RouterPlan p;
  p.split = dtype == MOE_BF16;
  p.gemv = p.split && N >= 1 && N <= RG_MAX_N;
  if (p.gemv) {
    p.ks = 1;
    p.kchunk = D;
    return p;
  }
  const int64_t bm = p.split ? RB_BM : LG_BM, bn = p.split ? 32 * router_nj(N, E) : LG_BN;
  int64_t tiles = ((N + bm - 1) / bm) * ((E + bn - 1) / bn);
  if (tiles < 1) tiles = 1;  // N = 0
  // aim for 256+ blocks (the bf16 kernel's ring takes most of a CU's LDS), 512+ for the float32 kernel
  const int64_t want = ((p.split ? MOE_ROUTER_BLOCKS : 512) + tiles - 1) / tiles;
  int64_t most = D / 256 > 0 ? D / 256 : 1;        // at least 256 of the hidden dimension per split
  if (most > 16) most = 16;                         // and at most 16 partials to add per logit
  const int64_t ks = want < 1 ? 1 : (want > most ? most : want);
  p.kchunk = (int)((D / ks + 31) / 32 * 32);
  p.ks = (D + p.kchunk - 1) / p.kchunk;
  return p;
}

hipError_t launch_router_split(const float* wg, int E, int D, uint16_t* w3, hipStream_t s) {
  const int64_t count = (int64_t)E * D;
  int64_t blocks = (count + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(split_kernel, dim3((unsigned)blocks), dim3(256), 0, s, wg, count, w3);
  return hipGetLastError();
}

hipError_t launch_logits(int dtype, const RouterPlan& p, const void* x, const float* wg, const uint16_t* w3, int64_t N,
                         int D, int E, float* part, hipStream_t s) {
  if (p.gemv) {
    auto go = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, dim3((unsigned)E), dim3(64), 0, s, (const uint16_t*)x, w3, D, E, part);
    };
    switch (N) {
      case 1: go(logits_gemv_kernel<1>); break;
      case 2: go(logits_gemv_kernel<2>); break;
      case 3: go(logits_gemv_kernel<3>); break;
      default: go(logits_gemv_kernel<4>); break;
    }
    return hipGetLastError();
  }
  if (p.split) {
    const int nj = router_nj(N, E);
    const int64_t blocks = (N + RB_BM - 1) / RB_BM * ((E + 32 * nj - 1) / (32 * nj)) * p.ks;
    dim3 grid((unsigned)((blocks + 7) / 8 * 8));
    auto go = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, grid, dim3(256), 0, s, (const uint16_t*)x, w3, N, D, E, p.kchunk, p.ks, part);
    };
    switch (nj) {
      case 1: go(logits_bf16x3_kernel<1>); break;
      case 2: go(logits_bf16x3_kernel<2>); break;
      case 3: go(logits_bf16x3_kernel<3>); break;
      case 4: go(logits_bf16x3_kernel<4>); break;
      case 5: go(logits_bf16x3_kernel<5>); break;
      case 6: go(logits_bf16x3_kernel<6>); break;
      case 7: go(logits_bf16x3_kernel<7>); break;
      default: go(logits_bf16x3_kernel<8>); break;
    }
  } else {
    dim3 grid((unsigned)((N + LG_BM - 1) / LG_BM), (unsigned)((E + LG_BN - 1) / LG_BN), (unsigned)p.ks);
    if (dtype == MOE_F32)
      hipLaunchKernelGGL(logits_f32_kernel<float>, grid, dim3(256), 0, s, (const float*)x, wg, N, D, E, p.kchunk,
                         part);
    else
      hipLaunchKernelGGL(logits_f32_kernel<uint16_t>, grid, dim3(256), 0, s, (const uint16_t*)x, wg, N, D, E,
                         p.kchunk, part);
  }
  return hipGetLastError();
}

hipError_t launch_select(float* scores, const float* part, int KS, const float* bias, int64_t N, int E, int G, int TG,
                         int k, float alpha, int norm, float eps, int32_t* idx, float* w, hipStream_t s) {
  dim3 grid((unsigned)((N + 3) / 4));
  // partial slots: the smallest power of two >= KS (KS <= SEL_MAX_KS); 1 when the scores are read
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, s, scores, part, KS, bias, N, E, G, TG, k, alpha, norm, eps, idx, w);
  };
  if (!part || KS <= 1)
    go(select_kernel<1>);
  else if (KS <= 2)
    go(select_kernel<2>);
  else if (KS <= 4)
    go(select_kernel<4>);
  else if (KS <= 8)
    go(select_kernel<8>);
  else
    go(select_kernel<SEL_MAX_KS>);
  return hipGetLastError();
}

}  // namespace moe
