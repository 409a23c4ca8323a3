// Token-choice dispatch ("MoE Forward", two facts #2; the per-expert token lists of the loop form on
// "GLM-5 . Mixture of experts"), as three deterministic kernels:
//   count: per chunk of tokens, an LDS histogram of expert ids;
//   scan : per expert, an exclusive scan over chunks, then an exclusive scan over experts (offsets),
//          and the row-tile lists the grouped GEMMs walk;
//   place: per chunk, each pair written at its expert's chunk base + its stable rank in the chunk.
// The result is the stable order: tokens ascending inside each expert.
#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int CH = kDispatchChunk;
constexpr int MAX_E = 512;
constexpr int PL = 512, PW = PL / 64;  // threads (pairs per round) and waves of a placement block

__global__ __launch_bounds__(256) void count_kernel(const int32_t* __restrict__ idx, int64_t N, int k, int E,
                                                    int32_t* __restrict__ chunk_counts) {
  __shared__ int hist[MAX_E];
  const int c = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += 256) hist[e] = 0;
  __syncthreads();
  const int64_t first = (int64_t)c * CH * k;
  const int64_t last = min((int64_t)(c + 1) * CH, N) * k;
  for (int64_t p = first + threadIdx.x; p < last; p += 256) {
    const int e = idx[p];
    if (e >= 0 && e < E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) chunk_counts[(int64_t)c * E + e] = hist[e];
}

// Exclusive scan of one int per thread over a 512-thread block (8 waves): shuffles inside each wave,
// then the wave totals. Returns the exclusive prefix; *total receives the block sum.
__device__ int block_exclusive_scan(int v, int* wsum, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
  for (int w = 0; w < 8; ++w) {
    const int t = wsum[w];
    before += w < wave ? t : 0;
    all += t;
  }
  __syncthreads();  // wsum is reused by the next scan
  *total = all;
  return before + incl - v;
}

// Row-tile list of one grouped GEMM (called by every thread of the scan block; thread e < E holds
// expert e's count and row offset). Order: the tiles of the routed experts in expert order, then the
// shared expert's; with ts.small_max > 0 the single tiles of experts with 1..small_max rows (which
// mostly stream their expert's weights) go after all of them. The persistent GEMM kernels balance the
// XCDs by claiming work, and their rasterization rectangles then hold the full tiles of the large
// experts, whose blocks run alike and share operands in L2, apart from the weight-streaming ones.
__device__ void build_tiles(const TileSpec& ts, bool valid, int e, int cnt, int off, int64_t N,
                            int n_shared_problem, int* wsum) {
  const int nt = valid ? (cnt + ts.bm - 1) / ts.bm : 0;
  const bool small = valid && cnt >= 1 && cnt <= ts.small_max && cnt <= ts.bm;
  // list slots of a large expert: its tiles, padded with empty ones (rows 0) to a multiple of
  // MOE_TILE_ALIGN in the 256-row lists, so that an expert's tiles start a rasterization row group;
  // hot experts (MOE_HOT_TILES tiles or more) come first, padded to MOE_HOT_ALIGN
  const bool lists256 = ts.small_max > 0;
  const bool hot = lists256 && MOE_HOT_TILES > 0 && !small && nt >= MOE_HOT_TILES;
  const int align = hot ? MOE_HOT_ALIGN : (lists256 && MOE_TILE_ALIGN > 1) ? MOE_TILE_ALIGN : 1;
  const int slots = small ? 0 : (nt + align - 1) / align * align;
  int na, nhot, nrest;
  const int ia = block_exclusive_scan(small ? 1 : 0, wsum, &na);
  const int ih = block_exclusive_scan(hot ? slots : 0, wsum, &nhot);
  const int ir = block_exclusive_scan(hot ? 0 : slots, wsum, &nrest);
  const int nrouted = nhot + nrest;
  const int nsh = n_shared_problem ? (int)((N + ts.bm - 1) / ts.bm) : 0;
  const int nb = nrouted + nsh;
  if (small) {
    ts.tiles[nb + ia] = Tile{0, e, off, cnt};
  } else {
    const int ib = hot ? ih : nhot + ir;
    for (int j = 0; j < nt; ++j) ts.tiles[ib + j] = Tile{0, e, off + j * ts.bm, min(ts.bm, cnt - j * ts.bm)};
    for (int j = nt; j < slots; ++j) ts.tiles[ib + j] = Tile{0, e, off, 0};
  }
  for (int j = threadIdx.x; j < nsh; j += blockDim.x)
    ts.tiles[nrouted + j] = Tile{1, 0, j * ts.bm, (int)min((int64_t)ts.bm, N - (int64_t)j * ts.bm)};
  if (threadIdx.x == 0) {
    *ts.n_tiles = na + nb;
    if (ts.n_hot) *ts.n_hot = nhot;
  }
  if (ts.work_ctr && threadIdx.x < 8) ts.work_ctr[threadIdx.x] = 0;
}

__global__ __launch_bounds__(512) void scan_kernel(const int32_t* __restrict__ chunk_counts, int nchunks, int64_t N,
                                                   int k, int E, int n_shared_problem, int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ offsets, int32_t* __restrict__ chunk_base,
                                                   TileSpec t0, TileSpec t1, int pick_rows) {
  __shared__ int wsum[8];
  __shared__ int max_cnt;
  if (threadIdx.x == 0) max_cnt = 0;
  __syncthreads();
  const int e = threadIdx.x;
  // per expert: its total over the chunks, then (once the expert offsets are known) the chunk bases;
  // eight independent loads in flight per round in both passes (a serial chain of loads, or a
  // read-modify-write pass over chunk_base, costs ~1 us per chunk)
  int cnt = 0;
  if (e < E) {
    for (int c0 = 0; c0 < nchunks; c0 += 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) cnt += c0 + u < nchunks ? chunk_counts[(int64_t)(c0 + u) * E + e] : 0;
    }
  }
  if (pick_rows > 0 && cnt > 0) atomicMax(&max_cnt, cnt);  // read after the scan's barriers
  int total;
  const int off = block_exclusive_scan(cnt, wsum, &total);
  if (e < E) {
    counts[e] = cnt;
    offsets[e] = off;
    int run = off;
    for (int c0 = 0; c0 < nchunks; c0 += 8) {
      int v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = c0 + u < nchunks ? chunk_counts[(int64_t)(c0 + u) * E + e] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (c0 + u < nchunks) chunk_base[(int64_t)(c0 + u) * E + e] = run;
        run += v[u];
      }
    }
  }
  if (e == 0) offsets[E] = total;
  // the shared expert's tiles cover all N tokens, in token order
  // (no lists when dispatch runs on its own: the tile pointers are null for every thread alike)
  if (t0.tiles) build_tiles(t0, e < E, e, cnt, off, N, n_shared_problem, wsum);
  if (t1.tiles) build_tiles(t1, e < E, e, cnt, off, N, n_shared_problem, wsum);
  // both lists built (t0 of 16-row tiles, t1 of 256-row tiles): empty the one whose kernels do not run
  // (thread 0 wrote both counts above)
  if (pick_rows > 0 && threadIdx.x == 0) *(max_cnt <= pick_rows ? t1.n_tiles : t0.n_tiles) = 0;
}

// Stable placement of one chunk: rounds of PL pairs (in pair order); inside a round, a pair's
// position is its expert's running offset + the pairs of that expert in earlier waves of the round +
// those in earlier lanes of its own wave (found with one ballot per bit of the expert id). Tokens stay
// ascending inside each expert because pairs are visited in (token, slot) order.

__global__ __launch_bounds__(PL) void place_kernel(const int32_t* __restrict__ idx, int64_t N, int k, int E,
                                                    const int32_t* __restrict__ chunk_base,
                                                    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ inv_row) {
  __shared__ int running[MAX_E];
  __shared__ int wcnt[PW][MAX_E];
  const int c = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t first = (int64_t)c * CH * k;
  const int npairs = (int)(min((int64_t)(c + 1) * CH, N) * k - first);
  const int ebits = E > 1 ? 32 - __clz(E - 1) : 0;  // bits of the largest expert id
  for (int e = t; e < E; e += PL) {
    running[e] = chunk_base[(int64_t)c * E + e];
    for (int w = 0; w < PW; ++w) wcnt[w][e] = 0;
  }
  __syncthreads();
  for (int r0 = 0; r0 < npairs; r0 += PL) {
    const int p = r0 + t;
    int e = -1;
    if (p < npairs) {
      e = idx[first + p];
      if (e < 0 || e >= E) {
        e = -1;
        inv_row[first + p] = -1;
      }
    }
    // lanes of this wave holding the same expert: one ballot per bit of the expert id
    uint64_t same = __ballot(e >= 0);
    for (int b = 0; b < ebits; ++b) {
      const bool bit = (e >> b) & 1;
      const uint64_t m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    const int rank = __popcll(same & ((1ull << lane) - 1));  // same-expert lanes before this one
    if (e >= 0 && rank == 0) wcnt[wave][e] = __popcll(same);
    __syncthreads();
    if (e >= 0) {
      int pos = running[e] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][e];
      sorted_pair[pos] = (int32_t)(first + p);
      inv_row[first + p] = pos;
    }
    __syncthreads();
    for (int e2 = t; e2 < E; e2 += PL) {
      int add = 0;
      for (int w = 0; w < PW; ++w) {
        add += wcnt[w][e2];
        wcnt[w][e2] = 0;
      }
      running[e2] += add;
    }
    __syncthreads();
  }
}

// The whole dispatch of a batch of at most one chunk (N <= kDispatchChunk tokens) in one block: the
// histogram, the scan and tile lists of scan_kernel, then the stable placement of place_kernel with the
// expert offsets as the chunk's bases. Same results, bit for bit, as the three kernels; one launch
// instead of three, which is most of the dispatch time of a decode step.
__global__ __launch_bounds__(PL) void dispatch_small_kernel(const int32_t* __restrict__ idx, int64_t N, int k, int E,
                                                            int n_shared_problem, int32_t* __restrict__ counts,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ sorted_pair,
                                                            int32_t* __restrict__ inv_row, TileSpec t0, TileSpec t1,
                                                            int pick_rows) {
  __shared__ int running[MAX_E];  // the histogram, then each expert's next free position
  __shared__ int wcnt[PW][MAX_E];
  __shared__ int wsum[8];
  __shared__ int max_cnt;
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int npairs = (int)(N * k);
  for (int e = t; e < E; e += PL) {
    running[e] = 0;
    for (int w = 0; w < PW; ++w) wcnt[w][e] = 0;
  }
  if (t == 0) max_cnt = 0;
  __syncthreads();
  for (int p = t; p < npairs; p += PL) {
    const int e = idx[p];
    if (e >= 0 && e < E) atomicAdd(&running[e], 1);
  }
  __syncthreads();
  const int e = t;  // E <= 512 = PL: one expert per thread
  const int cnt = e < E ? running[e] : 0;
  if (pick_rows > 0 && cnt > 0) atomicMax(&max_cnt, cnt);  // read after the scan's barriers
  int total;
  const int off = block_exclusive_scan(cnt, wsum, &total);
  if (e < E) {
    counts[e] = cnt;
    offsets[e] = off;
    running[e] = off;  // only thread e reads or writes entry e here; the barriers below publish it
  }
  if (e == 0) offsets[E] = total;
  if (t0.tiles) build_tiles(t0, e < E, e, cnt, off, N, n_shared_problem, wsum);
  if (t1.tiles) build_tiles(t1, e < E, e, cnt, off, N, n_shared_problem, wsum);
  if (pick_rows > 0 && t == 0) *(max_cnt <= pick_rows ? t1.n_tiles : t0.n_tiles) = 0;
  __syncthreads();
  const int ebits = E > 1 ? 32 - __clz(E - 1) : 0;
  for (int r0 = 0; r0 < npairs; r0 += PL) {
    const int p = r0 + t;
    int pe = -1;
    if (p < npairs) {
      pe = idx[p];
      if (pe < 0 || pe >= E) {
        pe = -1;
        inv_row[p] = -1;
      }
    }
    uint64_t same = __ballot(pe >= 0);
    for (int b = 0; b < ebits; ++b) {
      const bool bit = (pe >> b) & 1;
      const uint64_t m = __ballot(bit);
      same &= bit ? m : ~m;
    }
    const int rank = __popcll(same & ((1ull << lane) - 1));
    if (pe >= 0 && rank == 0) wcnt[wave][pe] = __popcll(same);
    __syncthreads();
    if (pe >= 0) {
      int pos = running[pe] + rank;
      for (int w = 0; w < wave; ++w) pos += wcnt[w][pe];
      sorted_pair[pos] = p;
      inv_row[p] = pos;
    }
    __syncthreads();
    for (int e2 = t; e2 < E; e2 += PL) {
      int add = 0;
      for (int w = 0; w < PW; ++w) {
        add += wcnt[w][e2];
        wcnt[w][e2] = 0;
      }
      running[e2] += add;
    }
    __syncthreads();
  }
}

// Tile lists of one dense problem (problem 0, expert 0) over N rows, for the dense FFN.
__global__ __launch_bounds__(256) void dense_tiles_kernel(int64_t N, TileSpec t0, TileSpec t1) {
  for (int which = 0; which < 2; ++which) {
    const TileSpec& ts = which ? t1 : t0;
    const int64_t nt = (N + ts.bm - 1) / ts.bm;
    for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < nt; j += (int64_t)gridDim.x * 256) {
      Tile t;
      t.problem = 0;
      t.expert = 0;
      t.row_start = (int)(j * ts.bm);
      t.rows = (int)min((int64_t)ts.bm, N - j * ts.bm);
      ts.tiles[j] = t;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      *ts.n_tiles = (int)nt;
      if (ts.n_hot) *ts.n_hot = 0;
    }
    if (blockIdx.x == 0 && threadIdx.x < 8 && ts.work_ctr) ts.work_ctr[threadIdx.x] = 0;
  }
}

__global__ __launch_bounds__(256) void fill2_i32_kernel(int32_t* __restrict__ p, int64_t n, int32_t* __restrict__ q,
                                                       int64_t m, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n + m; i += (int64_t)gridDim.x * 256) {
    if (i < n)
      p[i] = v;
    else
      q[i - n] = v;
  }
}

}  // namespace

hipError_t launch_fill2_i32(int32_t* p, int64_t n, int32_t* q, int64_t m, int32_t v, hipStream_t s) {
  if (n + m <= 0) return hipSuccess;
  const int64_t blocks = min((n + m + 255) / 256, (int64_t)1024);
  hipLaunchKernelGGL(fill2_i32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n, q, m, v);
  return hipGetLastError();
}

hipError_t launch_dense_tiles(int64_t N, TileSpec t0, TileSpec t1, hipStream_t s) {
  const int64_t nt = (N + min(t0.bm, t1.bm) - 1) / min(t0.bm, t1.bm);
  const int64_t blocks = max((int64_t)1, min((nt + 255) / 256, (int64_t)256));
  hipLaunchKernelGGL(dense_tiles_kernel, dim3((unsigned)blocks), dim3(256), 0, s, N, t0, t1);
  return hipGetLastError();
}

hipError_t launch_count(const int32_t* idx, int64_t N, int k, int E, int32_t* chunk_counts, hipStream_t s) {
  const int nchunks = (int)((N + CH - 1) / CH);
  hipLaunchKernelGGL(count_kernel, dim3(nchunks), dim3(256), 0, s, idx, N, k, E, chunk_counts);
  return hipGetLastError();
}

hipError_t launch_scan(const int32_t* chunk_counts, int nchunks, int64_t N, int k, int E, int n_shared_problem,
                       int32_t* counts, int32_t* offsets, int32_t* chunk_base, TileSpec t0, TileSpec t1,
                       int pick_rows, hipStream_t s) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(512), 0, s, chunk_counts, nchunks, N, k, E, n_shared_problem, counts,
                     offsets, chunk_base, t0, t1, pick_rows);
  return hipGetLastError();
}

hipError_t launch_dispatch_small(const int32_t* idx, int64_t N, int k, int E, int n_shared_problem, int32_t* counts,
                                 int32_t* offsets, int32_t* sorted_pair, int32_t* inv_row, TileSpec t0, TileSpec t1,
                                 int pick_rows, hipStream_t s) {
  if (N > CH) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dispatch_small_kernel, dim3(1), dim3(PL), 0, s, idx, N, k, E, n_shared_problem, counts, offsets,
                     sorted_pair, inv_row, t0, t1, pick_rows);
  return hipGetLastError();
}

hipError_t launch_place(const int32_t* idx, int64_t N, int k, int E, const int32_t* chunk_base, int32_t* sorted_pair,
                        int32_t* inv_row, hipStream_t s) {
  const int nchunks = (int)((N + CH - 1) / CH);
  hipLaunchKernelGGL(place_kernel, dim3(nchunks), dim3(PL), 0, s, idx, N, k, E, chunk_base, sorted_pair, inv_row);
  return hipGetLastError();
}

}  // namespace moe
