// Token-choice dispatch ("MoE Forward", two facts #2; the per-expert token lists of the loop form on
// "GLM-5 . Mixture of experts"), as three deterministic kernels:
//   count: per chunk of tokens, an LDS histogram of expert ids;
//   scan : per expert, an exclusive scan over chunks, then an exclusive scan over experts (offsets),
//          and the row-tile lists the grouped GEMMs walk;
//   place: per chunk, each expert's pairs written in token order from that chunk's base.
// The result is the stable order: tokens ascending inside each expert.
#include <hip/hip_runtime.h>

#include "moe_internal.h"

namespace moe {
namespace {

constexpr int CH = kDispatchChunk;
constexpr int MAX_E = 512;

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

__device__ void write_tiles(const TileSpec& ts, int e, int count, int offset, int first_tile) {
  for (int j = 0; j * ts.bm < count; ++j) {
    Tile t;
    t.problem = 0;
    t.expert = e;
    t.row_start = offset + j * ts.bm;
    t.rows = min(ts.bm, count - j * ts.bm);
    ts.tiles[first_tile + j] = t;
  }
}

__global__ __launch_bounds__(512) void scan_kernel(const int32_t* __restrict__ chunk_counts, int nchunks, int64_t N,
                                                   int k, int E, int n_shared_problem, int32_t* __restrict__ counts,
                                                   int32_t* __restrict__ offsets, int32_t* __restrict__ chunk_base,
                                                   TileSpec t0, TileSpec t1) {
  __shared__ int cnt[MAX_E];
  __shared__ int off[MAX_E + 1];
  __shared__ int toff0[MAX_E + 1];
  __shared__ int toff1[MAX_E + 1];
  const int e = threadIdx.x;
  int total = 0;
  if (e < E) {
    for (int c = 0; c < nchunks; ++c) {
      const int v = chunk_counts[(int64_t)c * E + e];
      chunk_base[(int64_t)c * E + e] = total;
      total += v;
    }
    cnt[e] = total;
  }
  __syncthreads();
  if (e == 0) {  // exclusive scans over experts (E <= 512: a short serial loop)
    int run = 0, r0 = 0, r1 = 0;
    for (int i = 0; i < E; ++i) {
      off[i] = run;
      toff0[i] = r0;
      toff1[i] = r1;
      run += cnt[i];
      r0 += (cnt[i] + t0.bm - 1) / t0.bm;
      r1 += (cnt[i] + t1.bm - 1) / t1.bm;
    }
    off[E] = run;
    toff0[E] = r0;
    toff1[E] = r1;
  }
  __syncthreads();
  if (e < E) {
    counts[e] = cnt[e];
    offsets[e] = off[e];
    for (int c = 0; c < nchunks; ++c) chunk_base[(int64_t)c * E + e] += off[e];
    write_tiles(t0, e, cnt[e], off[e], toff0[e]);
    write_tiles(t1, e, cnt[e], off[e], toff1[e]);
  }
  if (e == 0) offsets[E] = off[E];
  // the shared expert's tiles follow the routed ones: all N tokens, in token order
  const TileSpec* specs[2] = {&t0, &t1};
  const int routed_tiles[2] = {toff0[E], toff1[E]};
  for (int sidx = 0; sidx < 2; ++sidx) {
    const TileSpec& ts = *specs[sidx];
    const int64_t nsh = n_shared_problem ? (N + ts.bm - 1) / ts.bm : 0;
    for (int64_t j = threadIdx.x; j < nsh; j += blockDim.x) {
      Tile t;
      t.problem = 1;
      t.expert = 0;
      t.row_start = (int)(j * ts.bm);
      t.rows = (int)min((int64_t)ts.bm, N - j * ts.bm);
      ts.tiles[routed_tiles[sidx] + j] = t;
    }
    if (threadIdx.x == 0) *ts.n_tiles = routed_tiles[sidx] + (int)nsh;
  }
}

__global__ __launch_bounds__(256) void place_kernel(const int32_t* __restrict__ idx, int64_t N, int k, int E,
                                                    const int32_t* __restrict__ chunk_base,
                                                    int32_t* __restrict__ sorted_pair, int32_t* __restrict__ inv_row) {
  extern __shared__ int lidx[];  // CH * k ids of this chunk
  const int c = blockIdx.x;
  const int64_t first = (int64_t)c * CH * k;
  const int npairs = (int)(min((int64_t)(c + 1) * CH, N) * k - first);
  for (int p = threadIdx.x; p < npairs; p += 256) {
    const int e = idx[first + p];
    lidx[p] = e;
    if (e < 0 || e >= E) inv_row[first + p] = -1;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256) {
    int cur = chunk_base[(int64_t)c * E + e];
    for (int p = 0; p < npairs; ++p) {
      if (lidx[p] == e) {
        sorted_pair[cur] = (int32_t)(first + p);
        inv_row[first + p] = cur;
        ++cur;
      }
    }
  }
}

}  // namespace

hipError_t launch_count(const int32_t* idx, int64_t N, int k, int E, int32_t* chunk_counts, hipStream_t s) {
  const int nchunks = (int)((N + CH - 1) / CH);
  hipLaunchKernelGGL(count_kernel, dim3(nchunks), dim3(256), 0, s, idx, N, k, E, chunk_counts);
  return hipGetLastError();
}

hipError_t launch_scan(const int32_t* chunk_counts, int nchunks, int64_t N, int k, int E, int n_shared_problem,
                       int32_t* counts, int32_t* offsets, int32_t* chunk_base, TileSpec t0, TileSpec t1,
                       hipStream_t s) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(512), 0, s, chunk_counts, nchunks, N, k, E, n_shared_problem, counts,
                     offsets, chunk_base, t0, t1);
  return hipGetLastError();
}

hipError_t launch_place(const int32_t* idx, int64_t N, int k, int E, const int32_t* chunk_base, int32_t* sorted_pair,
                        int32_t* inv_row, hipStream_t s) {
  const int nchunks = (int)((N + CH - 1) / CH);
  const size_t lds = (size_t)CH * k * sizeof(int);
  hipLaunchKernelGGL(place_kernel, dim3(nchunks), dim3(256), lds, s, idx, N, k, E, chunk_base, sorted_pair, inv_row);
  return hipGetLastError();
}

}  // namespace moe
