// C ABI entry points (declared and documented in include/moe.h): argument checks on the host, the
// workspace carve-up, and the launch sequence of the forward on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <vector>

#include "moe_internal.h"

using namespace moe;

namespace {

constexpr int kMaxE = 512, kMaxG = 64, kMaxK = 32;

moe_status check_cfg(const moe_config* c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  const int D = c->hidden_size, E = c->n_routed_experts, G = c->n_group, TG = c->topk_group;
  const int k = c->num_experts_per_tok, d = c->moe_intermediate_size;
  if (D < 1 || E < 1 || d < 1 || k < 1 || c->n_shared_experts < 0) return MOE_ERR_INVALID_ARG;
  if (G < 1 || E % G != 0 || TG < 1 || TG > G) return MOE_ERR_INVALID_ARG;
  if (G > 1 && E / G < 2) return MOE_ERR_INVALID_ARG;  // a group's score needs two members
  if ((int64_t)k > (int64_t)TG * (E / G)) return MOE_ERR_INVALID_ARG;
  if (c->norm_topk_prob != 0 && c->norm_topk_prob != 1) return MOE_ERR_INVALID_ARG;
  if (c->dtype != MOE_F32 && c->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(c->routed_scaling_factor) || !std::isfinite(c->eps) || c->eps < 0.f) return MOE_ERR_INVALID_ARG;
  if (c->alpha_on_output != 0 && c->alpha_on_output != 1) return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(c->swiglu_limit) || c->swiglu_limit < 0.f) return MOE_ERR_INVALID_ARG;
  if (E > kMaxE || G > kMaxG || k > kMaxK) return MOE_ERR_UNSUPPORTED;
  if (D % 64 != 0 || d % 64 != 0) return MOE_ERR_UNSUPPORTED;
  if ((int64_t)d * c->n_shared_experts > (1 << 24)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status check_n(const moe_config* c, int64_t N) {
  if (N < 0) return MOE_ERR_INVALID_ARG;
  // row positions (N k routed + N shared) and token ids are int32
  if (N * (int64_t)(c->num_experts_per_tok + 1) >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The bf16 prefill GEMM addresses gathered rows of x and each expert matrix with 32-bit byte offsets
// (gemm_bf16.hip): x of N rows and every [rows, K] weight slab must stay under 4 GiB.
bool bf16_offsets_fit(int64_t N, int64_t D, int64_t d, int64_t dsh) {
  constexpr int64_t LIM = int64_t(1) << 32;
  return N * D * 2 < LIM && d * D * 2 < LIM && dsh * D * 2 < LIM;
}

size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

struct Workspace {
  size_t idx, w, chunk_counts, chunk_base, counts, offsets, sorted_pair, inv_row, tiles0, tiles1, ntiles;
  size_t w3, part, route_total;  // router: split weight, logit partials; bytes moe_route needs
  size_t H, Hsh, Y, Ysh, total;
  RouterPlan rp;
  int64_t max_tiles0, max_tiles1;
  int bm0, bm1;
  int pick;  // > 0: tiles0 holds 16-row and tiles1 256-row tiles, and the scan kernel picks one of them
};

Workspace layout(const moe_config* c, int64_t N) {
  Workspace w{};
  const int64_t E = c->n_routed_experts, k = c->num_experts_per_tok, D = c->hidden_size;
  const int64_t d = c->moe_intermediate_size, dsh = d * c->n_shared_experts;
  const int64_t es = c->dtype == MOE_F32 ? 4 : 2;
  const int64_t nchunks = (N + kDispatchChunk - 1) / kDispatchChunk;
  const int shp = c->n_shared_experts > 0;
  w.pick = device_pick_rows(c->dtype, N, (int)k, (int)E);
  w.bm0 = w.pick ? 16 : gemm_bm(c->dtype, N, (int)k, (int)E);
  w.bm1 = w.pick ? 256 : w.bm0;
  w.max_tiles0 = max_tiles(N, (int)k, (int)E, shp, w.bm0);
  w.max_tiles1 = max_tiles(N, (int)k, (int)E, shp, w.bm1);
  w.rp = router_plan(c->dtype, N, (int)D, (int)E);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  // router scratch first: moe_route needs only this prefix
  w.w3 = take(w.rp.split ? sizeof(uint16_t) * 3 * E * D : 0);
  w.part = take(sizeof(float) * w.rp.ks * N * E);
  w.route_total = o;
  w.idx = take(sizeof(int32_t) * N * k);
  w.w = take(sizeof(float) * N * k);
  w.chunk_counts = take(sizeof(int32_t) * nchunks * E);
  w.chunk_base = take(sizeof(int32_t) * nchunks * E);
  w.counts = take(sizeof(int32_t) * E);
  w.offsets = take(sizeof(int32_t) * (E + 1));
  w.sorted_pair = take(sizeof(int32_t) * N * k);
  w.inv_row = take(sizeof(int32_t) * N * k);
  w.tiles0 = take(sizeof(Tile) * w.max_tiles0);
  w.tiles1 = take(sizeof(Tile) * w.max_tiles1);
  w.ntiles = take(sizeof(int32_t) * 20);  // two tile counts, 8 work counters per list, two hot counts
  w.H = take(es * N * k * d);
  w.Hsh = take(es * N * dsh);
  w.Y = take(es * N * k * D);
  w.Ysh = take(es * N * D);
  w.total = o;
  return w;
}

// Workspace of moe_dispatch on its own: the per-chunk counts and bases (none for a one-chunk batch,
// which runs as a single kernel).
struct DispatchWorkspace {
  size_t chunk_counts, chunk_base, total;
};

DispatchWorkspace dispatch_layout(const moe_config* c, int64_t N) {
  DispatchWorkspace w{};
  const int64_t E = c->n_routed_experts;
  const int64_t nchunks = N <= kDispatchChunk ? 0 : (N + kDispatchChunk - 1) / kDispatchChunk;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  w.chunk_counts = take(sizeof(int32_t) * nchunks * E);
  w.chunk_base = take(sizeof(int32_t) * nchunks * E);
  w.total = o;
  return w;
}

// Dense FFN workspace: tile lists and the intermediate H [N, dff].
struct DenseWorkspace {
  size_t tiles0, tiles1, ntiles, H, total;
  int bm;
  int64_t max_tiles;
};

DenseWorkspace dense_layout(int64_t N, int dff, int dtype) {
  DenseWorkspace w{};
  const int64_t es = dtype == MOE_F32 ? 4 : 2;
  w.bm = gemm_bm(dtype, N, 1, 1);
  w.max_tiles = (N + w.bm - 1) / w.bm;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  w.tiles0 = take(sizeof(Tile) * w.max_tiles);
  w.tiles1 = take(sizeof(Tile) * w.max_tiles);
  w.ntiles = take(sizeof(int32_t) * 20);  // two tile counts, 8 work counters per list, two hot counts
  w.H = take(es * N * dff);
  w.total = o;
  return w;
}

moe_status check_dense(int64_t N, int32_t D, int32_t dff, int32_t dtype, float limit) {
  if (N < 0 || D < 1 || dff < 1) return MOE_ERR_INVALID_ARG;
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (!std::isfinite(limit) || limit < 0.f) return MOE_ERR_INVALID_ARG;
  if (D % 64 != 0 || dff % 64 != 0 || dff > (1 << 24)) return MOE_ERR_UNSUPPORTED;
  if (N >= (int64_t)1 << 31) return MOE_ERR_UNSUPPORTED;
  if (dtype == MOE_BF16 && !bf16_offsets_fit(256, D, dff, dff)) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

template <typename T>
T* at(void* ws, size_t off) {
  return (T*)((char*)ws + off);
}

// ---- per-stage timing ----
// The recording state is per calling thread: moe_profile_begin / _end bracket the calls one thread
// makes, and calls from other threads are not recorded. The event pool of a thread is reused across
// recordings and lives until the process ends.
struct ProfRec {
  int stage;
  hipEvent_t a, b;
};
thread_local bool g_prof_on = false;
thread_local uint32_t g_prof_mask = 0;  // bit i: record stage i
thread_local bool g_prof_err = false;
thread_local std::vector<ProfRec> g_recs;
thread_local std::vector<hipEvent_t> g_pool;
thread_local size_t g_pool_next = 0;

hipEvent_t next_event() {
  if (g_pool_next == g_pool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) {
      g_prof_err = true;
      return nullptr;
    }
    g_pool.push_back(e);
  }
  return g_pool[g_pool_next++];
}

const char* kStageNames[ST_COUNT_STAGES] = {"router_split", "router_logits", "router_select",  "dispatch_count",
                                            "dispatch_scan", "dispatch_place", "experts_gate_up", "experts_down",
                                            "combine"};

#define MOE_TRY(stage, expr)                 \
  do {                                       \
    prof_before((stage), s);                 \
    const hipError_t e_ = (expr);            \
    prof_after((stage), s);                  \
    if (e_ != hipSuccess) return MOE_ERR_HIP; \
  } while (0)

// Router. wg is the float32 router weight, or (prepared) the three bf16 pieces of moe_router_prepare;
// scores is read (MOE_ROUTE_SCORES_IN), written (non-null otherwise) or not kept (null).
moe_status route_impl(const moe_config* c, int64_t N, const void* x, const void* wg, bool prepared,
                      const float* bias, float* scores, bool scores_in, int32_t* idx, float* w, void* ws,
                      const Workspace& L, hipStream_t s) {
  const int E = c->n_routed_experts, D = c->hidden_size;
  float* part = nullptr;
  if (!scores_in) {
    const uint16_t* w3 = (const uint16_t*)wg;
    part = at<float>(ws, L.part);
    if (L.rp.split && !prepared) {
      uint16_t* split = at<uint16_t>(ws, L.w3);
      MOE_TRY(ST_ROUTER_SPLIT, launch_router_split((const float*)wg, E, D, split, s));
      w3 = split;
    }
    MOE_TRY(ST_LOGITS, launch_logits(c->dtype, L.rp, x, (const float*)wg, w3, N, D, E, part, s));
  }
  // alpha on the routed output instead: the weights carry a factor 1, which the product leaves exact
  const float alpha_w = c->alpha_on_output ? 1.0f : c->routed_scaling_factor;
  MOE_TRY(ST_SELECT, launch_select(scores, part, L.rp.ks, bias, N, E, c->n_group, c->topk_group,
                                   c->num_experts_per_tok, alpha_w, c->norm_topk_prob, c->eps, idx, w, s));
  return MOE_OK;
}

// Dispatch: one kernel for a one-chunk batch, else count / scan / place over per-chunk scratch. t0, t1:
// the tile lists to build (tiles == nullptr: none, for moe_dispatch on its own).
moe_status dispatch_impl(const moe_config* c, int64_t N, const int32_t* idx, int32_t* counts, int32_t* offsets,
                         int32_t* sorted_pair, int32_t* inv_row, int32_t* chunk_counts, int32_t* chunk_base,
                         const TileSpec& t0, const TileSpec& t1, int pick, hipStream_t s) {
  const int E = c->n_routed_experts, k = c->num_experts_per_tok;
  const int shared = c->n_shared_experts > 0;
  if (N <= kDispatchChunk) {
    MOE_TRY(ST_COUNT, launch_dispatch_small(idx, N, k, E, shared, counts, offsets, sorted_pair, inv_row, t0, t1,
                                            pick, s));
    return MOE_OK;
  }
  const int nchunks = (int)((N + kDispatchChunk - 1) / kDispatchChunk);
  MOE_TRY(ST_COUNT, launch_count(idx, N, k, E, chunk_counts, s));
  MOE_TRY(ST_SCAN, launch_scan(chunk_counts, nchunks, N, k, E, shared, counts, offsets, chunk_base, t0, t1, pick, s));
  MOE_TRY(ST_PLACE, launch_place(idx, N, k, E, chunk_base, sorted_pair, inv_row, s));
  return MOE_OK;
}

// The forward's dispatch: both tile lists in the workspace.
moe_status forward_dispatch(const moe_config* c, int64_t N, const int32_t* idx, void* ws, const Workspace& L,
                            hipStream_t s) {
  int32_t* ntiles = at<int32_t>(ws, L.ntiles);
  const TileSpec t0{L.bm0, at<Tile>(ws, L.tiles0), ntiles, small_expert_rows(c->dtype, L.bm0), ntiles + 2,
                    ntiles + 18};
  const TileSpec t1{L.bm1, at<Tile>(ws, L.tiles1), ntiles + 1, small_expert_rows(c->dtype, L.bm1), ntiles + 10,
                    ntiles + 19};
  return dispatch_impl(c, N, idx, at<int32_t>(ws, L.counts), at<int32_t>(ws, L.offsets),
                       at<int32_t>(ws, L.sorted_pair), at<int32_t>(ws, L.inv_row), at<int32_t>(ws, L.chunk_counts),
                       at<int32_t>(ws, L.chunk_base), t0, t1, L.pick, s);
}

// One grouped GEMM over the workspace's tile list `list` (0 or 1), with the 8 work counters at `ctr` in
// the count block.
hipError_t grouped_gemm(bool gate_up, int dtype, GroupedArgs g, void* ws, const Workspace& L, int list, int ctr,
                        hipStream_t s) {
  int32_t* block = at<int32_t>(ws, L.ntiles);  // the two tile counts, then the work counters
  g.tiles = at<Tile>(ws, list ? L.tiles1 : L.tiles0);
  g.n_tiles = block + list;
  g.work_ctr = block + ctr;
  g.n_hot = block + 18 + list;
  g.bm = list ? L.bm1 : L.bm0;
  const int64_t max_tile_count = list ? L.max_tiles1 : L.max_tiles0;
  return gate_up ? launch_gate_up(dtype, g, max_tile_count, s) : launch_down(dtype, g, max_tile_count, s);
}

// gate_up runs over list 0 (counters 2..9), down over list 1 (counters 10..17). When the device picks the
// kernel (L.pick), both GEMMs launch the decode kernel over list 0 and the prefill kernel over list 1, and
// the scan kernel has emptied one of the two lists, whose launch then does nothing.
hipError_t gemm_stage(bool gate_up, int dtype, const GroupedArgs& g, void* ws, const Workspace& L, hipStream_t s) {
  const int ctr = gate_up ? 2 : 10;
  if (!L.pick) return grouped_gemm(gate_up, dtype, g, ws, L, gate_up ? 0 : 1, ctr, s);
  const hipError_t e = grouped_gemm(gate_up, dtype, g, ws, L, 0, ctr, s);
  return e != hipSuccess ? e : grouped_gemm(gate_up, dtype, g, ws, L, 1, ctr, s);
}

// Routed experts, shared expert and combine for routing (idx, w) already dispatched into the workspace.
moe_status experts_impl(const moe_config* cfg, int64_t N, const void* x, const moe_weights* wt, const float* w,
                        void* y, void* ws, const Workspace& L, hipStream_t s) {
  const int k = cfg->num_experts_per_tok, D = cfg->hidden_size;
  const int d = cfg->moe_intermediate_size, dsh = d * cfg->n_shared_experts;
  const int64_t es = cfg->dtype == MOE_F32 ? 4 : 2;
  const bool shared = cfg->n_shared_experts > 0;
  GroupedArgs g{};
  g.sorted_pair = at<int32_t>(ws, L.sorted_pair);
  g.topk_w = w;
  g.k = k;
  g.swiglu_limit = cfg->swiglu_limit;
  g.gather_rows = N;
  // gate_up + SwiGLU: routed rows gather x through sorted_pair; the shared expert reads x in order
  g.prob[0] = ExpertProblem{x, D, 1, wt->gate_up, (const char*)wt->gate_up + es * (int64_t)d * D, 2LL * d * D, D, d,
                            at<void>(ws, L.H), d, 0};
  if (shared)
    g.prob[1] = ExpertProblem{x, D, 0, wt->sh_gate, wt->sh_up, 0, D, dsh, at<void>(ws, L.Hsh), dsh, 0};
  MOE_TRY(ST_GATE_UP, gemm_stage(true, cfg->dtype, g, ws, L, s));
  // down + mixture weight (routed) / weight 1 (shared)
  g.prob[0] = ExpertProblem{at<void>(ws, L.H), d, 0, wt->down, nullptr, (int64_t)D * d, d, D, at<void>(ws, L.Y), D, 1};
  if (shared)
    g.prob[1] = ExpertProblem{at<void>(ws, L.Hsh), dsh, 0, wt->sh_down, nullptr, 0, dsh, D, at<void>(ws, L.Ysh), D, 0};
  MOE_TRY(ST_DOWN, gemm_stage(false, cfg->dtype, g, ws, L, s));
  const float alpha_out = cfg->alpha_on_output ? cfg->routed_scaling_factor : 1.0f;
  MOE_TRY(ST_COMBINE, launch_combine(cfg->dtype, at<void>(ws, L.Y), shared ? at<void>(ws, L.Ysh) : nullptr,
                                     at<int32_t>(ws, L.inv_row), N, k, D, alpha_out, y, s));
  return MOE_OK;
}

// Host checks shared by the forward entry points: x, y and the expert weights.
moe_status check_expert_args(const moe_config* cfg, int64_t N, const void* x, const moe_weights* wt, const void* y) {
  const bool shared = cfg->n_shared_experts > 0;
  if (cfg->dtype == MOE_BF16 &&
      !bf16_offsets_fit(N, cfg->hidden_size, cfg->moe_intermediate_size,
                        (int64_t)cfg->moe_intermediate_size * cfg->n_shared_experts))
    return MOE_ERR_UNSUPPORTED;
  if (!x || !y || !wt->gate_up || !wt->down) return MOE_ERR_INVALID_ARG;
  if (shared && (!wt->sh_gate || !wt->sh_up || !wt->sh_down)) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(y) || !aligned16(wt->gate_up) || !aligned16(wt->down)) return MOE_ERR_INVALID_ARG;
  if (shared && (!aligned16(wt->sh_gate) || !aligned16(wt->sh_up) || !aligned16(wt->sh_down)))
    return MOE_ERR_INVALID_ARG;
  if (x == y) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// ---- scratch for moe_forward_noalloc ----
// A fixed device array that stands in for the caller's workspace. In host code `scratch` names a host
// stand-in, not device memory: its device address is taken once per device with hipGetSymbolAddress
// (scratch_on_current_device) and only that address is used.
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, or nullptr if the device or the symbol lookup fails.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

namespace moe {

void prof_before(int stage, hipStream_t s) {
  if (!g_prof_on || !((g_prof_mask >> stage) & 1u)) return;
  ProfRec r{stage, next_event(), next_event()};
  if (!r.a || !r.b || hipEventRecord(r.a, s) != hipSuccess) {
    g_prof_err = true;
    return;
  }
  g_recs.push_back(r);
}

void prof_after(int stage, hipStream_t s) {
  if (!g_prof_on || g_recs.empty() || g_recs.back().stage != stage) return;
  if (hipEventRecord(g_recs.back().b, s) != hipSuccess) g_prof_err = true;
}

}  // namespace moe

extern "C" {

moe_status moe_check_config(const moe_config* cfg) { return check_cfg(cfg); }

size_t moe_workspace_size(const moe_config* cfg, int64_t N) {
  if (check_cfg(cfg) != MOE_OK || check_n(cfg, N) != MOE_OK) return 0;
  // layout(n).total is not monotone in n: the router's K split and the GEMM tile height change with n,
  // and where they do the buffers they size can shrink by more than a token's worth. The size reported
  // is the most any batch of at most N tokens needs, so a workspace sized for the largest batch serves
  // every smaller one. Between the points where the plan changes form the size grows with n, so the
  // candidates are N and the last n before each change: the multiples of the router's row block (its
  // tile count, and with it the K split, changes there; from 512 row blocks on the split is 1) and the
  // last n under each tile-height threshold.
  size_t most = layout(cfg, N).total;
  auto consider = [&](int64_t n) {
    if (n >= 1 && n < N) most = std::max(most, layout(cfg, n).total);
  };
  const int64_t rb = router_rows_per_block(cfg->dtype);
  for (int64_t m = 1; m <= 513 && m * rb < N; ++m) consider(m * rb);
  const int64_t E = cfg->n_routed_experts, k = cfg->num_experts_per_tok;
  for (int i = 0; i < 2; ++i) consider((tile_plan_rows(i) * E + k - 1) / k - 1);
  return most;
}

size_t moe_router_prepared_size(const moe_config* cfg) {
  if (check_cfg(cfg) != MOE_OK || cfg->dtype != MOE_BF16) return 0;
  return sizeof(uint16_t) * 3 * (size_t)cfg->n_routed_experts * (size_t)cfg->hidden_size;
}

moe_status moe_router_prepare(const moe_config* cfg, const float* w_router, void* prepared, size_t bytes,
                              void* stream) {
  moe_status st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if (cfg->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;  // float32 layers use w_router as given
  if (!w_router || !prepared || !aligned16(w_router) || !aligned16(prepared)) return MOE_ERR_INVALID_ARG;
  if (bytes < moe_router_prepared_size(cfg)) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  MOE_TRY(ST_ROUTER_SPLIT,
          launch_router_split(w_router, cfg->n_routed_experts, cfg->hidden_size, (uint16_t*)prepared, s));
  return MOE_OK;
}

moe_status moe_route(const moe_config* cfg, int64_t N, const void* x, const void* w_router, const float* e_bias,
                     float* scores, uint32_t flags, int32_t* topk_idx, float* topk_w, void* workspace, size_t ws_bytes,
                     void* stream) {
  moe_status st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_n(cfg, N)) != MOE_OK) return st;
  if (flags & ~(MOE_ROUTE_SCORES_IN | MOE_ROUTE_SCORES_OUT | MOE_ROUTE_PREPARED)) return MOE_ERR_INVALID_ARG;
  const bool scores_in = flags & MOE_ROUTE_SCORES_IN, prepared = flags & MOE_ROUTE_PREPARED;
  if (scores_in && (flags & (MOE_ROUTE_SCORES_OUT | MOE_ROUTE_PREPARED))) return MOE_ERR_INVALID_ARG;
  if (prepared && cfg->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (N == 0) return MOE_OK;
  if (!e_bias || !topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
  if ((scores_in || (flags & MOE_ROUTE_SCORES_OUT)) && !scores) return MOE_ERR_INVALID_ARG;
  const Workspace L = layout(cfg, N);
  if (!scores_in) {
    if (!x || !w_router) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(w_router)) return MOE_ERR_INVALID_ARG;
    if (!workspace || ws_bytes < L.route_total || !aligned16(workspace)) return MOE_ERR_WORKSPACE;
  }
  float* sc = scores_in || (flags & MOE_ROUTE_SCORES_OUT) ? scores : nullptr;
  return route_impl(cfg, N, x, w_router, prepared, e_bias, sc, scores_in, topk_idx, topk_w, workspace, L,
                    (hipStream_t)stream);
}

size_t moe_dispatch_workspace_size(const moe_config* cfg, int64_t N) {
  if (check_cfg(cfg) != MOE_OK || check_n(cfg, N) != MOE_OK) return 0;
  return dispatch_layout(cfg, N).total;
}

moe_status moe_dispatch(const moe_config* cfg, int64_t N, const int32_t* topk_idx, int32_t* counts, int32_t* offsets,
                        int32_t* sorted_pair, int32_t* inv_row, void* workspace, size_t ws_bytes, void* stream) {
  moe_status st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_n(cfg, N)) != MOE_OK) return st;
  if (!counts || !offsets) return MOE_ERR_INVALID_ARG;
  if (N > 0 && (!topk_idx || !sorted_pair || !inv_row)) return MOE_ERR_INVALID_ARG;
  const DispatchWorkspace L = dispatch_layout(cfg, N);
  if (L.total > 0 && (!workspace || ws_bytes < L.total || !aligned16(workspace))) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  if (N == 0) {
    // empty lists: counts and offsets are all zero (one fill over both)
    if (launch_fill2_i32(counts, cfg->n_routed_experts, offsets, cfg->n_routed_experts + 1, 0, s) != hipSuccess)
      return MOE_ERR_HIP;
    return MOE_OK;
  }
  const TileSpec none{0, nullptr, nullptr, 0, nullptr, nullptr};
  return dispatch_impl(cfg, N, topk_idx, counts, offsets, sorted_pair, inv_row, at<int32_t>(workspace, L.chunk_counts),
                       at<int32_t>(workspace, L.chunk_base), none, none, 0, s);
}

moe_status moe_forward(const moe_config* cfg, int64_t N, const void* x, const moe_weights* wt, void* y,
                       int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out, void* workspace, size_t ws_bytes,
                       void* stream) {
  moe_status st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_n(cfg, N)) != MOE_OK) return st;
  if (!wt) return MOE_ERR_INVALID_ARG;
  if (N == 0) return MOE_OK;
  if ((st = check_expert_args(cfg, N, x, wt, y)) != MOE_OK) return st;
  if (!wt->e_bias) return MOE_ERR_INVALID_ARG;
  const bool prepared = wt->w_router_prepared != nullptr;
  if (prepared && cfg->dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  const void* wg = prepared ? wt->w_router_prepared : (const void*)wt->w_router;
  if (!wg || !aligned16(wg)) return MOE_ERR_INVALID_ARG;
  const Workspace L = layout(cfg, N);
  if (!workspace || ws_bytes < L.total || !aligned16(workspace)) return MOE_ERR_WORKSPACE;

  hipStream_t s = (hipStream_t)stream;
  void* ws = workspace;
  const int E = cfg->n_routed_experts, k = cfg->num_experts_per_tok;
  int32_t* idx = at<int32_t>(ws, L.idx);
  float* w = at<float>(ws, L.w);
  int32_t* counts = at<int32_t>(ws, L.counts);

  // the scores are not kept
  if ((st = route_impl(cfg, N, x, wg, prepared, wt->e_bias, nullptr, false, idx, w, ws, L, s)) != MOE_OK) return st;
  if ((st = forward_dispatch(cfg, N, idx, ws, L, s)) != MOE_OK) return st;
  if ((st = experts_impl(cfg, N, x, wt, w, y, ws, L, s)) != MOE_OK) return st;

  if (topk_idx_out && hipMemcpyAsync(topk_idx_out, idx, sizeof(int32_t) * N * k, hipMemcpyDeviceToDevice, s))
    return MOE_ERR_HIP;
  if (topk_w_out && hipMemcpyAsync(topk_w_out, w, sizeof(float) * N * k, hipMemcpyDeviceToDevice, s))
    return MOE_ERR_HIP;
  if (counts_out && hipMemcpyAsync(counts_out, counts, sizeof(int32_t) * E, hipMemcpyDeviceToDevice, s))
    return MOE_ERR_HIP;
  return MOE_OK;
}

moe_status moe_forward_routed(const moe_config* cfg, int64_t N, const void* x, const moe_weights* wt,
                              const int32_t* topk_idx, const float* topk_w, void* y, int32_t* counts_out,
                              void* workspace, size_t ws_bytes, void* stream) {
  moe_status st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_n(cfg, N)) != MOE_OK) return st;
  if (!wt) return MOE_ERR_INVALID_ARG;
  if (N == 0) return MOE_OK;
  if ((st = check_expert_args(cfg, N, x, wt, y)) != MOE_OK) return st;
  if (!topk_idx || !topk_w) return MOE_ERR_INVALID_ARG;
  const Workspace L = layout(cfg, N);
  if (!workspace || ws_bytes < L.total || !aligned16(workspace)) return MOE_ERR_WORKSPACE;

  hipStream_t s = (hipStream_t)stream;
  void* ws = workspace;
  int32_t* counts = at<int32_t>(ws, L.counts);
  if ((st = forward_dispatch(cfg, N, topk_idx, ws, L, s)) != MOE_OK) return st;
  if ((st = experts_impl(cfg, N, x, wt, topk_w, y, ws, L, s)) != MOE_OK) return st;
  if (counts_out && hipMemcpyAsync(counts_out, counts, sizeof(int32_t) * cfg->n_routed_experts,
                                   hipMemcpyDeviceToDevice, s))
    return MOE_ERR_HIP;
  return MOE_OK;
}

size_t moe_noalloc_scratch_bytes(void) { return kScratchBytes; }

moe_status moe_forward_noalloc(const moe_config* cfg, int64_t N, const void* x, const moe_weights* w, void* y,
                               int32_t* topk_idx_out, float* topk_w_out, int32_t* counts_out, void* stream) {
  moe_status st = check_cfg(cfg);
  if (st != MOE_OK) return st;
  if ((st = check_n(cfg, N)) != MOE_OK) return st;
  if (N == 0) return w ? MOE_OK : MOE_ERR_INVALID_ARG;
  const size_t need = layout(cfg, N).total;
  if (need > kScratchBytes) return MOE_ERR_WORKSPACE;  // the batch needs more than the fixed scratch
  void* ws = scratch_on_current_device();
  if (!ws) return MOE_ERR_HIP;
  return moe_forward(cfg, N, x, w, y, topk_idx_out, topk_w_out, counts_out, ws, kScratchBytes, stream);
}

size_t moe_dense_workspace_size(int64_t N, int32_t D, int32_t dff, int32_t dtype) {
  if (check_dense(N, D, dff, dtype, 0.f) != MOE_OK) return 0;
  return dense_layout(N, dff, dtype).total;
}

moe_status moe_dense_forward(int64_t N, int32_t D, int32_t dff, int32_t dtype, float swiglu_limit, const void* x,
                             const void* gate, const void* up, const void* down, void* y, void* workspace,
                             size_t ws_bytes, void* stream) {
  moe_status st = check_dense(N, D, dff, dtype, swiglu_limit);
  if (st != MOE_OK) return st;
  if (N == 0) return MOE_OK;
  if (!x || !gate || !up || !down || !y || x == y) return MOE_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(gate) || !aligned16(up) || !aligned16(down) || !aligned16(y))
    return MOE_ERR_INVALID_ARG;
  const DenseWorkspace L = dense_layout(N, dff, dtype);
  if (!workspace || ws_bytes < L.total || !aligned16(workspace)) return MOE_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  void* ws = workspace;
  int32_t* ntiles = at<int32_t>(ws, L.ntiles);
  TileSpec t0{L.bm, at<Tile>(ws, L.tiles0), ntiles, 0, ntiles + 2, nullptr};
  TileSpec t1{L.bm, at<Tile>(ws, L.tiles1), ntiles + 1, 0, ntiles + 10, nullptr};
  if (launch_dense_tiles(N, t0, t1, s) != hipSuccess) return MOE_ERR_HIP;
  // one dense problem through the grouped GEMMs: no gather, no row scale
  GroupedArgs g{};
  g.k = 1;
  g.swiglu_limit = swiglu_limit;
  g.tiles = t0.tiles;
  g.n_tiles = ntiles;
  g.work_ctr = t0.work_ctr;
  g.bm = L.bm;
  g.prob[0] = ExpertProblem{x, D, 0, gate, up, 0, D, dff, at<void>(ws, L.H), dff, 0};
  MOE_TRY(ST_GATE_UP, launch_gate_up(dtype, g, L.max_tiles, s));
  g.tiles = t1.tiles;
  g.n_tiles = ntiles + 1;
  g.work_ctr = t1.work_ctr;
  g.prob[0] = ExpertProblem{at<void>(ws, L.H), dff, 0, down, nullptr, 0, dff, D, y, D, 0};
  MOE_TRY(ST_DOWN, launch_down(dtype, g, L.max_tiles, s));
  return MOE_OK;
}

const char* moe_status_str(moe_status status) {
  switch (status) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: invalid config field, size or pointer";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: valid layer outside the kernels' limits";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a HIP launch or runtime call failed";
  }
  return "unknown moe_status";
}

moe_status moe_profile_begin(void) { return moe_profile_begin_mask(~0u); }

moe_status moe_profile_begin_mask(uint32_t stage_mask) {
  g_prof_mask = stage_mask;
  g_recs.clear();
  g_pool_next = 0;
  g_prof_err = false;
  g_prof_on = true;
  return MOE_OK;
}

moe_status moe_profile_end(double* ms_per_stage, int32_t* launches_per_stage, int32_t n_stages) {
  g_prof_on = false;
  for (int i = 0; i < n_stages; ++i) {
    if (ms_per_stage) ms_per_stage[i] = 0.0;
    if (launches_per_stage) launches_per_stage[i] = 0;
  }
  moe_status st = g_prof_err ? MOE_ERR_HIP : MOE_OK;
  for (const ProfRec& r : g_recs) {
    float ms = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
      st = MOE_ERR_HIP;
      continue;
    }
    if (r.stage < n_stages) {
      if (ms_per_stage) ms_per_stage[r.stage] += ms;
      if (launches_per_stage) launches_per_stage[r.stage] += 1;
    }
  }
  g_recs.clear();
  g_pool_next = 0;
  return st;
}

const char* moe_stage_name(int32_t stage) {
  return (stage >= 0 && stage < ST_COUNT_STAGES) ? kStageNames[stage] : nullptr;
}

int32_t moe_stage_count(void) { return ST_COUNT_STAGES; }

}  // extern "C"
