"""GPU parity of the router and the dispatch against the oracle, through the C ABI.

Bar: given the oracle's float32 scores, the GPU's expert ids and weights are bit-identical
(moe_route with MOE_ROUTE_SCORES_IN); the GPU's own scores are within a float32 accumulation bound of
the oracle's (one a bfloat16 gate fails, tests/test_router_bound.py); the GPU's ids and weights are
bit-identical to the oracle's selection applied to the scores the GPU wrote, and differ from the
oracle's routing only at near-ties; counts, offsets, sorted_pair and inv_row are bit-identical.
"""
from dataclasses import replace

import numpy as np
import pytest

import oracle
import synth
from tests import _harness as H

pytestmark = pytest.mark.gpu

ALL = synth.WORKLOAD_ORDER


def _route_gpu(w, N, s_host=None, x_host=None, wg=None, b=None):
    import torch

    import sparse_moe_layer_gate_amd as moe

    cfg = moe.config_of(w)
    idx = torch.empty((N, w.k), dtype=torch.int32, device="cuda")
    wt = torch.empty((N, w.k), dtype=torch.float32, device="cuda")
    b_d = H.to_device(b)
    if s_host is not None:
        s_d = H.to_device(s_host)
        moe.moe_route(cfg, N, None, None, b_d, s_d, idx, wt, flags=moe.MOE_ROUTE_SCORES_IN)
    else:
        s_d = torch.empty((N, w.E), dtype=torch.float32, device="cuda")
        moe.moe_route(cfg, N, H.to_device(x_host), H.to_device(wg), b_d, s_d, idx, wt,
                      flags=moe.MOE_ROUTE_SCORES_OUT, workspace=moe.alloc_workspace(cfg, N))
    torch.cuda.synchronize()
    return H.to_host(s_d), H.to_host(idx), H.to_host(wt)


@pytest.mark.parametrize("name", ALL)
def test_selection_bitexact_given_scores(name):
    w = synth.WORKLOADS[name]
    print(f"[select] {name} N={w.N}", flush=True)
    x = synth.x_host(w)
    wg, b = synth.router_host(w)
    s = oracle.scores(w, x, wg)
    idx_ref, w_ref = oracle.select(w, s, b)
    _, idx, wt = _route_gpu(w, w.N, s_host=s, b=b)
    assert np.array_equal(idx, idx_ref)
    assert np.array_equal(wt.view(np.uint32), w_ref.view(np.uint32))


TIE_CASES = [
    dict(E=16, G=4, TG=2, k=4),
    dict(E=24, G=3, TG=2, k=5),
    dict(E=288, G=1, TG=1, k=8),
    dict(E=512, G=64, TG=8, k=32),
    dict(E=256, G=8, TG=4, k=8, norm=False),
    dict(E=64, G=8, TG=8, k=6),
    dict(E=8, G=1, TG=1, k=1),
]


@pytest.mark.parametrize("case", TIE_CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
@pytest.mark.parametrize("grid", [True, False])
def test_selection_bitexact_tie_rich(case, grid):
    """Scores on a 1/8 grid (ties everywhere) or continuous; bias on the same grid; signed zeros."""
    w = replace(synth.WORKLOADS["tiny_fp32"], N=777, **case)
    rng = np.random.default_rng(w.E + w.k)
    if grid:
        s = (rng.integers(0, 9, (w.N, w.E)) / 8.0).astype(np.float32)
        b = (rng.integers(-1, 2, w.E) / 8.0).astype(np.float32)
        b[::5] = -0.0
    else:
        s = rng.uniform(0, 1, (w.N, w.E)).astype(np.float32)
        b = rng.uniform(-0.05, 0.05, w.E).astype(np.float32)
    s[:7] = 0.0  # all-zero rows: eps keeps the weights at 0
    idx_ref, w_ref = oracle.select(w, s, b)
    _, idx, wt = _route_gpu(w, w.N, s_host=s, b=b)
    assert np.array_equal(idx, idx_ref)
    assert np.array_equal(wt.view(np.uint32), w_ref.view(np.uint32))


def check_scores(w, x, wg, b, s, idx, wt):
    """The GPU router's float32 scores against the oracle's, and its routing against both the oracle's
    routing and the oracle's selection applied to the GPU's own scores."""
    s_ref = oracle.scores(w, x, wg)
    tol = H.score_tolerance(w, x, wg)
    err = np.abs(s.astype(np.float64) - s_ref)
    ratio = err / tol
    print(f"  {w.name}: max |ds| {err.max():.3g}, max |ds| / bound {ratio.max():.3g}", flush=True)
    assert np.all(err <= tol), f"max err {err.max():.3g}, worst ratio {ratio.max():.3g}"
    # the ids and weights are exactly what the selection makes of the scores the kernel wrote
    idx_s, wt_s = oracle.select(w, s, b)
    assert np.array_equal(idx, idx_s)
    assert np.array_equal(wt.view(np.uint32), wt_s.view(np.uint32))
    # against the oracle's routing: differences only where the oracle's decision margin is within what
    # this token's actual score errors can flip
    idx_ref, _ = oracle.select(w, s_ref, b)
    margin = oracle.select_margin(w, s_ref, b)
    differ = np.any(idx != idx_ref, axis=1)
    if differ.any():
        print(f"  {int(differ.sum())} tokens differ, oracle margins {np.sort(margin[differ])[:8]}", flush=True)
    assert np.all(H.within_near_tie(margin[differ], err.max(axis=1)[differ]))


@pytest.mark.parametrize("name", ALL)
def test_scores_within_bound(name):
    w = synth.WORKLOADS[name]
    print(f"[scores] {name}", flush=True)
    x = synth.x_host(w)
    wg, b = synth.router_host(w)
    s, idx, wt = _route_gpu(w, w.N, x_host=x, wg=wg, b=b)
    check_scores(w, x, wg, b, s, idx, wt)


# Router GEMM tile shapes: E past 256 and not a multiple of 32 (two blocks of five 32-expert tiles, the
# last partly past E), E = 100 (four tiles, the last partly past E), batches of one token block and of
# one partial block (two tiles per block), token counts that leave a partial 128-token block; and
# batches of one to four tokens (the one-wave-per-expert kernel), among them D = 64 (fewer 8-element
# chunks than lanes), E = 512 and the GLM-5 router's D = 6144.
GEMM_SHAPES = [
    dict(N=777, D=256, E=300, k=8),
    dict(N=260, D=512, E=100, k=6),
    dict(N=5, D=320, E=40, k=4),
    dict(N=128, D=192, E=96, k=2),
    dict(N=1, D=6144, E=256, k=8),
    dict(N=2, D=5120, E=160, k=8),
    dict(N=3, D=320, E=40, k=4),
    dict(N=4, D=64, E=512, k=8),
]


@pytest.mark.parametrize("case", GEMM_SHAPES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_scores_within_bound_gemm_shapes(case):
    w = replace(synth.WORKLOADS["tiny_fp32"], name="router_shape", G=1, TG=1, dtype="bf16", seed=13, **case)
    print(f"[scores] {case}", flush=True)
    x = synth.x_host(w)
    wg, b = synth.router_host(w)
    s, idx, wt = _route_gpu(w, w.N, x_host=x, wg=wg, b=b)
    check_scores(w, x, wg, b, s, idx, wt)


def _dispatch_gpu(w, idx):
    import torch

    import sparse_moe_layer_gate_amd as moe

    cfg = moe.config_of(w)
    N = idx.shape[0]
    ws = moe.alloc_workspace(cfg, N)
    counts = torch.empty(w.E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(w.E + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(N * w.k, dtype=torch.int32, device="cuda")
    inv = torch.empty(N * w.k, dtype=torch.int32, device="cuda")
    moe.moe_dispatch(cfg, N, H.to_device(np.ascontiguousarray(idx, np.int32)), counts, offsets, sp, inv, ws)
    torch.cuda.synchronize()
    return H.to_host(counts), H.to_host(offsets), H.to_host(sp), H.to_host(inv)


@pytest.mark.parametrize("name", ALL)
def test_dispatch_bitexact(name):
    w = synth.WORKLOADS[name]
    x = synth.x_host(w)
    wg, b = synth.router_host(w)
    idx, _ = oracle.select(w, oracle.scores(w, x, wg), b)
    got = _dispatch_gpu(w, idx)
    ref = oracle.dispatch(w, idx)
    for g, r, what in zip(got, ref, ["counts", "offsets", "sorted_pair", "inv_row"]):
        assert np.array_equal(g, r), what


@pytest.mark.parametrize("N,E,k,skew", [(1, 16, 4, 0), (255, 16, 4, 0), (257, 16, 4, 0), (70001, 160, 8, 0),
                                        (5000, 256, 8, 1), (3000, 512, 32, 0), (1000, 7, 7, 1)])
def test_dispatch_random(N, E, k, skew):
    w = replace(synth.WORKLOADS["tiny_fp32"], N=N, E=E, G=1, TG=1, k=k)
    rng = np.random.default_rng(N + E)
    if skew:  # most tokens on the first k experts
        base = np.arange(k)
        idx = np.stack([base if rng.random() < 0.9 else rng.choice(E, k, replace=False) for _ in range(N)])
    else:
        idx = np.argsort(rng.random((N, E)), axis=1)[:, :k]
    idx = idx.astype(np.int32)
    got = _dispatch_gpu(w, idx)
    ref = oracle.dispatch(w, idx)
    for g, r, what in zip(got, ref, ["counts", "offsets", "sorted_pair", "inv_row"]):
        assert np.array_equal(g, r), what


@pytest.mark.parametrize("N", [1, 200, 256, 257, 5000])
def test_dispatch_own_workspace(N):
    """moe_dispatch with a workspace of exactly moe_dispatch_workspace_size bytes (none for a batch of one
    256-token chunk, which runs as one kernel; per-chunk scratch above) is bit-exact."""
    import torch

    import sparse_moe_layer_gate_amd as moe

    w = replace(synth.WORKLOADS["tiny_fp32"], N=N, E=64, G=8, TG=4, k=6)
    rng = np.random.default_rng(N)
    idx = np.argsort(rng.random((N, w.E)), axis=1)[:, :w.k].astype(np.int32)
    cfg = moe.config_of(w)
    size = moe.moe_dispatch_workspace_size(cfg, N)
    assert (size == 0) == (N <= 256)
    ws = torch.empty(size, dtype=torch.uint8, device="cuda") if size else None
    counts = torch.empty(w.E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(w.E + 1, dtype=torch.int32, device="cuda")
    sp = torch.empty(N * w.k, dtype=torch.int32, device="cuda")
    inv = torch.empty(N * w.k, dtype=torch.int32, device="cuda")
    moe.moe_dispatch(cfg, N, H.to_device(idx), counts, offsets, sp, inv, ws)
    torch.cuda.synchronize()
    for g, r, what in zip((counts, offsets, sp, inv), oracle.dispatch(w, idx), ["counts", "offsets", "sp", "inv"]):
        assert np.array_equal(H.to_host(g), r), what


@pytest.mark.parametrize("name,tokens", [("glm5_decode", None), ("air_prefill", None), ("glm5_decode", 1),
                                         ("glm5_decode", 3)])
def test_route_prepared_and_without_scores(name, tokens):
    """moe_route on the prepared router weight (moe_router_prepare) gives the same scores, ids and weights,
    bit for bit, as on the float32 weight; without MOE_ROUTE_SCORES_OUT the ids and weights are the same
    and no scores are needed. One and three tokens run the small-batch gate kernel."""
    import torch

    import sparse_moe_layer_gate_amd as moe

    w = synth.WORKLOADS[name]
    if tokens is not None:
        w = w.with_tokens(tokens)
    x = synth.x_host(w)
    wg, b = synth.router_host(w)
    cfg = moe.config_of(w)
    x_d, wg_d, b_d = H.to_device(x), H.to_device(wg), H.to_device(b)
    prep = moe.moe_router_prepare(cfg, wg_d)
    ws = moe.alloc_workspace(cfg, w.N)
    outs = []
    for weight, flags in [(wg_d, moe.MOE_ROUTE_SCORES_OUT), (prep, moe.MOE_ROUTE_SCORES_OUT | moe.MOE_ROUTE_PREPARED),
                          (wg_d, 0), (prep, moe.MOE_ROUTE_PREPARED)]:
        s = torch.full((w.N, w.E), -1.0, device="cuda") if flags & moe.MOE_ROUTE_SCORES_OUT else None
        idx = torch.empty((w.N, w.k), dtype=torch.int32, device="cuda")
        wt = torch.empty((w.N, w.k), dtype=torch.float32, device="cuda")
        moe.moe_route(cfg, w.N, x_d, weight, b_d, s, idx, wt, flags=flags, workspace=ws)
        torch.cuda.synchronize()
        outs.append((None if s is None else H.to_host(s), H.to_host(idx), H.to_host(wt)))
    assert np.array_equal(outs[0][0].view(np.uint32), outs[1][0].view(np.uint32))
    for o in outs[1:]:
        assert np.array_equal(o[1], outs[0][1]) and np.array_equal(o[2].view(np.uint32), outs[0][2].view(np.uint32))


def test_dispatch_leaves_out_invalid_ids():
    w = replace(synth.WORKLOADS["tiny_fp32"], N=300, E=16, G=1, TG=1, k=4)
    rng = np.random.default_rng(9)
    idx = np.argsort(rng.random((300, 16)), axis=1)[:, :4].astype(np.int32)
    bad = rng.random(idx.shape) < 0.05
    idx[bad] = np.where(rng.random(bad.sum()) < 0.5, -1, 16)
    counts, offsets, sp, inv = _dispatch_gpu(w, idx)
    flat = idx.ravel()
    valid = (flat >= 0) & (flat < 16)
    assert np.array_equal(counts, np.bincount(flat[valid], minlength=16))
    n_valid = int(valid.sum())
    assert offsets[-1] == n_valid
    assert np.all(inv[~valid] == -1)
    assert np.array_equal(sp[:n_valid], np.flatnonzero(valid)[np.argsort(flat[valid], kind="stable")])
    assert np.array_equal(inv[sp[:n_valid]], np.arange(n_valid))


def test_zero_tokens_is_noop():
    import torch

    import sparse_moe_layer_gate_amd as moe

    w = synth.WORKLOADS["tiny_fp32"]
    cfg = moe.config_of(w)
    e = torch.empty(0, device="cuda")
    z = torch.zeros((0, w.k), dtype=torch.int32, device="cuda")
    moe.moe_route(cfg, 0, None, None, torch.zeros(w.E, device="cuda"), torch.empty((0, w.E), device="cuda"), z,
                  torch.empty((0, w.k), device="cuda"), flags=moe.MOE_ROUTE_SCORES_IN)
    ws = moe.alloc_workspace(cfg, 0)
    counts = torch.full((w.E,), 7, dtype=torch.int32, device="cuda")
    offsets = torch.full((w.E + 1,), 7, dtype=torch.int32, device="cuda")
    moe.moe_dispatch(cfg, 0, z, counts, offsets, torch.empty(0, dtype=torch.int32, device="cuda"),
                     torch.empty(0, dtype=torch.int32, device="cuda"), ws)
    torch.cuda.synchronize()
    assert int(counts.abs().sum()) == 0 and int(offsets.abs().sum()) == 0
    del e


def test_profile_stage_mask():
    """Per-stage timing records every launched stage, or only the stages of the mask."""
    import torch

    import sparse_moe_layer_gate_amd as moe
    from tests import _harness as H

    w = synth.WORKLOADS["tiny_fp32"]
    _, _, dev = H.device_weights(w, generate_on_device=False)
    x = H.to_device(synth.x_host(w))
    cfg = moe.config_of(w)
    ws = moe.alloc_workspace(cfg, w.N)
    y = torch.empty_like(x)
    moe.profile_begin()
    moe.moe_forward(cfg, w.N, x, dev, y, ws)
    every = moe.profile_end()
    moe.profile_begin(["experts_gate_up"])
    moe.moe_forward(cfg, w.N, x, dev, y, ws)
    only = moe.profile_end()
    assert every["experts_gate_up"][1] == 1 and every["combine"][1] == 1 and every["router_select"][1] == 1
    assert only["experts_gate_up"][1] == 1 and only["experts_gate_up"][0] > 0
    assert all(n == 0 for name, (_, n) in only.items() if name != "experts_gate_up")
