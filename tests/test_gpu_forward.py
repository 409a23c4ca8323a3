"""GPU parity of the whole layer (moe_forward through the C ABI) against the oracle.

Protocol: the GPU's expert ids must equal the oracle's for every token whose oracle decision gap exceeds
what the float32 score bound can flip (near-ties may flip); the output is compared per token with the
oracle evaluated on the oracle's routing, or on the GPU's routing for the near-tie tokens, at
max|dy| / max|y| <= 1e-4 (float32 layers) or <= 2e-2 (bfloat16 layers). Full-size workloads are checked
on a token set that covers every row tile of both grouped GEMMs (every token's routing is checked);
small shapes that span several tiles and ragged tails are checked whole.
"""
from dataclasses import replace

import numpy as np
import pytest

import oracle
import synth
from tests import _harness as H

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", synth.WORKLOAD_ORDER)
def test_forward_workload(name):
    """Full-size workloads. Routing is checked on every token. The output is checked on every token of
    the small batches, and elsewhere on a set of tokens that puts at least one row into every row tile
    of both grouped GEMMs (each routed expert's 256-row tiles including its partial last one, and the
    shared expert's tiles); a full output row spans every column tile of both GEMMs."""
    w = synth.WORKLOADS[name]
    print(f"[forward] {name} N={w.N} D={w.D} E={w.E} k={w.k} d={w.d}", flush=True)
    big = w.E * w.d * w.D > 50_000_000
    wg, b, dev = H.device_weights(w, generate_on_device=big)
    x = synth.x_host(w)
    x_dev = H.to_device(x)
    y, idx, wt, counts = H.gpu_forward(w, x_dev, dev)
    # the forward's routing is moe_route's, bit for bit, and is what the oracle's selection makes of the
    # scores moe_route writes
    s_g, idx_r, wt_r = route_gpu(w, x_dev, dev)
    assert np.array_equal(idx, idx_r) and np.array_equal(wt.view(np.uint32), wt_r.view(np.uint32))
    idx_s, wt_s = oracle.select(w, s_g, b)
    assert np.array_equal(idx_s, idx) and np.array_equal(wt_s.view(np.uint32), wt.view(np.uint32))
    if w.N <= 512:
        tokens = np.arange(w.N)
    else:
        bm = 16 if w.N * w.k < 4 * w.E else 256
        tokens, n_tiles, covered = H.tile_cover_tokens(w, idx, bm)
        print(f"  tile coverage: {covered}/{n_tiles} tiles of {bm} rows ({100.0 * covered / n_tiles:.1f}%), "
              f"{tokens.size} tokens", flush=True)
        assert covered == n_tiles
    H.check_forward(w, x, wg, b, y, idx, wt, counts, tokens)


def route_gpu(w, x_dev, dev):
    """moe_route on device inputs; returns (scores, idx, wt) as host arrays."""
    import torch

    import sparse_moe_layer_gate_amd as moe

    cfg = moe.config_of(w)
    N = x_dev.shape[0]
    s = torch.empty((N, w.E), dtype=torch.float32, device="cuda")
    idx = torch.empty((N, w.k), dtype=torch.int32, device="cuda")
    wt = torch.empty((N, w.k), dtype=torch.float32, device="cuda")
    moe.moe_route(cfg, N, x_dev, dev["w_router"], dev["e_bias"], s, idx, wt, flags=moe.MOE_ROUTE_SCORES_OUT,
                  workspace=moe.alloc_workspace(cfg, N))
    torch.cuda.synchronize()
    return H.to_host(s), H.to_host(idx), H.to_host(wt)


SMALL = [
    # several row tiles per expert, column tails on both GEMMs (D = 320, d = 192), ragged rows
    dict(N=300, D=320, E=24, G=4, TG=2, k=5, d=192, n_shared=1, alpha=2.5),
    dict(N=1000, D=512, E=8, G=1, TG=1, k=2, d=256, n_shared=1, alpha=1.0),
    # experts averaging 384+ rows: 256-row tiles, with column tails on both GEMMs
    dict(N=2000, D=320, E=8, G=2, TG=1, k=2, d=192, n_shared=1, alpha=2.5),
    # 256-row tiles with one- and two-step K loops (D = 64 / 128, d = 128 / 64), skewed loads
    dict(N=700, D=64, E=4, G=1, TG=1, k=2, d=128, n_shared=1, alpha=2.5, skew=1.0),
    dict(N=900, D=128, E=6, G=2, TG=1, k=2, d=64, n_shared=0, alpha=2.5),
    dict(N=77, D=256, E=32, G=8, TG=3, k=6, d=128, n_shared=2, alpha=2.5),
    dict(N=129, D=192, E=12, G=1, TG=1, k=3, d=64, n_shared=0, alpha=2.5),
    dict(N=50, D=256, E=16, G=4, TG=2, k=4, d=128, n_shared=1, alpha=2.5, norm=False),
    # gate_up tiles of at most 64 rows (the weight-streaming ring) with one- and two-step K loops
    dict(N=100, D=64, E=8, G=1, TG=1, k=2, d=128, n_shared=1, alpha=2.5),
    dict(N=100, D=128, E=8, G=2, TG=1, k=2, d=64, n_shared=0, alpha=2.5),
    # 256-row tiles holding few rows (~19 per expert), skewed: some experts span two tiles
    dict(N=150, D=320, E=16, G=1, TG=1, k=2, d=192, n_shared=1, alpha=2.5, skew=1.0),
    # the widest routing the ABI takes (E = 512 in 64 groups, k = 32): decode tiles, then 256-row tiles,
    # and a combine over 32 slots
    dict(N=48, D=128, E=512, G=64, TG=8, k=32, d=64, n_shared=1, alpha=2.5),
    dict(N=1024, D=128, E=512, G=64, TG=8, k=32, d=64, n_shared=1, alpha=2.5),
    # 16-row (decode) tiles with column tails and a short last K stage (D = 320, d = 192); the
    # skewed router gives some experts several 16-row tiles
    dict(N=23, D=320, E=24, G=4, TG=2, k=4, d=192, n_shared=1, alpha=2.5),
    dict(N=60, D=320, E=64, G=1, TG=1, k=4, d=192, n_shared=1, alpha=2.5, skew=1.0),
    dict(N=1, D=256, E=16, G=4, TG=2, k=4, d=128, n_shared=1, alpha=2.5),
    dict(N=3, D=128, E=8, G=2, TG=1, k=1, d=64, n_shared=1, alpha=2.5),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"N{c['N']}-D{c['D']}-E{c['E']}-k{c['k']}-d{c['d']}")
def test_forward_small_whole(case, dtype):
    w = replace(synth.WORKLOADS["tiny_fp32"], name="small", dtype=dtype, seed=3, **case)
    print(f"[small] {case} {dtype}", flush=True)
    wg, b, dev = H.device_weights(w, generate_on_device=False)
    x = synth.x_host(w)
    y, idx, wt, counts = H.gpu_forward(w, H.to_device(x), dev)
    H.check_forward(w, x, wg, b, y, idx, wt, counts, np.arange(w.N))


def test_forward_deterministic_and_permutation_equivariant():
    """Same inputs, same bits; a permutation of the tokens permutes the output rows bit for bit."""
    w = replace(synth.WORKLOADS["tiny_fp32"], name="perm", N=700, D=512, E=32, G=4, TG=2, k=6, d=256,
                dtype="bf16", seed=5)
    _, _, dev = H.device_weights(w, generate_on_device=False)
    x = synth.x_host(w)
    y1, i1, w1, _ = H.gpu_forward(w, H.to_device(x), dev)
    y2, i2, w2, _ = H.gpu_forward(w, H.to_device(x), dev)
    assert np.array_equal(y1, y2) and np.array_equal(i1, i2) and np.array_equal(w1, w2)
    perm = np.random.default_rng(0).permutation(w.N)
    y3, i3, w3, _ = H.gpu_forward(w, H.to_device(x[perm]), dev)
    assert np.array_equal(y3, y1[perm]) and np.array_equal(i3, i1[perm]) and np.array_equal(w3, w1[perm])


@pytest.mark.parametrize("name,tokens", [("glm5_decode", None), ("air_prefill", None), ("glm5_decode", 1)])
def test_forward_prepared_router_bitexact(name, tokens):
    """The forward on moe_router_prepare's output (the split taken once) equals the forward that splits
    the float32 router weight itself, bit for bit (one token: the small-batch gate kernel)."""
    import sparse_moe_layer_gate_amd as moe

    w = synth.WORKLOADS[name]
    if tokens is not None:
        w = w.with_tokens(tokens)
    _, _, dev = H.device_weights(w, generate_on_device=True)
    x_dev = H.to_device(synth.x_host(w))
    y1, i1, w1, c1 = H.gpu_forward(w, x_dev, dev)
    dev2 = dict(dev)
    dev2["w_router_prepared"] = moe.moe_router_prepare(moe.config_of(w), dev["w_router"])
    del dev2["w_router"]
    y2, i2, w2, c2 = H.gpu_forward(w, x_dev, dev2)
    assert np.array_equal(y1, y2) and np.array_equal(i1, i2) and np.array_equal(w1, w2) and np.array_equal(c1, c2)


def test_device_generator_matches_host():
    """The device build of the seeded generator reproduces the host build bit for bit."""
    w = synth.WORKLOADS["glm5_prefill"]
    _, _, dev = H.device_weights(w, generate_on_device=True)
    for e in (0, 77, w.E - 1):
        gu, dn = synth.expert_host(w, e)
        assert np.array_equal(H.to_host(dev["gate_up"][e]), gu)
        assert np.array_equal(H.to_host(dev["down"][e]), dn)
    sg, su, sd = synth.shared_host(w)
    assert np.array_equal(H.to_host(dev["sh_gate"]), sg)
    assert np.array_equal(H.to_host(dev["sh_up"]), su)
    assert np.array_equal(H.to_host(dev["sh_down"]), sd)


def test_forward_reuses_workspace():
    """One workspace, sized for the largest batch, serves calls of falling and rising N (256-row tiles,
    then 16-row tiles, then both lists, then 256-row tiles again): every output equals that of a call with a fresh
    workspace, bit for bit. Each call rebuilds the tile lists and zeroes the prefill kernels' work
    counters, whatever the workspace held."""
    import torch

    import sparse_moe_layer_gate_amd as moe

    w = replace(synth.WORKLOADS["tiny_fp32"], name="reuse", N=1500, D=256, E=16, G=4, TG=2, k=4, d=128,
                n_shared=1, alpha=2.5, dtype="bf16", seed=11, skew=1.0)
    _, _, dev = H.device_weights(w, generate_on_device=False)
    x_dev = H.to_device(synth.x_host(w))
    cfg = moe.config_of(w)
    ws = moe.alloc_workspace(cfg, w.N)
    # 10 tokens: 40 pairs on 16 experts run the 16-row tiles; 20 and 30 tokens (5 and 7.5 rows per
    # expert) build both lists and let the device pick
    for n in (1500, 700, 10, 30, 20, 1500):
        print(f"[reuse] N={n}", flush=True)
        y = torch.empty((n, w.D), dtype=x_dev.dtype, device="cuda")
        moe.moe_forward(cfg, n, x_dev[:n], dev, y, ws)
        torch.cuda.synchronize()
        y_fresh, _, _, _ = H.gpu_forward(w, x_dev[:n], dev)
        assert np.array_equal(H.to_host(y), y_fresh), n


# 4 to 12 rows per expert on average (bf16): both tile lists are built and the scan kernel keeps the
# 16-row list when the largest expert has at most 24 rows, else the 256-row list.
PICK = [
    (dict(N=100, D=320, E=64, G=1, TG=1, k=4, d=192, n_shared=1, alpha=2.5), "decode"),
    (dict(N=120, D=320, E=64, G=1, TG=1, k=4, d=192, n_shared=1, alpha=2.5, skew=1.0), "prefill"),
    (dict(N=100, D=128, E=512, G=64, TG=8, k=32, d=64, n_shared=1, alpha=2.5), None),
]


@pytest.mark.parametrize("case,kind", PICK, ids=lambda c: f"N{c['N']}-E{c['E']}" if isinstance(c, dict) else str(c))
def test_forward_device_picked_kernels(case, kind):
    w = replace(synth.WORKLOADS["tiny_fp32"], name="pick", dtype="bf16", seed=5, **case)
    assert 4 * w.E <= w.N * w.k < 12 * w.E
    print(f"[pick] {case} expect {kind}", flush=True)
    wg, b, dev = H.device_weights(w, generate_on_device=False)
    x = synth.x_host(w)
    y, idx, wt, counts = H.gpu_forward(w, H.to_device(x), dev)
    if kind == "decode":
        assert counts.max() <= 24
    elif kind == "prefill":
        assert counts.max() > 24
    H.check_forward(w, x, wg, b, y, idx, wt, counts, np.arange(w.N))
