"""Shared GPU test plumbing: seeded inputs on host and device, calls through the C ABI, oracle references.

Inputs come only from synth (the seeded generator); expected values come only from oracle. Nothing
here computes any step of the layer itself.
"""
from __future__ import annotations

import math

import numpy as np

import oracle
import synth


def torch_mod():
    import torch

    return torch


def to_device(a: np.ndarray, device="cuda"):
    """Host array (float32, int32, or bf16 bits as uint16) -> device tensor of the matching dtype."""
    torch = torch_mod()
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(a)).to(device)


def to_host(t) -> np.ndarray:
    torch = torch_mod()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def as_f32(a: np.ndarray) -> np.ndarray:
    return synth.bf16_to_f32(a) if a.dtype == np.uint16 else a.astype(np.float32)


_weight_cache = {}


def device_weights(w: synth.Workload, generate_on_device: bool):
    """Router (host + device) and expert weights (device) of workload w; the expert weights are cached per
    weight recipe so that workloads sharing weights (prefill / decode) generate them once."""
    torch = torch_mod()
    key = (w.seed, w.D, w.E, w.d, w.n_shared, w.dtype, w.skew)
    if key not in _weight_cache:
        _weight_cache.clear()
        torch.cuda.empty_cache()
        wg, b = synth.router_host(w)
        if generate_on_device:
            dev = synth.experts_device(w)
        else:
            gu, dn = synth.all_experts_host(w)
            dev = {"gate_up": to_device(gu), "down": to_device(dn)}
            sh = synth.shared_host(w)
            if sh is not None:
                dev.update(sh_gate=to_device(sh[0]), sh_up=to_device(sh[1]), sh_down=to_device(sh[2]))
        dev["w_router"] = to_device(wg)
        dev["e_bias"] = to_device(b)
        torch.cuda.synchronize()
        _weight_cache[key] = (wg, b, dev)
    return _weight_cache[key]


def drop_weights():
    torch = torch_mod()
    _weight_cache.clear()
    torch.cuda.empty_cache()


def expert_table(w: synth.Workload, experts) -> oracle.ExpertTable:
    """Host copies of the listed experts (regenerated from the seeded streams) and the shared expert."""
    needed = {int(e): synth.expert_host(w, int(e)) for e in sorted(set(int(e) for e in experts))}
    return oracle.ExpertTable(w, needed, synth.shared_host(w))


def gpu_forward(w: synth.Workload, x_dev, dev_w: dict):
    """moe_forward through the C ABI; returns (y, idx, wt, counts) as host arrays."""
    import sparse_moe_layer_gate_amd as moe

    torch = torch_mod()
    cfg = moe.config_of(w)
    N = x_dev.shape[0]
    ws = moe.alloc_workspace(cfg, N)
    y = torch.empty_like(x_dev)
    idx = torch.empty((N, w.k), dtype=torch.int32, device="cuda")
    wt = torch.empty((N, w.k), dtype=torch.float32, device="cuda")
    counts = torch.empty((w.E,), dtype=torch.int32, device="cuda")
    moe.moe_forward(cfg, N, x_dev, dev_w, y, ws, idx, wt, counts)
    torch.cuda.synchronize()
    out = to_host(y), to_host(idx), to_host(wt), to_host(counts)
    del ws, y
    return out


def gpu_forward_routed(w: synth.Workload, x_dev, dev_w: dict, idx: np.ndarray, wt: np.ndarray):
    """moe_forward_routed through the C ABI with host routing (idx, wt); returns (y, counts) as host arrays."""
    import sparse_moe_layer_gate_amd as moe

    torch = torch_mod()
    cfg = moe.config_of(w)
    N = x_dev.shape[0]
    ws = moe.alloc_workspace(cfg, N)
    y = torch.empty_like(x_dev)
    counts = torch.empty((w.E,), dtype=torch.int32, device="cuda")
    moe.moe_forward_routed(cfg, N, x_dev, dev_w, to_device(np.ascontiguousarray(idx, np.int32)),
                           to_device(np.ascontiguousarray(wt, np.float32)), y, ws, counts)
    torch.cuda.synchronize()
    out = to_host(y), to_host(counts)
    del ws, y
    return out


# Constant of the statistical float32 accumulation bound below (in standard-deviation-like units of the
# rounding random walk). Sequential float32 accumulation of the 3 D exact products, the order with the
# most roundings, stays under 2.6 of these units on 64 tokens of the GLM-4.5 / Air / GLM-5 shapes; a
# router evaluated with W_g rounded to bfloat16 lands at 100-700 units (median) on the same inputs.
ROUTER_ACC_C = 8.0
U32 = 2.0 ** -24  # unit roundoff of float32


def logit_tolerance(w: synth.Workload, x: np.ndarray, wg: np.ndarray) -> np.ndarray:
    """Bound on |r_gpu - r_oracle| per (token, expert) for a float32 gate ("Group Router", How it works:
    the gate is evaluated in float32). The device logit is a float32 accumulation of at most 3 D exact
    products (bf16 activations times the three bf16 pieces of the router weight; D fused products for
    float32 activations). Each rounding adds at most u times a partial sum, and for products of random
    sign the partial sums grow like a random walk, so the accumulated error is of order
    sqrt(n) u ||x o W||_2 with n = 3 D roundings -- far tighter than the worst-case n u sum |x W|, and
    a bfloat16 gate (relative error 2^-9 per weight) exceeds it by two orders of magnitude. The
    oracle's own rounding of r adds one float32 spacing."""
    xf = as_f32(x).astype(np.float64)
    w64 = np.asarray(wg, np.float64)
    l2 = np.sqrt((xf * xf) @ (w64 * w64).T)
    r = xf @ w64.T
    return ROUTER_ACC_C * math.sqrt(3 * w.D) * U32 * l2 + np.spacing(np.abs(r).astype(np.float32)).astype(np.float64)


def score_tolerance(w: synth.Workload, x: np.ndarray, wg: np.ndarray) -> np.ndarray:
    """Bound on |s_gpu - s_oracle| per (token, expert): the logit bound through the sigmoid's slope
    s (1 - s) at the exact logit, plus 4 float32 spacings of s for the device exponential and divide,
    plus 2^-125: below about 1e-38 (logits under -87) a float32 exponential overflows or the quotient
    leaves the normal range, where the oracle's double sigmoid still rounds to a subnormal."""
    xf = as_f32(x).astype(np.float64)
    r = xf @ np.asarray(wg, np.float64).T
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-r))
    return (s * (1.0 - s) * logit_tolerance(w, x, wg) + 4 * np.spacing(s.astype(np.float32)).astype(np.float64)
            + 2.0 ** -125)


def within_near_tie(margin: np.ndarray, ds: np.ndarray) -> np.ndarray:
    """Whether a routing difference is explained by score errors of at most ds per expert: a decision
    between two experts flips only if their s' gap is at most 2 ds, one between two groups (each group
    score sums two s') only if the gap is at most 4 ds, plus a few float32 spacings of the s' and group
    score roundings (values below 4). The oracle's margin is the smallest such gap."""
    return margin <= 4.0 * ds + 2.0 ** -20


def sample_tokens(N: int, count: int, seed: int = 0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    fixed = [0, N - 1, N // 2]
    extra = rng.choice(N, size=min(count, N), replace=False)
    return np.unique(np.concatenate([np.array(fixed[: min(3, N)]), extra]))[:max(count, 1) + 3]


def tile_cover_tokens(w: synth.Workload, idx: np.ndarray, bm: int):
    """Tokens that put at least one row into every row tile of the grouped GEMMs' tile lists: for each
    routed expert (rows = its (token, slot) pairs in ascending token order, as dispatch places them) and
    for the shared expert (rows = tokens in order), the first and last row of every bm-row tile, so each
    expert's partial last tile is included. Returns (tokens, tiles, covered)."""
    flat = idx.ravel()
    order = np.argsort(flat, kind="stable")  # pairs grouped by expert, ascending pair index inside
    counts = np.bincount(flat, minlength=w.E)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    tok_of_row = order // w.k
    picks = []
    tiles = []  # (first row token set) per tile, for the coverage count
    for e in range(w.E):
        for t0 in range(0, int(counts[e]), bm):
            rows = tok_of_row[offsets[e] + t0: offsets[e] + min(t0 + bm, int(counts[e]))]
            picks += [rows[0], rows[-1]]
            tiles.append(rows)
    if w.n_shared > 0:
        for t0 in range(0, w.N, bm):
            rows = np.arange(t0, min(t0 + bm, w.N))
            picks += [rows[0], rows[-1]]
            tiles.append(rows)
    tokens = np.unique(np.asarray(picks, np.int64))
    covered = sum(bool(np.intersect1d(rows, tokens).size) for rows in tiles)
    return tokens, len(tiles), covered


def rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    ref64 = ref.astype(np.float64)
    den = np.abs(ref64).max()
    return float(np.abs(y.astype(np.float64) - ref64).max() / (den if den > 0 else 1.0))


TOL = {"f32": 1e-4, "bf16": 2e-2}


def bf16_bits(a: np.ndarray) -> np.ndarray:
    return synth.f32_to_bf16(a)


def isclose_ulps(a, b, n):
    a = np.asarray(a, np.float32)
    b = np.asarray(b, np.float32)
    return np.abs(a.astype(np.float64) - b) <= n * np.spacing(np.maximum(np.abs(a), np.abs(b)))


def std_of(fan_in):
    return 1.0 / math.sqrt(fan_in)


def check_forward(w, x, wg, b, y, idx, wt, counts, tokens):
    """Routing check over all tokens, output check over `tokens`. A token's expert ids may differ from
    the oracle's only at a near-tie: the oracle's decision margin within what the score bound can flip."""
    s_ref = oracle.scores(w, x, wg)
    idx_ref, w_ref = oracle.select(w, s_ref, b)
    margin = oracle.select_margin(w, s_ref, b)
    tol_s = score_tolerance(w, x, wg).max(axis=1)
    differ = np.any(idx != idx_ref, axis=1)
    assert np.all(within_near_tie(margin[differ], tol_s[differ])), "a routing difference away from a near-tie"
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=w.E))
    same = ~differ
    # weights from the GPU's own scores: the score bound t propagated through w_i = alpha s_i / S,
    # |dw_i| <= alpha (t / S + s_i k t / S^2), plus 4 ulp of the float32 steps
    chosen = np.take_along_axis(s_ref, idx_ref.astype(np.int64), 1).astype(np.float64)
    aw = 1.0 if w.alpha_on_output else w.alpha  # the factor the weights carry
    if w.norm:
        S = chosen.sum(axis=1, keepdims=True) + w.eps
        bound = aw * (tol_s[:, None] / S + chosen * w.k * tol_s[:, None] / S**2)
    else:
        bound = aw * tol_s[:, None] * np.ones_like(chosen)
    bound = bound + 4 * np.spacing(np.abs(w_ref).astype(np.float32))
    dev_w = np.abs(wt.astype(np.float64) - w_ref)
    assert np.all(dev_w[same] <= bound[same]), f"weight deviation {dev_w[same].max():.3g}"
    # per-token reference: the oracle's routing, or the GPU's where they differ at a near-tie
    tokens = np.unique(np.concatenate([tokens, np.flatnonzero(differ)[:8]]))
    r_idx = np.where(differ[:, None], idx, idx_ref)
    r_w = np.where(differ[:, None], wt, w_ref)
    table = expert_table(w, r_idx[tokens].ravel())
    y_ref = oracle.forward_tokens(w, tokens, x, table, r_idx, r_w)
    err = rel_err(as_f32(y[tokens]), y_ref)
    print(f"  {w.name}: tokens={tokens.size} differ={int(differ.sum())} "
          f"max_w_dev={dev_w[same].max() if same.any() else 0:.3g} rel_err={err:.3g}", flush=True)
    assert err <= TOL[w.dtype], err
    return err
