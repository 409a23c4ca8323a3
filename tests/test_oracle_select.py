"""Pins for the oracle's selection and weights (router steps after the gate), independent of the oracle.

Sources: page "Group Router" (GLM-4.5), How it works (s' = s + b; group score = sum of the two largest
s'; keep topk_group groups; top-k inside; w = alpha * s / (sum s + eps)); page "Module 02 -- MoE:
Capacity, Work, and Traffic", section 2 (bias for selection only; test IDs and weights separately with
inputs where s and s + b disagree).
"""
import itertools
import json
import os
from types import SimpleNamespace

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def cfg(E, G, TG, k, alpha=2.5, norm=True, eps=1e-20, D=8, d=8, n_shared=1):
    return SimpleNamespace(D=D, E=E, G=G, TG=TG, k=k, d=d, n_shared=n_shared, alpha=alpha, norm=norm, eps=eps)


def beats(a_val, a_idx, b_val, b_idx):
    """The (value descending, index ascending) order, on IEEE values (+0 == -0)."""
    return a_val > b_val or (a_val == b_val and a_idx < b_idx)


def brute_force_selection(c, s_row, b_row):
    """Enumerate every group subset and every expert subset; return the unique valid expert set."""
    sp = (s_row.astype(np.float32) + b_row.astype(np.float32)).astype(np.float32)
    E, G, TG, k = c.E, c.G, c.TG, c.k
    gs = E // G
    groups = list(range(G))
    if G > 1 and TG < G:
        # Group score as the largest pairwise sum inside the group (equals the top-2 sum: rounding is monotone).
        gscore = []
        for g in groups:
            mem = range(g * gs, (g + 1) * gs)
            gscore.append(max(np.float32(sp[i] + sp[j]) for i in mem for j in mem if i != j))
        valid = [K for K in itertools.combinations(groups, TG)
                 if all(beats(gscore[g], g, gscore[h], h) for g in K for h in groups if h not in K)]
        assert len(valid) == 1, "exactly one kept-group set can be valid"
        kept = set(valid[0])
    else:
        kept = set(groups)
    elig = [e for e in range(E) if e // gs in kept]
    valid = [S for S in itertools.combinations(elig, k)
             if all(beats(sp[i], i, sp[j], j) for i in S for j in elig if j not in S)]
    assert len(valid) == 1, "exactly one expert set can be valid"
    return set(valid[0]), kept, sp


def check_slot_order(idx_row, sp):
    for a, b in zip(idx_row[:-1], idx_row[1:]):
        assert beats(sp[a], a, sp[b], b)


@pytest.mark.parametrize("seed", range(6))
def test_bruteforce_group_case(seed):
    c = cfg(E=16, G=4, TG=2, k=4)
    rng = np.random.default_rng(seed)
    N = 40
    s = rng.uniform(0, 1, (N, c.E)).astype(np.float32)
    b = rng.uniform(-0.05, 0.05, c.E).astype(np.float32)
    idx, w, kept = oracle.select(c, s, b, want_kept=True)
    for n in range(N):
        S, K, sp = brute_force_selection(c, s[n], b)
        assert set(idx[n]) == S
        assert {g for g in range(c.G) if kept[n, g]} == K
        check_slot_order(idx[n], sp)


@pytest.mark.parametrize("E,G,TG,k", [(8, 2, 1, 2), (12, 3, 2, 3), (16, 4, 3, 5), (32, 8, 2, 4), (16, 8, 4, 3),
                                      (12, 1, 1, 3), (16, 4, 4, 4)])
def test_bruteforce_sweep(E, G, TG, k):
    c = cfg(E=E, G=G, TG=TG, k=k)
    rng = np.random.default_rng(E * 100 + G * 10 + k)
    N = 12
    s = rng.uniform(0, 1, (N, E)).astype(np.float32)
    b = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    idx, _ = oracle.select(c, s, b)
    for n in range(N):
        S, _, sp = brute_force_selection(c, s[n], b)
        assert set(idx[n]) == S
        check_slot_order(idx[n], sp)


@pytest.mark.parametrize("seed", range(4))
def test_bruteforce_tie_rich(seed):
    """Scores and bias on a 1/8 grid, so equal s' values and equal group scores are common."""
    c = cfg(E=16, G=4, TG=2, k=4)
    rng = np.random.default_rng(1000 + seed)
    N = 60
    s = (rng.integers(0, 8, (N, c.E)) / 8.0).astype(np.float32)
    b = (rng.integers(-1, 2, c.E) / 8.0).astype(np.float32)
    idx, _ = oracle.select(c, s, b)
    ties = 0
    for n in range(N):
        S, _, sp = brute_force_selection(c, s[n], b)
        ties += len(set(sp.tolist())) < c.E
        assert set(idx[n]) == S
        check_slot_order(idx[n], sp)
    assert ties > N // 2


def test_signed_zero_ties_go_to_lower_index():
    # s' = +0 and -0 compare equal, so the lower index wins.
    c = cfg(E=4, G=1, TG=1, k=1)
    s = np.array([[0.25, 0.25, 0.0, 0.0]], np.float32)
    b = np.array([-0.25, -0.5, -0.0, 0.0], np.float32)  # s' = [+0, -0.25, -0, +0]
    idx, _ = oracle.select(c, s, b)
    assert idx[0, 0] == 0


@pytest.mark.parametrize("E,k", [(16, 4), (128, 8), (160, 8)])
def test_single_group_is_plain_topk(E, k):
    """With one group the selection equals a plain sort by (s' desc, index asc) ('Group Router': G = 1)."""
    c = cfg(E=E, G=1, TG=1, k=k)
    rng = np.random.default_rng(E)
    s = rng.uniform(0, 1, (50, E)).astype(np.float32)
    b = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    idx, _ = oracle.select(c, s, b)
    sp = (s + b).astype(np.float32)
    for n in range(50):
        ref = sorted(range(E), key=lambda e: (-float(sp[n, e]), e))[:k]
        assert list(idx[n]) == ref


def test_all_groups_kept_is_noop():
    rng = np.random.default_rng(7)
    s = rng.uniform(0, 1, (30, 32)).astype(np.float32)
    b = rng.uniform(-0.05, 0.05, 32).astype(np.float32)
    a, wa = oracle.select(cfg(E=32, G=4, TG=4, k=6), s, b)
    g1, w1 = oracle.select(cfg(E=32, G=1, TG=1, k=6), s, b)
    assert np.array_equal(a, g1) and np.array_equal(wa, w1)


def test_discarded_groups_are_excluded_not_zeroed():
    """Reading of 'zero (or -inf) the other groups': excluded. With every s' negative a zero mask would pick
    discarded experts (0 > s'); the oracle keeps to the kept groups."""
    c = cfg(E=8, G=4, TG=1, k=2)
    s = np.full((1, 8), 0.01, np.float32)
    s[0, 2:4] = 0.02  # group 1 is the best group
    b = np.full(8, -0.04, np.float32)
    idx, w, kept = oracle.select(c, s, b, want_kept=True)
    assert list(kept[0]) == [0, 1, 0, 0]
    assert sorted(idx[0]) == [2, 3]


def test_worked_examples():
    for ex in json.load(open(os.path.join(GOLDEN, "router_worked_examples.json")))["examples"]:
        c = cfg(E=ex["E"], G=ex["G"], TG=ex["TG"], k=ex["k"], alpha=ex["alpha"], norm=ex["norm"])
        idx, w = oracle.select(c, np.array([ex["s"]], np.float32), np.array(ex["b"], np.float32))
        assert list(idx[0]) == ex["idx"], ex["name"]
        exact = np.array(ex["w_num"], np.float64) / ex["w_den"]
        # two float32 roundings (quotient, then alpha times it)
        assert np.all(np.abs(w[0] - exact) <= 2.5 * 2.0**-24 * exact), (ex["name"], w[0], exact)


@pytest.mark.parametrize("G,TG", [(1, 1), (4, 2)])
def test_invariants(G, TG):
    c = cfg(E=32, G=G, TG=TG, k=6, alpha=2.5)
    rng = np.random.default_rng(11)
    N = 500
    s = rng.uniform(0, 1, (N, 32)).astype(np.float32)
    b = rng.uniform(-0.05, 0.05, 32).astype(np.float32)
    idx, w, kept = oracle.select(c, s, b, want_kept=True)
    gs = 32 // G
    for n in range(N):
        assert len(set(idx[n])) == c.k  # exactly k distinct experts
        assert kept[n].sum() == (TG if G > 1 else 1)
        assert all(kept[n, e // gs] for e in idx[n])
    # Weights sum to alpha (norm_topk_prob): k float32 roundings at most.
    assert np.all(np.abs(w.astype(np.float64).sum(1) - c.alpha) <= c.k * c.alpha * 2.0**-23)
    # Weights are proportional to the raw scores of the chosen experts.
    chosen = np.take_along_axis(s, idx.astype(np.int64), 1).astype(np.float64)
    ratio = w / chosen
    assert np.allclose(ratio, ratio[:, :1], rtol=4e-7, atol=0)


def test_bias_changes_selection_never_weights():
    """'Module 02', section 2: b decides which experts fire; the weights come from s alone."""
    c = cfg(E=16, G=4, TG=2, k=4)
    rng = np.random.default_rng(5)
    N = 200
    s = rng.uniform(0, 1, (N, 16)).astype(np.float32)
    b = rng.uniform(-0.05, 0.05, 16).astype(np.float32)
    idx, w = oracle.select(c, s, b)
    # (1) a tiny bias perturbation that keeps each token's selection leaves its weights bit-identical
    b2 = (b + rng.uniform(-1e-7, 1e-7, 16)).astype(np.float32)
    idx2, w2 = oracle.select(c, s, b2)
    same = np.all(idx == idx2, axis=1)
    assert same.sum() > N * 0.9
    assert np.array_equal(w[same], w2[same])
    # (2) inputs where s and s + b select differently: the set follows s + b, the weights follow s
    s1 = np.array([[0.9, 0.8, 0.3, 0.2, 0.5, 0.4, 0.1, 0.05]], np.float32)
    b1 = np.array([-0.7, -0.7, 0.0, 0.0, 0.0, 0.0, 0.0, 0.0], np.float32)
    c1 = cfg(E=8, G=1, TG=1, k=2)
    i_b, w_b = oracle.select(c1, s1, b1)
    i_0, w_0 = oracle.select(c1, s1, np.zeros(8, np.float32))
    assert set(i_0[0]) == {0, 1} and set(i_b[0]) == {4, 5}
    assert np.allclose(w_b[0], c1.alpha * np.array([0.5, 0.4]) / 0.9, rtol=1e-6)
    sp = s1[0] + b1
    assert not np.allclose(w_b[0], c1.alpha * sp[[4, 5]] / sp[[4, 5]].sum(), rtol=1e-3) or np.allclose(
        sp[[4, 5]], s1[0, [4, 5]])


def test_equal_scores_closed_form():
    """All scores equal and no bias: the lowest-index experts of the lowest-index groups are chosen and every
    weight is alpha / k exactly (W_g = 0 gives s = 1/2 everywhere)."""
    for G, TG, expect in [(1, 1, [0, 1, 2, 3]), (4, 2, [0, 1, 2, 3]), (8, 4, [0, 1, 2, 3])]:
        c = cfg(E=32, G=G, TG=TG, k=4, alpha=2.5)
        s = np.full((3, 32), 0.5, np.float32)
        idx, w = oracle.select(c, s, np.zeros(32, np.float32))
        assert np.all(idx == expect)
        assert np.all(w == np.float32(2.5 / 4))
    # groups of 4, keep 2, k = 6: experts 0..5 (group 0 whole, then group 1's first two)
    c = cfg(E=16, G=4, TG=2, k=6)
    idx, w = oracle.select(c, np.full((1, 16), 0.5, np.float32), np.zeros(16, np.float32))
    assert list(idx[0]) == [0, 1, 2, 3, 4, 5]


def test_eps_guard():
    """eps keeps an all-zero chosen set finite: w = 0, not NaN. With tiny scores eps dominates."""
    c = cfg(E=8, G=1, TG=1, k=2)
    s = np.zeros((1, 8), np.float32)
    idx, w = oracle.select(c, s, np.zeros(8, np.float32))
    assert np.all(w == 0.0) and not np.any(np.isnan(w))
    s2 = np.full((1, 8), 1e-30, np.float32)
    _, w2 = oracle.select(c, s2, np.zeros(8, np.float32))
    exact = 2.5 * 1e-30 / (2e-30 + 1e-20)
    assert np.allclose(w2[0], exact, rtol=1e-5)
    c0 = cfg(E=8, G=1, TG=1, k=2, eps=0.0)
    _, w0 = oracle.select(c0, s, np.zeros(8, np.float32))
    assert np.all(np.isnan(w0))  # the guard is what eps is there for


def test_norm_false_is_alpha_times_s():
    c = cfg(E=16, G=4, TG=2, k=4, norm=False, alpha=2.5)
    rng = np.random.default_rng(3)
    s = rng.uniform(0, 1, (20, 16)).astype(np.float32)
    idx, w = oracle.select(c, s, np.zeros(16, np.float32))
    chosen = np.take_along_axis(s, idx.astype(np.int64), 1)
    assert np.array_equal(w, (np.float32(2.5) * chosen).astype(np.float32))


def test_invalid_configs_rejected():
    for bad in [cfg(E=10, G=3, TG=1, k=1), cfg(E=8, G=8, TG=2, k=1), cfg(E=8, G=2, TG=3, k=1),
                cfg(E=8, G=2, TG=1, k=5), cfg(E=8, G=1, TG=1, k=0)]:
        assert not oracle.check_cfg(bad)
    assert oracle.check_cfg(cfg(E=8, G=2, TG=1, k=4))


def test_margin_detects_ties():
    c = cfg(E=8, G=1, TG=1, k=2)
    s = np.array([[0.9, 0.5, 0.5, 0.1, 0.2, 0.3, 0.0, 0.0],
                  [0.9, 0.7, 0.5, 0.1, 0.2, 0.3, 0.0, 0.0]], np.float32)
    m = oracle.select_margin(c, s, np.zeros(8, np.float32))
    assert m[0] == 0.0
    assert abs(m[1] - 0.2) < 1e-6


def test_margin_golden_cases():
    """Hand-derived cases (tests/golden/select_margin_cases.json) in which the group branch of the margin
    (weakest kept group against the best discarded one) or the expert branch decides, with ties and a
    bias that changes the group ranking."""
    with open(os.path.join(GOLDEN, "select_margin_cases.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        c = cfg(E=case["E"], G=case["G"], TG=case["TG"], k=case["k"])
        s = np.array([case["s"]], np.float32)
        b = np.array(case["b"], np.float32)
        idx, _ = oracle.select(c, s, b)
        m = oracle.select_margin(c, s, b)
        assert idx[0].tolist() == case["idx"], case["name"]
        assert m[0] == case["margin"], (case["name"], m[0])


def brute_force_margin(c, s_row, b_row):
    """The decision margin from sorted lists: group scores as the largest pairwise sum inside each group,
    groups ranked by a sort on (score desc, index asc), the gap between the TG-th and (TG+1)-th; the
    eligible experts' s' sorted descending, the gaps between consecutive values among the k + 1 best."""
    sp = (s_row.astype(np.float32) + b_row.astype(np.float32)).astype(np.float32)
    gs = c.E // c.G
    gaps = []
    kept = set(range(c.G))
    if c.G > 1 and c.TG < c.G:
        gscore = [max(np.float32(sp[i] + sp[j]) for i in range(g * gs, (g + 1) * gs)
                      for j in range(g * gs, (g + 1) * gs) if i != j) for g in range(c.G)]
        order = sorted(range(c.G), key=lambda g: (-float(gscore[g]), g))
        kept = set(order[:c.TG])
        gaps.append(float(gscore[order[c.TG - 1]]) - float(gscore[order[c.TG]]))
    vals = sorted((float(sp[e]) for e in range(c.E) if e // gs in kept), reverse=True)[:c.k + 1]
    gaps += [a - b for a, b in zip(vals[:-1], vals[1:])]
    return min(gaps)


@pytest.mark.parametrize("E,G,TG,k,grid", [(16, 4, 2, 4, False), (16, 4, 2, 4, True), (12, 3, 2, 3, False),
                                           (32, 8, 3, 5, True), (24, 6, 5, 6, False), (12, 1, 1, 3, False),
                                           (16, 8, 4, 3, True)])
def test_margin_matches_sorted_definition(E, G, TG, k, grid):
    c = cfg(E=E, G=G, TG=TG, k=k)
    rng = np.random.default_rng(E * 7 + G * 3 + k + grid)
    N = 60
    if grid:
        s = (rng.integers(0, 17, (N, E)) / 16.0).astype(np.float32)
        b = (rng.integers(-2, 3, E) / 16.0).astype(np.float32)
    else:
        s = rng.uniform(0, 1, (N, E)).astype(np.float32)
        b = rng.uniform(-0.05, 0.05, E).astype(np.float32)
    m = oracle.select_margin(c, s, b)
    for n in range(N):
        assert m[n] == brute_force_margin(c, s[n], b), n


def test_margin_is_robustness_radius():
    """Perturbing every score by less than a quarter of the token's margin (a group score sums two s')
    leaves the chosen experts and their slot order unchanged."""
    c = cfg(E=16, G=4, TG=2, k=4)
    rng = np.random.default_rng(5)
    N = 400
    s = rng.uniform(0, 1, (N, c.E)).astype(np.float32)
    b = rng.uniform(-0.05, 0.05, c.E).astype(np.float32)
    m = oracle.select_margin(c, s, b)
    idx, _ = oracle.select(c, s, b)
    for trial in range(5):
        delta = rng.uniform(-1, 1, s.shape) * (0.24 * m)[:, None]
        idx2, _ = oracle.select(c, (s + delta).astype(np.float32), b)
        assert np.array_equal(idx, idx2)
