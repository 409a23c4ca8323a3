"""Pins for the oracle's layer variants, independent of the oracle's own formulas.

Sources:
- page "Module 02 -- MoE: Capacity, Work, and Traffic", section 3: every expert, routed or shared, caps
  its gate projection from above at 10 (no lower bound) and clips its up projection to [-10, 10]
  before SiLU(gate) * up;
- page "MoE Forward" (GLM-4.5), Official code: some kernels apply alpha on the routed output instead of
  inside the router, never both -- the two placements give the same layer;
- page "GLM-5 . Mixture of experts": the expert loop skips the id E (one past the last expert), so a
  slot holding E contributes nothing.
"""
from types import SimpleNamespace

import numpy as np
import pytest

import oracle


def cfg(E=8, G=1, TG=1, k=2, D=16, d=8, n_shared=1, alpha=2.5, norm=True, limit=0.0, alpha_on_output=False):
    return SimpleNamespace(D=D, E=E, G=G, TG=TG, k=k, d=d, n_shared=n_shared, alpha=alpha, norm=norm, eps=1e-20,
                           limit=limit, alpha_on_output=alpha_on_output)


def act(g, u, limit):
    """The oracle's one-column SwiGLU: gate = [[g]], up = [[u]], down = [[1]], x = [1]."""
    one = np.ones((1, 1), np.float32)
    return float(oracle.swiglu(np.array([[g]], np.float32), np.array([[u]], np.float32), one, [1.0], limit)[0])


# ---- clamped SwiGLU ------------------------------------------------------------------------------

def test_clamp_gate_saturates_above_only():
    L = 10.0
    for u in (3.0, -7.5, 10.0):
        at = act(L, u, L)
        assert act(10.5, u, L) == at and act(1000.0, u, L) == at and act(1e30, u, L) == at
        # below the bound the gate is untouched, however negative (a symmetric clamp would change these)
        for g in (9.99, 0.3, -10.0, -10.5, -50.0):
            assert act(g, u, L) == act(g, u, 0.0)
        assert act(-50.0, u, L) != act(-10.0, u, L)


def test_clamp_up_clips_both_sides():
    L = 10.0
    for g in (2.0, -1.0, 12.0):
        assert act(g, 12.0, L) == act(g, 10.0, L) == act(g, 1e6, L)
        assert act(g, -12.0, L) == act(g, -10.0, L) == act(g, -1e6, L)
        for u in (0.5, 7.0, 10.0):
            assert act(g, -u, L) == -act(g, u, L)  # odd in u
            assert act(g, u, L) == act(g, u, 0.0) if g <= L else True
    # the clip happens before the product: SiLU(2) * 10, not a clip of the product
    assert act(2.0, 12.0, L) == pytest.approx(2.0 / (1.0 + np.exp(-2.0)) * 10.0, rel=1e-15)
    assert abs(act(2.0, 12.0, 0.0)) > abs(act(2.0, 12.0, L))


def test_clamp_zero_bound_is_plain_swiglu():
    rng = np.random.default_rng(0)
    D, dff = 24, 10
    g, u = rng.normal(size=(dff, D)).astype(np.float32), rng.normal(size=(dff, D)).astype(np.float32)
    dn = rng.normal(size=(D, dff)).astype(np.float32)
    x = 30.0 * rng.normal(size=D)  # large projections, so a bound would bite
    plain = oracle.swiglu(g, u, dn, x)
    assert np.array_equal(oracle.swiglu(g, u, dn, x, 0.0), plain)
    assert not np.allclose(oracle.swiglu(g, u, dn, x, 10.0), plain)


def test_clamped_layer_uses_clamp_in_routed_and_shared_experts():
    """forward_tokens with limit > 0 equals the sum of clamped single-expert MLPs (routed + shared)."""
    c = cfg(E=6, k=2, D=32, d=16, limit=10.0)
    rng = np.random.default_rng(1)
    N = 5
    x = (40.0 * rng.normal(size=(N, c.D))).astype(np.float32)
    gu = (rng.normal(size=(c.E, 2 * c.d, c.D)) / np.sqrt(c.D)).astype(np.float32)
    dn = (rng.normal(size=(c.E, c.D, c.d)) / np.sqrt(c.d)).astype(np.float32)
    sh = tuple((rng.normal(size=s) / np.sqrt(c.D)).astype(np.float32)
               for s in ((c.d, c.D), (c.d, c.D), (c.D, c.d)))
    idx = np.stack([rng.choice(c.E, c.k, replace=False) for _ in range(N)]).astype(np.int32)
    w = rng.uniform(0.1, 1.0, (N, c.k)).astype(np.float32)
    table = oracle.ExpertTable(c, (gu, dn), sh)
    y = oracle.forward_tokens(c, np.arange(N), x, table, idx, w)
    y_loop = oracle.forward_expert_loop(c, x, table, idx, w)
    for n in range(N):
        xd = x[n].astype(np.float64)
        ref = oracle.swiglu(*sh, xd, 10.0)
        for s in range(c.k):
            e = idx[n, s]
            ref = ref + float(w[n, s]) * oracle.swiglu(gu[e, :c.d], gu[e, c.d:], dn[e], xd, 10.0)
        assert np.allclose(y[n], ref, rtol=1e-6, atol=1e-6)
    assert np.allclose(y, y_loop, rtol=1e-6, atol=1e-6)
    # the bound matters on these inputs: the plain layer differs
    y_plain = oracle.forward_tokens(cfg(E=6, k=2, D=32, d=16), np.arange(N), x, table, idx, w)
    assert not np.allclose(y, y_plain, rtol=1e-3)


# ---- alpha placement -----------------------------------------------------------------------------

def test_alpha_on_output_weights_carry_no_alpha():
    c_in, c_out = cfg(E=16, k=4, alpha=2.5), cfg(E=16, k=4, alpha=2.5, alpha_on_output=True)
    rng = np.random.default_rng(2)
    s = rng.uniform(0.01, 0.99, (50, 16)).astype(np.float32)
    b = rng.uniform(-0.05, 0.05, 16).astype(np.float32)
    i_in, w_in = oracle.select(c_in, s, b)
    i_out, w_out = oracle.select(c_out, s, b)
    assert np.array_equal(i_in, i_out)  # selection does not depend on where alpha goes
    assert np.allclose(w_out.sum(axis=1), 1.0, rtol=1e-6)
    assert np.allclose(w_in, 2.5 * w_out, rtol=1e-6)


def test_alpha_placements_give_the_same_layer():
    rng = np.random.default_rng(3)
    for n_shared in (0, 1):
        c_in = cfg(E=8, k=3, D=32, d=16, n_shared=n_shared, alpha=2.5)
        c_out = cfg(E=8, k=3, D=32, d=16, n_shared=n_shared, alpha=2.5, alpha_on_output=True)
        N = 7
        x = rng.normal(size=(N, c_in.D)).astype(np.float32)
        wg = (rng.normal(size=(c_in.E, c_in.D)) / np.sqrt(c_in.D)).astype(np.float32)
        b = rng.uniform(-0.05, 0.05, c_in.E).astype(np.float32)
        gu = (rng.normal(size=(c_in.E, 2 * c_in.d, c_in.D)) / np.sqrt(c_in.D)).astype(np.float32)
        dn = (rng.normal(size=(c_in.E, c_in.D, c_in.d)) / np.sqrt(c_in.d)).astype(np.float32)
        sh = None
        if n_shared:
            sh = tuple((rng.normal(size=s) / np.sqrt(c_in.D)).astype(np.float32)
                       for s in ((c_in.d, c_in.D), (c_in.d, c_in.D), (c_in.D, c_in.d)))
        y_in = oracle.forward(c_in, x, wg, b, (gu, dn), sh)[0]
        y_out, _, _, w_out = oracle.forward(c_out, x, wg, b, (gu, dn), sh)
        assert np.allclose(y_in, y_out, rtol=1e-6, atol=1e-7)
        # "never both": alpha applied twice would scale the routed part by alpha^2
        table = oracle.ExpertTable(c_in, (gu, dn), sh)
        _, i_in, w_in = oracle.route(c_in, x, wg, b)
        y_twice = oracle.forward_tokens(c_out, np.arange(N), x, table, i_in, w_in)
        assert not np.allclose(y_twice, y_in, rtol=1e-3)


# ---- empty slots (id E) --------------------------------------------------------------------------

def test_empty_slot_contributes_nothing():
    c = cfg(E=6, k=3, D=16, d=8)
    rng = np.random.default_rng(4)
    N = 9
    x = rng.normal(size=(N, c.D)).astype(np.float32)
    gu = rng.normal(size=(c.E, 2 * c.d, c.D)).astype(np.float32)
    dn = rng.normal(size=(c.E, c.D, c.d)).astype(np.float32)
    sh = tuple(rng.normal(size=s).astype(np.float32) for s in ((c.d, c.D), (c.d, c.D), (c.D, c.d)))
    idx = np.stack([rng.choice(c.E, c.k, replace=False) for _ in range(N)]).astype(np.int32)
    w = rng.uniform(0.1, 1.0, (N, c.k)).astype(np.float32)
    empty = rng.random((N, c.k)) < 0.3
    empty[0] = True  # a token with every slot empty: only the shared expert remains
    idx_e = np.where(empty, c.E, idx).astype(np.int32)
    w_zero = np.where(empty, 0.0, w).astype(np.float32)
    table = oracle.ExpertTable(c, (gu, dn), sh)
    y_e = oracle.forward_tokens(c, np.arange(N), x, table, idx_e, w)
    y_z = oracle.forward_tokens(c, np.arange(N), x, table, idx, w_zero)
    assert np.allclose(y_e, y_z, rtol=1e-6, atol=1e-6)
    assert np.array_equal(y_e[0], oracle.swiglu(*sh, x[0].astype(np.float64)).astype(np.float32))
    assert np.allclose(oracle.forward_expert_loop(c, x, table, idx_e, w), y_e, rtol=1e-6, atol=1e-6)
    counts, offsets, sp, inv = oracle.dispatch(c, idx_e)
    flat = idx_e.ravel()
    assert np.array_equal(counts, np.bincount(flat[flat < c.E], minlength=c.E))
    assert offsets[-1] == int((~empty).sum())
    assert np.all(inv[empty.ravel()] == -1)
    live = np.flatnonzero(~empty.ravel())
    assert np.array_equal(sp[:offsets[-1]], live[np.argsort(flat[live], kind="stable")])
