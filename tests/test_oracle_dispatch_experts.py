"""Pins for the oracle's dispatch, SwiGLU experts and combine, independent of the oracle.

Sources: page "MoE Forward" (GLM-4.5), How it works (eq. E_i, the packed gate_up layout, eq. y_n, alpha
scaling only the routed sum, token-choice dispatch); page "GLM-5 . Mixture of experts" (the loop over
experts with index_add into the output); page "Shared output" (bias-free SwiGLU MLP).
"""
from types import SimpleNamespace

import numpy as np
import pytest

import oracle
import synth


def cfg(E=8, G=1, TG=1, k=2, D=16, d=8, n_shared=1, alpha=2.5, norm=True):
    return SimpleNamespace(D=D, E=E, G=G, TG=TG, k=k, d=d, n_shared=n_shared, alpha=alpha, norm=norm, eps=1e-20)


def silu_tanh(z):
    """SiLU through the identity sigma(z) = (1 + tanh(z / 2)) / 2 -- a different evaluation route."""
    return z * 0.5 * (1.0 + np.tanh(0.5 * z))


def random_routing(c, N, rng):
    idx = np.stack([rng.choice(c.E, c.k, replace=False) for _ in range(N)]).astype(np.int32)
    w = rng.uniform(0.05, 1.0, (N, c.k)).astype(np.float32)
    return idx, w


def test_dispatch_invariants():
    c = cfg(E=16, k=4)
    rng = np.random.default_rng(0)
    N = 300
    idx, _ = random_routing(c, N, rng)
    counts, offsets, sp, inv = oracle.dispatch(c, idx)
    assert np.array_equal(counts, np.bincount(idx.ravel(), minlength=c.E))
    assert offsets[0] == 0 and offsets[-1] == N * c.k and np.all(np.diff(offsets) == counts)
    assert np.array_equal(np.sort(sp), np.arange(N * c.k))  # each (n, slot) exactly once
    assert np.array_equal(sp[inv], np.arange(N * c.k))  # inverse maps
    flat = idx.ravel()
    for e in range(c.E):
        seg = sp[offsets[e]:offsets[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg // c.k) > 0)  # tokens ascending inside each expert
    # a numpy stable sort by expert gives the same permutation
    assert np.array_equal(sp, np.argsort(flat, kind="stable"))


def test_dispatch_rejects_out_of_range():
    """Ids outside [0, E] are invalid (E itself is the empty slot, covered in test_oracle_variants)."""
    c = cfg(E=4, k=2)
    for bad in (5, -1):
        with pytest.raises(ValueError):
            oracle.dispatch(c, np.array([[0, bad]], np.int32))


def test_swiglu_identity_closed_form():
    """gate = up = I and down a permutation: out = P (SiLU(x) * x), which pins each matrix's orientation."""
    D = 12
    rng = np.random.default_rng(1)
    x = rng.normal(size=D)
    eye = np.eye(D, dtype=np.float32)
    perm = rng.permutation(D)
    P = eye[perm]  # (P v)[i] = v[perm[i]]
    out = oracle.swiglu(eye, eye, P, x)
    assert np.allclose(out, (silu_tanh(x) * x)[perm], rtol=1e-14, atol=1e-15)
    # gate and up play different roles: gate = I, up = 2I gives 2 SiLU(x) x, gate = 2I, up = I gives SiLU(2x) x
    assert np.allclose(oracle.swiglu(eye, 2 * eye, eye, x), 2 * silu_tanh(x) * x, rtol=1e-14)
    assert np.allclose(oracle.swiglu(2 * eye, eye, eye, x), silu_tanh(2 * x) * x, rtol=1e-14)


def test_swiglu_rectangular_against_numpy():
    """A rectangular MLP against numpy float64 matmuls (library routine) and the tanh form of SiLU."""
    rng = np.random.default_rng(2)
    D, dff = 24, 40
    g = rng.normal(size=(dff, D)).astype(np.float32)
    u = rng.normal(size=(dff, D)).astype(np.float32)
    dn = rng.normal(size=(D, dff)).astype(np.float32)
    x = rng.normal(size=D)
    ref = dn.astype(np.float64) @ (silu_tanh(g.astype(np.float64) @ x) * (u.astype(np.float64) @ x))
    assert np.allclose(oracle.swiglu(g, u, dn, x), ref, rtol=1e-12, atol=1e-12)
    # bf16 weights are widened exactly
    gb, ub, db = synth.f32_to_bf16(g), synth.f32_to_bf16(u), synth.f32_to_bf16(dn)
    gw, uw, dw = (synth.bf16_to_f32(a).astype(np.float64) for a in (gb, ub, db))
    refb = dw @ (silu_tanh(gw @ x) * (uw @ x))
    assert np.allclose(oracle.swiglu(gb, ub, db, x), refb, rtol=1e-12, atol=1e-12)


def make_layer(c, rng, dtype=np.float32):
    gu = rng.normal(0, c.D ** -0.5, (c.E, 2 * c.d, c.D)).astype(np.float32)
    dn = rng.normal(0, c.d ** -0.5, (c.E, c.D, c.d)).astype(np.float32)
    dsh = c.d * c.n_shared
    sh = (rng.normal(0, c.D ** -0.5, (dsh, c.D)).astype(np.float32),
          rng.normal(0, c.D ** -0.5, (dsh, c.D)).astype(np.float32),
          rng.normal(0, dsh ** -0.5, (c.D, dsh)).astype(np.float32))
    return gu, dn, sh


def test_packed_gate_up_split():
    """Rows [0, d) of gate_up are the gate, rows [d, 2d) the up projection ('MoE Forward', packed layout)."""
    c = cfg(E=3, k=1, D=16, d=8)
    rng = np.random.default_rng(3)
    gu, dn, sh = make_layer(c, rng)
    x = rng.normal(size=(4, c.D)).astype(np.float32)
    idx = np.array([[0], [1], [2], [1]], np.int32)
    w = np.ones((4, 1), np.float32)
    c0 = cfg(E=3, k=1, D=16, d=8, n_shared=0)
    y = oracle.forward_tokens(c0, np.arange(4), x, oracle.ExpertTable(c0, (gu, dn), None), idx, w)
    for n in range(4):
        e = idx[n, 0]
        ref = oracle.swiglu(gu[e, :c.d], gu[e, c.d:], dn[e], x[n].astype(np.float64))
        assert np.array_equal(y[n], ref.astype(np.float32))


def test_identical_experts_closed_form():
    """All routed experts equal: y = alpha E(x) + E_sh(x) whatever the routing (weights sum to alpha).
    Pins the combine, alpha applied once, and the unscaled shared expert ('MoE Forward', two facts #1)."""
    c = cfg(E=8, k=3, D=16, d=8, alpha=2.5)
    rng = np.random.default_rng(4)
    gu1, dn1, sh = make_layer(SimpleNamespace(**{**vars(c), "E": 1}), rng)
    gu = np.repeat(gu1, c.E, 0)
    dn = np.repeat(dn1, c.E, 0)
    N = 20
    x = rng.normal(size=(N, c.D)).astype(np.float32)
    wg = rng.normal(size=(c.E, c.D)).astype(np.float32)
    b = rng.uniform(-0.05, 0.05, c.E).astype(np.float32)
    y, s, idx, w = oracle.forward(c, x, wg, b, (gu, dn), sh)
    for n in range(N):
        xd = x[n].astype(np.float64)
        ref = float(w[n].astype(np.float64).sum()) * oracle.swiglu(gu1[0, :c.d], gu1[0, c.d:], dn1[0], xd) + \
            oracle.swiglu(*sh, xd)
        assert np.allclose(y[n], ref, rtol=1e-6, atol=1e-6)
        alpha_ref = c.alpha * oracle.swiglu(gu1[0, :c.d], gu1[0, c.d:], dn1[0], xd) + oracle.swiglu(*sh, xd)
        assert np.allclose(y[n], alpha_ref, rtol=2e-6, atol=2e-6)


def test_ablations():
    c = cfg(E=8, k=2, D=16, d=8)
    rng = np.random.default_rng(5)
    gu, dn, sh = make_layer(c, rng)
    N = 10
    x = rng.normal(size=(N, c.D)).astype(np.float32)
    idx, w = random_routing(c, N, rng)
    toks = np.arange(N)
    # zero routed down => y = E_sh(x)
    y = oracle.forward_tokens(c, toks, x, oracle.ExpertTable(c, (gu, np.zeros_like(dn)), sh), idx, w)
    for n in range(N):
        assert np.array_equal(y[n], oracle.swiglu(*sh, x[n].astype(np.float64)).astype(np.float32))
    # zero shared down => y = sum_slot w E(x)
    sh0 = (sh[0], sh[1], np.zeros_like(sh[2]))
    y = oracle.forward_tokens(c, toks, x, oracle.ExpertTable(c, (gu, dn), sh0), idx, w)
    c0 = cfg(E=8, k=2, D=16, d=8, n_shared=0)
    y0 = oracle.forward_tokens(c0, toks, x, oracle.ExpertTable(c0, (gu, dn), None), idx, w)
    assert np.array_equal(y, y0)
    for n in range(N):
        xd = x[n].astype(np.float64)
        ref = sum(float(w[n, j]) * oracle.swiglu(gu[e, :c.d], gu[e, c.d:], dn[e], xd) for j, e in enumerate(idx[n]))
        assert np.allclose(y[n], ref, rtol=1e-6, atol=1e-7)


def test_weight_linearity():
    """Doubling every routed weight doubles the routed part only."""
    c = cfg(E=8, k=2, D=16, d=8)
    rng = np.random.default_rng(6)
    gu, dn, sh = make_layer(c, rng)
    N = 8
    x = rng.normal(size=(N, c.D)).astype(np.float32)
    idx, w = random_routing(c, N, rng)
    t = oracle.ExpertTable(c, (gu, dn), sh)
    y1 = oracle.forward_tokens(c, np.arange(N), x, t, idx, w).astype(np.float64)
    y2 = oracle.forward_tokens(c, np.arange(N), x, t, idx, 2 * w).astype(np.float64)
    ysh = np.stack([oracle.swiglu(*sh, x[n].astype(np.float64)) for n in range(N)])
    assert np.allclose(y2 - ysh, 2 * (y1 - ysh), rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_loop_forms_agree(dtype):
    """The per-expert loop form equals the per-token sum within 2 float32 ulp (both accumulate in double)."""
    c = cfg(E=8, k=3, D=32, d=16, n_shared=2)
    rng = np.random.default_rng(7)
    gu, dn, sh = make_layer(c, rng)
    N = 40
    x = rng.normal(size=(N, c.D)).astype(np.float32)
    if dtype == "bf16":
        gu, dn, x = synth.f32_to_bf16(gu), synth.f32_to_bf16(dn), synth.f32_to_bf16(x)
        sh = tuple(synth.f32_to_bf16(a) for a in sh)
    idx, w = random_routing(c, N, rng)
    t = oracle.ExpertTable(c, (gu, dn), sh)
    y_tok = oracle.forward_tokens(c, np.arange(N), x, t, idx, w)
    y_exp = oracle.forward_expert_loop(c, x, t, idx, w)
    ulp = np.spacing(np.abs(y_tok))
    assert np.all(np.abs(y_tok - y_exp) <= 2 * ulp)


def test_forward_tokens_subset_matches_full():
    c = cfg(E=8, k=2, D=16, d=8)
    rng = np.random.default_rng(8)
    gu, dn, sh = make_layer(c, rng)
    N = 12
    x = rng.normal(size=(N, c.D)).astype(np.float32)
    idx, w = random_routing(c, N, rng)
    t = oracle.ExpertTable(c, (gu, dn), sh)
    full = oracle.forward_tokens(c, np.arange(N), x, t, idx, w)
    sub_tokens = np.array([11, 3, 5])
    needed = {int(e): (gu[e], dn[e]) for e in np.unique(idx[sub_tokens])}
    t2 = oracle.ExpertTable(c, needed, sh)
    sub = oracle.forward_tokens(c, sub_tokens, x, t2, idx, w)
    assert np.array_equal(sub, full[sub_tokens])
