"""GPU parity of the layer variants against the oracle, through the C ABI.

- Clamped SwiGLU ("Module 02 -- MoE: Capacity, Work, and Traffic", section 3): layers with bound 10 on
  inputs whose outlier tokens (x times 32) push the gate and up projections far past the bound, on both
  the decode (16-row tiles) and prefill kernels, float32 and bfloat16, plus the 288-expert decode shape.
- alpha on the routed output ("MoE Forward", Official code): the weights carry no alpha and the layer is
  the same.
- Routing given by the caller with empty slots (id E, "GLM-5 . Mixture of experts"): moe_forward_routed
  against the oracle on that routing, and against moe_forward on the GPU's own routing (bit for bit).
Tolerances and the routing protocol are those of test_gpu_forward.
"""
from dataclasses import replace

import numpy as np
import pytest

import oracle
import synth
from tests import _harness as H

pytestmark = pytest.mark.gpu

BASE = synth.WORKLOADS["tiny_fp32"]

CLAMP = [
    # 16-row (decode) tiles, a group stage, 2 shared experts
    dict(N=21, D=256, E=32, G=8, TG=3, k=6, d=128, n_shared=2),
    # 256-row prefill tiles with few rows per expert (150 on average) and column tails
    dict(N=600, D=320, E=16, G=4, TG=2, k=4, d=192, n_shared=1),
    # 256-row prefill tiles
    dict(N=1500, D=256, E=8, G=1, TG=1, k=2, d=128, n_shared=1),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", CLAMP, ids=lambda c: f"N{c['N']}-E{c['E']}-k{c['k']}")
def test_clamped_swiglu(case, dtype):
    w = replace(BASE, name="clamp", dtype=dtype, seed=7, limit=10.0, outlier_every=3, **case)
    print(f"[clamp] {case} {dtype}", flush=True)
    wg, b, dev = H.device_weights(w, generate_on_device=False)
    x = synth.x_host(w)
    y, idx, wt, counts = H.gpu_forward(w, H.to_device(x), dev)
    H.check_forward(w, x, wg, b, y, idx, wt, counts, np.arange(w.N))
    # the bound bites on these inputs: the plain layer is far from the clamped one on the outlier tokens
    plain = replace(w, limit=0.0)
    tok = np.arange(0, w.N, w.outlier_every)
    table = H.expert_table(w, idx[tok].ravel())
    y_plain = oracle.forward_tokens(plain, tok, x, table, idx, wt)
    assert H.rel_err(H.as_f32(y[tok]), y_plain) > 0.1


def test_clamped_swiglu_288_expert_decode():
    w = replace(synth.WORKLOADS["glm53_flash_decode"], outlier_every=4)
    print(f"[clamp] {w.name} with outliers", flush=True)
    wg, b, dev = H.device_weights(w, generate_on_device=True)
    x = synth.x_host(w)
    y, idx, wt, counts = H.gpu_forward(w, H.to_device(x), dev)
    H.check_forward(w, x, wg, b, y, idx, wt, counts, np.arange(w.N))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("N", [37, 900])
def test_alpha_on_output(N, dtype):
    w = replace(BASE, name="alpha_out", dtype=dtype, seed=8, N=N, D=256, E=16, G=4, TG=2, k=4, d=128, alpha=2.5,
                alpha_on_output=True)
    print(f"[alpha_out] N={N} {dtype}", flush=True)
    wg, b, dev = H.device_weights(w, generate_on_device=False)
    x = synth.x_host(w)
    y, idx, wt, counts = H.gpu_forward(w, H.to_device(x), dev)
    assert np.allclose(wt.sum(axis=1), 1.0, rtol=1e-5)  # no alpha in the weights
    H.check_forward(w, x, wg, b, y, idx, wt, counts, np.arange(w.N))
    # the same layer as alpha inside the weights
    y_in, _, _, _ = H.gpu_forward(replace(w, alpha_on_output=False), H.to_device(x), dev)
    assert H.rel_err(H.as_f32(y), H.as_f32(y_in)) <= H.TOL[dtype]


ROUTED = [
    dict(N=45, D=256, E=16, G=1, TG=1, k=4, d=128, n_shared=1),
    dict(N=700, D=320, E=12, G=1, TG=1, k=3, d=192, n_shared=0),
    dict(N=1200, D=256, E=8, G=1, TG=1, k=2, d=128, n_shared=1),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", ROUTED, ids=lambda c: f"N{c['N']}-E{c['E']}-k{c['k']}")
def test_forward_routed_with_empty_slots(case, dtype):
    w = replace(BASE, name="routed", dtype=dtype, seed=9, **case)
    print(f"[routed] {case} {dtype}", flush=True)
    wg, b, dev = H.device_weights(w, generate_on_device=False)
    x = synth.x_host(w)
    rng = np.random.default_rng(11)
    idx = np.stack([rng.choice(w.E, w.k, replace=False) for _ in range(w.N)]).astype(np.int32)
    wt = rng.uniform(0.05, 1.5, (w.N, w.k)).astype(np.float32)
    empty = rng.random((w.N, w.k)) < 0.25
    empty[0] = True  # one token with every slot empty
    idx[empty] = w.E
    y, counts = H.gpu_forward_routed(w, H.to_device(x), dev, idx, wt)
    flat = idx.ravel()
    assert np.array_equal(counts, np.bincount(flat[flat < w.E], minlength=w.E))
    table = H.expert_table(w, flat[flat < w.E])
    y_ref = oracle.forward_tokens(w, np.arange(w.N), x, table, idx, wt)
    err = H.rel_err(H.as_f32(y), y_ref)
    print(f"  rel_err={err:.3g}", flush=True)
    assert err <= H.TOL[dtype]


def test_forward_routed_matches_forward_bitwise():
    """Fed the GPU's own routing, moe_forward_routed reproduces moe_forward bit for bit."""
    w = replace(BASE, name="routed_eq", dtype="bf16", seed=10, N=500, D=256, E=16, G=4, TG=2, k=4, d=128)
    _, _, dev = H.device_weights(w, generate_on_device=False)
    x = synth.x_host(w)
    xd = H.to_device(x)
    y, idx, wt, counts = H.gpu_forward(w, xd, dev)
    y2, counts2 = H.gpu_forward_routed(w, xd, dev, idx, wt)
    assert np.array_equal(y, y2) and np.array_equal(counts, counts2)
