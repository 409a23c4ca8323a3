"""GPU parity of the dense SwiGLU FFN (moe_dense_forward through the C ABI) against the oracle's MLP.

The dense prefix FFN is the shared expert's bias-free SwiGLU MLP at the model's full intermediate width
("Shared output" (GLM-5), the evidence from the shared expert); the oracle evaluates it per token in
double (oracle_swiglu, pinned in test_oracle_dispatch_experts / test_oracle_variants). Tolerance: max|dy|
/ max|y| <= 1e-4 (float32) or <= 2e-2 (bfloat16), as for the MoE layer.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import _harness as H

pytestmark = pytest.mark.gpu


def _run(w, dev, x):
    import sparse_moe_layer_gate_amd as moe

    torch = H.torch_mod()
    xd = H.to_device(x)
    ws = torch.empty(max(moe.moe_dense_workspace_size(w.N, w.D, w.dff, w.dtype), 256), dtype=torch.uint8,
                     device="cuda")
    y = torch.empty_like(xd)
    moe.moe_dense_forward(w.N, xd, dev["gate"], dev["up"], dev["down"], y, ws, limit=w.limit)
    torch.cuda.synchronize()
    return H.to_host(y)


def _check(w, x, y, tokens, weights):
    g, u, dn = weights
    ref = np.stack([oracle.swiglu(g, u, dn, H.as_f32(x[n]).astype(np.float64), w.limit) for n in tokens])
    err = H.rel_err(H.as_f32(y[tokens]), ref)
    print(f"  {w.name} N={w.N} tokens={len(tokens)} rel_err={err:.3g}", flush=True)
    assert err <= H.TOL[w.dtype], err


CASES = [
    dict(N=1, D=256, dff=128), dict(N=3, D=320, dff=192),           # 16-row (decode) tiles
    dict(N=9, D=320, dff=192), dict(N=300, D=256, dff=384),         # 256-row tiles, ragged
    dict(N=1000, D=320, dff=192),
    dict(N=200, D=256, dff=256, limit=10.0, outlier_every=3),       # clamped, outlier tokens
]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_dense_small_whole(case, dtype):
    w = synth.DenseWorkload("dense_small", dtype=dtype, seed=12, **case)
    print(f"[dense] {case} {dtype}", flush=True)
    weights = synth.dense_host(w)
    dev = {"gate": H.to_device(weights[0]), "up": H.to_device(weights[1]), "down": H.to_device(weights[2])}
    x = synth.x_host(w)
    y = _run(w, dev, x)
    _check(w, x, y, np.arange(w.N), weights)


def test_dense_full_size_sampled():
    w = synth.DENSE_WORKLOADS["glm45_dense_ffn"]
    print(f"[dense] {w.name} N={w.N} D={w.D} dff={w.dff}", flush=True)
    H.drop_weights()
    dev = synth.dense_device(w)
    x = synth.x_host(w)
    y = _run(w, dev, x)
    tokens = H.sample_tokens(w.N, 12, seed=2)
    _check(w, x, y, tokens, synth.dense_host(w))
