"""The router score bound used by the GPU parity tests, checked from both sides on the CPU.

"Group Router" (GLM-4.5), How it works: the gate is a bias-free linear map evaluated in float32;
"Module 02 -- MoE: Capacity, Work, and Traffic", section 2: router logits in float32. The GPU tests accept
|s_gpu - s_oracle| up to tests/_harness.score_tolerance. That bound must
  - admit a genuine float32 gate: float32 accumulation of the exact products x * W_g in the order with
    the most roundings (one after every product) stays inside it, and
  - reject a bfloat16 gate: the same router with W_g rounded to bfloat16 (the first of the three pieces
    the device splits W_g into, used alone) falls outside it on every bfloat16 workload.
Neither side touches the HIP library.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import _harness as H

BF16_WORKLOADS = ["air_prefill", "glm45_prefill_skewed", "glm5_prefill", "glm45_prefill_mild_skew"]


def _inputs(name, tokens):
    w = synth.WORKLOADS[name].with_tokens(tokens)
    x = synth.x_host(w)
    wg, b = synth.router_host(w)
    return w, x, wg, b


@pytest.mark.parametrize("name", BF16_WORKLOADS)
def test_bf16_gate_fails_the_bound(name):
    w, x, wg, b = _inputs(name, 256)
    s_ref = oracle.scores(w, x, wg).astype(np.float64)
    hi = synth.bf16_to_f32(synth.f32_to_bf16(wg)).astype(np.float64)
    r = H.as_f32(x).astype(np.float64) @ hi.T
    with np.errstate(over="ignore"):
        s_bf16 = (1.0 / (1.0 + np.exp(-r))).astype(np.float32).astype(np.float64)
    tol = H.score_tolerance(w, x, wg)
    out = np.abs(s_bf16 - s_ref) > tol
    print(f"{name}: bf16 gate outside the bound on {out.mean():.1%} of scores, "
          f"max ratio {(np.abs(s_bf16 - s_ref) / tol).max():.0f}")
    assert out.any()
    assert out.mean() > 0.05  # not a few unlucky elements: most of the non-saturated scores


@pytest.mark.parametrize("name", BF16_WORKLOADS + ["tiny_fp32"])
def test_sequential_float32_gate_within_the_bound(name):
    """Float32 accumulation, rounding after each of the 3 D exact products (hi, mid and lo pieces in
    turn), through a float32 sigmoid: inside the bound on every score."""
    w, x, wg, b = _inputs(name, 12)
    xf = H.as_f32(x)
    hi = synth.bf16_to_f32(synth.f32_to_bf16(wg))
    rest = (wg - hi).astype(np.float32)
    mid = synth.bf16_to_f32(synth.f32_to_bf16(rest))
    lo = (rest - mid).astype(np.float32)
    assert np.array_equal(synth.bf16_to_f32(synth.f32_to_bf16(lo)), lo)  # three bf16 pieces hold W_g exactly
    s_ref = oracle.scores(w, x, wg).astype(np.float64)
    tol = H.score_tolerance(w, x, wg)
    worst = 0.0
    for n in range(w.N):
        prods = np.concatenate([xf[n][None, :].astype(np.float64) * p for p in (hi, mid, lo)], axis=1)
        r = np.add.accumulate(prods.astype(np.float32), axis=1, dtype=np.float32)[:, -1]
        with np.errstate(over="ignore"):
            s = (np.float32(1.0) / (np.float32(1.0) + np.exp(-r, dtype=np.float32))).astype(np.float64)
        ratio = np.abs(s - s_ref[n]) / tol[n]
        worst = max(worst, float(ratio.max()))
    print(f"{name}: sequential float32 gate at {worst:.3f} of the bound")
    assert worst <= 1.0
