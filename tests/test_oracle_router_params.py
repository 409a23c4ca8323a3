"""Pins for the oracle's gate GEMM, sigmoid and parameter accounting.

Sources: page "Group Router" (GLM-4.5), eq. s = sigma(x W_g^T) (a bias-free fp32 linear map, then a
sigmoid); page "GLM-5 . Mixture of experts", 'Exact per-instance accounting' and 'In numbers'; page
"Module 02 -- MoE: Capacity, Work, and Traffic", section 4 (per-expert derivation).

The logits and the sigmoid have no printed worked values; beyond the definition they are pinned by a
library routine (numpy float64 matmul / scipy expit) and sanity cases, which the oracle header records as
"parity unpinned" beyond those.
"""
import json
import os
from types import SimpleNamespace

import numpy as np
import pytest
from scipy.special import expit

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def cfg(D, E, d=8, k=2, G=1, TG=1, n_shared=1):
    return SimpleNamespace(D=D, E=E, G=G, TG=TG, k=k, d=d, n_shared=n_shared, alpha=2.5, norm=True, eps=1e-20)


def test_logits_one_hot_rows():
    c = cfg(D=64, E=4)
    rng = np.random.default_rng(0)
    x = rng.normal(size=(10, 64)).astype(np.float32)
    wg = np.zeros((4, 64), np.float32)
    cols, scale = [3, 17, 40, 63], [1.0, -0.5, 3.0, 0.125]
    for e in range(4):
        wg[e, cols[e]] = scale[e]
    r = oracle.logits(c, x, wg)
    for e in range(4):
        assert np.array_equal(r[:, e], (np.float32(scale[e]) * x[:, cols[e]]).astype(np.float32))


@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_logits_against_float64_matmul(xdt):
    c = cfg(D=512, E=16)
    rng = np.random.default_rng(1)
    x = rng.normal(size=(33, 512)).astype(np.float32)
    wg = rng.normal(0, 512 ** -0.5, (16, 512)).astype(np.float32)
    if xdt == "bf16":
        xb = synth.f32_to_bf16(x)
        r = oracle.logits(c, xb, wg)
        x = synth.bf16_to_f32(xb)
    else:
        r = oracle.logits(c, x, wg)
    ref = x.astype(np.float64) @ wg.astype(np.float64).T
    # both are double dot products (different summation order); after one rounding: equal or 1 ulp apart
    assert np.all(np.abs(r.astype(np.float64) - ref) <= np.spacing(np.abs(ref).astype(np.float32)))


def test_sigmoid_sanity():
    r = np.array([0.0, 1.0, -1.0, 20.0, -20.0, 104.0, -104.0, -200.0, 200.0], np.float32)
    s = oracle.sigmoid(r)
    assert s[0] == 0.5
    assert np.all(s >= 0) and np.all(s <= 1)
    assert s[-2] == 0.0 and s[-1] == 1.0
    rng = np.random.default_rng(2)
    rr = rng.normal(0, 4, 10000).astype(np.float32)
    a, b = oracle.sigmoid(rr), oracle.sigmoid(-rr)
    # sigma(-r) = 1 - sigma(r) within one ulp of the larger
    assert np.all(np.abs(a.astype(np.float64) + b - 1.0) <= np.spacing(np.maximum(a, b)))
    ref = expit(rr.astype(np.float64)).astype(np.float32)
    assert np.all(np.abs(a - ref) <= np.spacing(ref))
    srt = np.sort(rr)
    assert np.all(np.diff(oracle.sigmoid(srt)) >= 0)  # monotone


def test_scores_are_sigmoid_not_softmax():
    c = cfg(D=8, E=4)
    x = np.zeros((1, 8), np.float32)
    s = oracle.scores(c, x, np.ones((4, 8), np.float32))
    assert np.all(s == 0.5)  # a softmax would give 1/4; scores need not sum to 1


def test_param_counts_printed():
    g = json.load(open(os.path.join(GOLDEN, "glm5_param_counts.json")))
    a = g["glm5"]
    sh = a["shape"]
    pc = oracle.param_count(cfg(D=sh["D"], E=sh["E"], d=sh["d"], k=sh["k"], G=sh["G"], TG=sh["TG"]))
    assert pc["router"] == a["router"]
    assert pc["expert"] == a["routed_expert"]
    assert pc["routed"] == a["routed_all"]
    assert pc["shared"] == a["shared"]
    assert pc["total"] == a["total"]
    assert pc["used_per_token"] == a["used_per_token"]
    assert pc["total"] * a["blocks"] == a["all_blocks"]
    assert sh["E"] * a["blocks"] == a["bias_values_all_blocks"]
    assert round(pc["total"] * 2 / 2**30, 1) == a["held_gib_bf16"]
    assert round(pc["used_per_token"] * 2 / 2**20) == a["used_mib_bf16"]
    assert round(100 * pc["used_per_token"] / pc["total"], 1) == 3.5
    m = g["module02_checkpoint"]
    sh = m["shape"]
    pc = oracle.param_count(cfg(D=sh["D"], E=sh["E"], d=sh["d"], k=sh["k"]))
    assert pc["expert"] == m["per_expert"]
    assert m["layers"] * sh["E"] == m["experts_total"]
    assert round(m["experts_total"] * pc["expert"] / 1e9, 1) == m["routed_total_billions_approx"]


def test_workloads_are_valid_configs():
    for name in synth.WORKLOAD_ORDER:
        assert oracle.check_cfg(synth.WORKLOADS[name]), name
