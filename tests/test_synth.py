"""The seeded input generator: Philox4x32-10 known-answer vectors, slice consistency, moments.

Philox4x32-10 is the counter-based generator of Salmon, Moraes, Dror and Shaw ("Parallel random numbers:
as easy as 1, 2, 3", SC'11); the three vectors below are its published known-answer tests.
"""
import numpy as np
import pytest

import synth

KAT = [
    ((0x00000000, 0x00000000), (0x00000000, 0x00000000, 0x00000000, 0x00000000),
     (0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8)),
    ((0xffffffff, 0xffffffff), (0xffffffff, 0xffffffff, 0xffffffff, 0xffffffff),
     (0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd)),
    ((0xa4093822, 0x299f31d0), (0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344),
     (0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1)),
]


@pytest.mark.parametrize("key,ctr,out", KAT)
def test_philox_known_answers(key, ctr, out):
    assert tuple(synth.philox_block(key[0], key[1], ctr)) == out


def test_slices_are_consistent():
    full = synth.normal(0, 4, 0, 10000, 0.5, "bf16")
    part = synth.normal(0, 4, 1234, 777, 0.5, "bf16")
    assert np.array_equal(full[1234:1234 + 777], part)
    f64 = synth.normal(3, 2, 0, 5000, 1.0, "f64")
    f32 = synth.normal(3, 2, 0, 5000, 1.0, "f32")
    assert np.array_equal(f64.astype(np.float32), f32)
    assert np.array_equal(synth.f32_to_bf16(f32), synth.normal(3, 2, 0, 5000, 1.0, "bf16"))


def test_streams_differ_by_key():
    a = synth.normal(0, 1, 0, 1000, 1.0, "f64")
    b = synth.normal(0, 2, 0, 1000, 1.0, "f64")
    c = synth.normal(1, 1, 0, 1000, 1.0, "f64")
    assert abs(np.corrcoef(a, b)[0, 1]) < 0.1 and abs(np.corrcoef(a, c)[0, 1]) < 0.1


def test_normal_moments():
    z = synth.normal(0, 1, 0, 1 << 20, 1.0, "f64")
    assert abs(z.mean()) < 5e-3
    assert abs(z.std() - 1.0) < 5e-3
    kurt = ((z - z.mean()) ** 4).mean() / z.var() ** 2
    assert abs(kurt - (3.0 - 1.2 / 8)) < 0.02  # Irwin-Hall(8)
    assert np.abs(z).max() < 4.9


def test_uniform_range_and_bf16_rounding():
    u = synth.uniform_f32(0, 3, 0, 100000, -0.05, 0.05)
    assert u.min() >= -0.05 and u.max() <= 0.05 and abs(u.mean()) < 1e-3
    # round to nearest even on bf16 bits
    f = np.array([1.0, 1.00390625, 1.01171875, 1.0 + 2**-8 + 2**-20], np.float32)
    assert list(synth.f32_to_bf16(f)) == [0x3F80, 0x3F80, 0x3F82, 0x3F81]


def test_workload_shapes():
    w = synth.WORKLOADS["tiny_fp32"]
    x = synth.x_host(w)
    wg, b = synth.router_host(w)
    gu, dn = synth.expert_host(w, 3)
    assert x.shape == (64, 256) and x.dtype == np.float32
    assert wg.shape == (16, 256) and b.shape == (16,)
    assert gu.shape == (256, 256) and dn.shape == (256, 128)
    gua, dna = synth.all_experts_host(w)
    assert np.array_equal(gua[3], gu) and np.array_equal(dna[3], dn)
    ws = synth.WORKLOADS["glm45_prefill_skewed"]
    wg, _ = synth.router_host(ws)
    plain = synth.normal(ws.seed, synth.ID_WG, 0, ws.E * ws.D, ws.D ** -0.5, "f32").reshape(ws.E, ws.D)
    off = wg - plain
    assert np.allclose(off, off[:, :1], atol=1e-6)  # one offset per router row
    assert 0.2 < off[:, 0].std() < 0.8


def test_skew_workloads_saturation_and_load():
    """The two GLM-4.5 prefill recipes on their first 1,024 tokens: offsets of std 0.5 saturate a share of
    the sigmoid scores and pile the rows on a few experts; offsets of std 0.02 saturate none and still
    load the experts unevenly (largest well above the mean)."""
    import oracle

    for name, saturated, skewed in [("glm45_prefill_skewed", True, 6.0), ("glm45_prefill_mild_skew", False, 3.0)]:
        w = synth.WORKLOADS[name].with_tokens(1024)
        x = synth.x_host(w)
        wg, b = synth.router_host(w)
        s = oracle.scores(w, x, wg)
        sat = float(np.mean(s == np.float32(1.0)))
        idx, _ = oracle.select(w, s, b)
        load = np.bincount(idx.ravel(), minlength=w.E)
        assert (sat > 0.05) if saturated else (sat == 0.0), (name, sat)
        assert load.max() > skewed * load.mean(), (name, load.max(), load.mean())
