"""Pins of the norm-ratio monitor oracle (oracle/monitor.py) against what the mathematics
fixes, independent of the oracle's own code: the identity at k = n, the Gaussian energy
fraction of the top 1%, the Pythagorean split between what is sent and the residual, an
exact special case of QSGD, the QSGD variance in expectation, and scale invariance."""
import math

import numpy as np
import pytest

import oracle

F32 = np.float32


def test_keep_everything_is_ratio_one():
    g = np.random.default_rng(1).standard_normal(10_001).astype(F32)
    (sc, sg, ratio), _, _ = oracle.monitored_step(g, np.zeros_like(g), g.size)
    assert sc == sg and ratio == 1.0
    (sc, sg, ratio), _, _ = oracle.monitored_step(g, np.zeros_like(g), 0)
    assert sg == 0.0 and ratio == 0.0 and sc > 0
    z = np.zeros(100, F32)
    assert oracle.monitored_step(z, z, 10)[0] == (0.0, 0.0, 1.0)


def test_top1pct_of_gaussian_energy_fraction():
    # for X ~ N(0,1) and t with P(|X| > t) = 1%, E[X^2; |X| > t] = 2 (t phi(t) + 0.005)
    t = 2.5758293035489004
    frac = 2.0 * (t * math.exp(-t * t / 2.0) / math.sqrt(2.0 * math.pi) + 0.005)
    g = np.random.default_rng(42).standard_normal(1_000_000).astype(F32)
    (_, _, ratio), _, _ = oracle.monitored_step(g, np.zeros_like(g), 10_000)
    assert abs(ratio * ratio / frac - 1.0) < 0.02, (ratio * ratio, frac)
    assert ratio < 0.9          # Top-1% alone would raise the pages' alarm


def test_random_k_keeps_its_share_of_the_energy():
    g = np.random.default_rng(3).standard_normal(400_000).astype(F32)
    (_, _, ratio), _, _ = oracle.monitored_step(g, np.zeros_like(g), 40_000, select="randk", select_seed=5)
    assert abs(ratio * ratio / 0.1 - 1.0) < 0.03


def test_pythagoras_with_the_residual():
    rng = np.random.default_rng(7)
    g = rng.standard_normal(50_000).astype(F32)
    r = (rng.standard_normal(50_000) * 0.3).astype(F32)
    (sc, sg, _), _, new_res = oracle.monitored_step(g, r, 777)
    rr = new_res.astype(np.float64)
    assert abs(sc - (sg + float(rr @ rr))) <= 1e-12 * sc


def test_qsgd_exact_case_and_expected_variance():
    # groups of 64 equal magnitudes a = 2^-3 with s = 8: |v|/nu * s = 1 exactly, so
    # every level is 1 and g_hat = v: the monitor sees no loss at all
    rng = np.random.default_rng(11)
    g = (np.where(rng.random(64 * 50) < 0.5, -1.0, 1.0) * 0.125).astype(F32)
    (sc, sg, ratio), _, _ = oracle.monitored_step(g, np.zeros_like(g), g.size, levels=8, group=64, qsgd_seed=3)
    assert ratio == 1.0 and sc == sg
    # in general E[g_hat^2] = v^2 + (nu/s)^2 p (1 - p), p the fractional part of |v| s / nu
    v = rng.standard_normal(64 * 8).astype(F32)
    s = 15
    nu = np.sqrt((v.astype(np.float64) ** 2).reshape(-1, 64).sum(1)).repeat(64)
    u = np.abs(v) * s / nu
    p = u - np.floor(u)
    expect = float(np.sum(v.astype(np.float64) ** 2) + np.sum((nu / s) ** 2 * p * (1 - p)))
    sgs = [oracle.monitored_step(v, np.zeros_like(v), v.size, levels=s, group=64, qsgd_seed=sd)[0][1]
           for sd in range(400)]
    assert abs(np.mean(sgs) / expect - 1.0) < 0.005


@pytest.mark.parametrize("e", [-20, 3])
def test_ratio_is_scale_invariant(e):
    rng = np.random.default_rng(13)
    g = rng.standard_normal(20_000).astype(F32)
    r = (rng.standard_normal(20_000) * 0.1).astype(F32)
    a = oracle.monitored_step(g, r, 300)[0]
    b = oracle.monitored_step((g * F32(2.0 ** e)).astype(F32), (r * F32(2.0 ** e)).astype(F32), 300)[0]
    assert a[2] == b[2] and b[0] == a[0] * 4.0 ** e
