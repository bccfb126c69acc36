"""Pins for the oracle's error-feedback Top-K (CPU only).

* brute force: a pure-Python selection loop (repeatedly take the largest key, lowest
  index first) on tiny adversarial inputs -- a different algorithm from the oracle's
  sort;
* the exact error-feedback identity scatter(idx, val) + r' == c;
* the O(n) invariant checker, itself checked on planted mistakes;
* a closed form: the residual energy of one 1%-step on N(0,1) data.
"""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from hypothesis.extra import numpy as hnp

import oracle
from golden_io import read_kv
import workloads

F32 = np.float32


def brute_force_topk(c, k):
    keys = [int(v) & 0x7FFFFFFF for v in np.asarray(c, F32).view(np.uint32)]
    left = list(range(len(keys)))
    chosen = []
    for _ in range(k):
        best = None
        for i in left:
            if best is None or keys[i] > keys[best] or (keys[i] == keys[best] and i < best):
                best = i
        chosen.append(best)
        left.remove(best)
    return sorted(chosen)


special = st.sampled_from([0.0, -0.0, 1.0, -1.0, 2.0, -2.0, np.inf, -np.inf, 1e-45, -1e-45,
                           1.1754942e-38, 3.4028235e38, 0.5, -0.5])
values = st.one_of(special, st.floats(-4, 4, width=32, allow_nan=False))


@settings(max_examples=300, deadline=None)
@given(g=hnp.arrays(F32, st.integers(1, 48), elements=values),
       data=st.data())
def test_matches_brute_force(g, data):
    n = g.size
    r = data.draw(hnp.arrays(F32, n, elements=values))
    k = data.draw(st.integers(0, n))
    with np.errstate(all="ignore"):
        c = (g + r).astype(F32)
    idx, val, res = oracle.ef_topk(g, r, k)
    assert idx.dtype == np.int64
    assert idx.tolist() == brute_force_topk(c, k)
    assert np.array_equal(val.view(np.uint32), c[idx].view(np.uint32))
    # new residual: c with the kept entries set to +0.0, bit for bit
    want = c.copy()
    want[idx] = 0.0
    assert np.array_equal(res.view(np.uint32), want.view(np.uint32))
    assert oracle.topk_invariant_holds(c, idx, k)


def test_all_ties_take_lowest_indices():
    g = np.full(100, 0.25, F32)
    idx, _, _ = oracle.ef_topk(g, np.zeros_like(g), 7)
    assert idx.tolist() == list(range(7))
    g[50] = -0.25      # same magnitude, opposite sign: still a tie
    g[3] = 0.125       # smaller
    idx, _, _ = oracle.ef_topk(g, np.zeros_like(g), 7)
    assert idx.tolist() == [0, 1, 2, 4, 5, 6, 7]


def test_index_base_and_edges():
    g = np.arange(10, dtype=F32) - 4.5
    idx, val, res = oracle.ef_topk(g, np.zeros_like(g), 0, index_base=5)
    assert idx.size == 0 and np.array_equal(res, g)
    idx, val, res = oracle.ef_topk(g, np.zeros_like(g), 10, index_base=1 << 40)
    assert idx.tolist() == [(1 << 40) + i for i in range(10)]
    assert not res.any()


def test_error_feedback_identity_two_steps():
    g1, g2 = workloads.ef_demo_gradients(20000)
    r = np.zeros_like(g1)
    for g in (g1, g2):
        c = (g + r).astype(F32)
        idx, val, r = oracle.ef_topk(g, r, 200)
        rebuilt = r.copy()
        rebuilt[idx] = rebuilt[idx] + val
        assert np.array_equal(rebuilt.view(np.uint32) & 0x7FFFFFFF, c.view(np.uint32) & 0x7FFFFFFF)
        assert np.array_equal(rebuilt, c)


def test_invariant_checker_catches_planted_mistakes():
    rng = np.random.default_rng(5)
    c = rng.standard_normal(5000).astype(F32)
    c[100:110] = F32(3.0)          # ties at the threshold region
    k = 105
    idx, _, _ = oracle.ef_topk(c, np.zeros_like(c), k)
    assert oracle.topk_invariant_holds(c, idx, k)
    key = oracle.magnitude_key(c)
    # swap the smallest kept entry for the largest dropped one
    kept_small = idx[np.argmin(key[idx])]
    dropped = np.setdiff1d(np.arange(c.size), idx)
    bad = np.sort(np.concatenate([idx[idx != kept_small], [dropped[np.argmax(key[dropped])]]]))
    assert not oracle.topk_invariant_holds(c, bad, k)
    # wrong order
    assert not oracle.topk_invariant_holds(c, idx[::-1].copy(), k)
    # tie broken toward the higher index
    c2 = np.zeros(10, F32)
    c2[[2, 5, 8]] = 1.0
    assert oracle.topk_invariant_holds(c2, np.array([2, 5]), 2)
    assert not oracle.topk_invariant_holds(c2, np.array([2, 8]), 2)


def test_demo_payload_sizes():
    kv = read_kv("demo_payload_sizes.txt")
    g1, _ = workloads.ef_demo_gradients()
    assert g1.nbytes == kv["grad_bytes"] and g1.size == kv["n"]
    k = max(1, int(g1.size * 0.01))
    assert k == kv["k"]
    idx, val, _ = oracle.ef_topk(g1, np.zeros_like(g1), k)
    assert idx.nbytes + val.nbytes == kv["topk_bytes"]
    assert int(10 * g1.nbytes / (idx.nbytes + val.nbytes)) == kv["topk_ratio_x10"]
    codes, *_ = oracle.quant_minmax(g1, 0, 8)
    assert codes.nbytes == kv["int8_bytes"] and g1.nbytes == 4 * codes.nbytes
    assert oracle.pack_int4(oracle.quant_minmax(g1, 0, 4)[0]).nbytes == kv["int4_bytes"]


def test_closed_form_residual_energy():
    """Energy left after keeping the top 1% of n N(0,1) values: with t the 99.5%
    two-sided point, E[Z^2; |Z| < t] = P(|Z| < t) - 2 t phi(t) (integration by parts)."""
    from scipy.stats import norm
    g1, _ = workloads.ef_demo_gradients()
    n, k = g1.size, 10_000
    _, _, r = oracle.ef_topk(g1, np.zeros_like(g1), k)
    t = norm.ppf(1 - k / n / 2)
    expect = n * ((1 - k / n) - 2 * t * norm.pdf(t))
    got = float(np.sum(r.astype(np.float64) ** 2))
    assert abs(got - expect) / expect < 5e-3, (got, expect)
    assert math.isclose(expect, 915_508, rel_tol=1e-4)
