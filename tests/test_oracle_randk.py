"""Pins of the Random-K oracle (oracle/randk.py), independent of its own code paths.

* the selection keys are recomputed element by element from the Philox4x32-10 block
  function (itself pinned to rocRAND in test_oracle_philox.py), with the word, the
  shift and the global index written out here;
* the k-largest selection with ties to the lower index is checked against a plain sort
  of (-key, position) pairs, on keys with many ties;
* exactly k, ascending, values bit-equal to c, and the error-feedback identity;
* the choice does not depend on the values, and over many seeds every position is kept
  with probability k/n (chi-square).
"""
import numpy as np
import pytest

import oracle
from oracle.philox import philox4x32_10

F32 = np.float32


def key_by_hand(seed, e):
    ctr = e >> 2
    w = philox4x32_10(ctr & 0xFFFFFFFF, ctr >> 32, 0, 0, seed & 0xFFFFFFFF, seed >> 32)
    return int(w[e & 3]) >> 1


@pytest.mark.parametrize("seed,base", [(5, 0), (2 ** 40 + 17, 3), (123, 2 ** 33 + 1)])
def test_keys_element_by_element(seed, base):
    n = 37
    keys = oracle.randk_keys(seed, n, base)
    assert keys.dtype == np.uint32 and np.all(keys < 2 ** 31)
    assert [int(x) for x in keys] == [key_by_hand(seed, base + e) for e in range(n)]


def test_selection_rule_with_ties():
    rng = np.random.default_rng(1)
    for _ in range(200):
        n = int(rng.integers(1, 60))
        key = rng.integers(0, 4, n).astype(np.uint32)          # four values: many ties
        k = int(rng.integers(0, n + 1))
        want = sorted(sorted(range(n), key=lambda i: (-int(key[i]), i))[:k])
        assert list(oracle.randk.select_largest(key, k)) == want


@pytest.mark.parametrize("n,k,seed,base", [(1000, 10, 5, 0), (4097, 4097, 9, 11), (50, 0, 1, 0), (777, 300, 2, 5)])
def test_ef_randk_step(n, k, seed, base):
    rng = np.random.default_rng(n)
    g = rng.standard_normal(n).astype(F32)
    r = (rng.standard_normal(n) * 0.1).astype(F32)
    idx, val, new_r = oracle.ef_randk(g, r, k, seed, base)
    c = (g + r).astype(F32)
    assert idx.size == k and np.all(np.diff(idx) > 0)
    pos = idx - base
    keys = np.array([key_by_hand(seed, base + e) for e in range(n)], dtype=np.int64)
    want = sorted(sorted(range(n), key=lambda i: (-keys[i], i))[:k])
    assert list(pos) == want
    assert np.array_equal(val.view(np.uint32), c[pos].view(np.uint32))
    sent = np.zeros(n, F32)
    sent[pos] = val
    assert np.array_equal(sent + new_r, c)                        # EF identity, exact
    assert np.all(new_r[pos] == 0)


def test_choice_ignores_values_and_is_uniform():
    n, k, seeds = 64, 8, 3000
    hits = np.zeros(n, np.int64)
    g0 = np.zeros(n, F32)
    g1 = np.arange(n, dtype=F32)
    for s in range(seeds):
        i0, _, _ = oracle.ef_randk(g0, np.zeros(n, F32), k, s)
        i1, _, _ = oracle.ef_randk(g1, np.zeros(n, F32), k, s)
        assert np.array_equal(i0, i1)
        hits[i0] += 1
    expect = seeds * k / n
    chi2 = float(((hits - expect) ** 2 / expect).sum())
    # 63 degrees of freedom: the 1e-6 upper quantile is about 132
    assert chi2 < 132, chi2


def test_ef_randk_qsgd_matches_its_parts():
    rng = np.random.default_rng(4)
    n, k = 5000, 500
    g = rng.standard_normal(n).astype(F32)
    r = np.zeros(n, F32)
    idx, codes, norms, new_r, val = oracle.ef_randk_qsgd(g, r, k, seed=3, levels=127, group=64, qsgd_seed=8)
    i2, v2, _ = oracle.ef_randk(g, r, k, 3)
    assert np.array_equal(idx, i2) and np.array_equal(val, v2)
    c2, n2, gh, _ = oracle.qsgd(val, 64, 127, 8)
    assert np.array_equal(codes, c2) and np.array_equal(norms, n2)
    c = (g + r).astype(F32)
    assert np.array_equal(new_r[idx], (val - gh).astype(F32))
    rest = np.ones(n, bool)
    rest[idx] = False
    assert np.array_equal(new_r[rest], c[rest])
