"""Pins for the oracle's Philox4x32-10 stream (CPU only).

The reference is rocRAND's own Philox4x32-10 engine, run as a library on the host
(tests/pins/philox_rocrand_ref.cpp, built by the
`rocrand_ref` fixture in conftest.py): a different implementation of the SC'11
definition, so a wrong constant, a swapped word or a wrong counter/key layout
fails here.
"""
import numpy as np
import pytest

import oracle
from oracle.philox import random_words


def test_blocks_match_rocrand(rocrand_ref):
    rng = np.random.default_rng(0)
    seeds = [0, 1, 7, 42, 43, 500, 501, 0xFFFFFFFF, 0x1_0000_0000, 0xFFFFFFFFFFFFFFFF,
             int(rng.integers(0, 2**63))]
    ctrs = [0, 1, 2, 3, 255, 2**31 - 1, 2**32 - 1, 2**32, 2**32 + 5, 1_750_000_000,
            int(rng.integers(0, 2**40))]
    pairs = [(s, c) for s in seeds for c in ctrs]
    ref = rocrand_ref(pairs)
    for (s, c), row in zip(pairs, ref):
        got = oracle.philox4x32_10(c & 0xFFFFFFFF, c >> 32, 0, 0, s & 0xFFFFFFFF, s >> 32)
        assert [int(w) for w in got] == [int(v) for v in row], (s, c)


def test_element_word_layout(rocrand_ref):
    # element e takes word (e & 3) of block (e >> 2)
    seed = 7
    e = np.arange(0, 64, dtype=np.int64) + (1 << 34) - 32
    blocks = rocrand_ref([(seed, int(b)) for b in (e >> 2)])
    want = blocks[np.arange(e.size), e & 3].astype(np.uint32)
    assert np.array_equal(random_words(seed, e), want)


def test_uniform24_is_exact_and_in_range():
    e = np.arange(1 << 16, dtype=np.int64)
    u = oracle.uniform24(123, e)
    assert u.dtype == np.float32
    assert u.min() >= 0.0 and u.max() < 1.0
    # exactly 24 random bits: u * 2^24 is an integer below 2^24
    scaled = u.astype(np.float64) * 2.0 ** 24
    assert np.all(scaled == np.floor(scaled))
    assert np.array_equal(scaled.astype(np.uint64),
                          (random_words(123, e) >> np.uint32(8)).astype(np.uint64))


def test_uniform24_chi_square():
    from scipy import stats
    u = oracle.uniform24(99, np.arange(1 << 18, dtype=np.int64))
    hist, _ = np.histogram(u, bins=64, range=(0.0, 1.0))
    chi2 = stats.chisquare(hist).pvalue
    assert chi2 > 1e-4
