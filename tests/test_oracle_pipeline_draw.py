"""Pins of the Top-K + 8-bit QSGD pipeline's random draw (oracle.ef_topk_qsgd), CPU only.

The 8-bit stage quantizes the kept values in ascending index order, and kept value j
takes the draw of element index j, its position in the kept list, under the step's
seed (5688vip.com "梯度累积与梯度压缩" section 4.3 for the hybrid; hotdry.top
"gradient-compression-quantization-sparsification" section 1.1 for stochastic
rounding).  The tests below fix that choice against rocRAND's Philox4x32-10 engine run
as a library, so they do not lean on the oracle's own generator:

* the kept magnitudes are planted so that every group's norm, every |v|/nu and every
  fractional part p are exact (p = 0.875 at s = 127), so each level is 15 + (U < p) with
  U taken from rocRAND's word for the kept position;
* the planted positions are such that the global-index draw gives other codes, so a
  pipeline that drew by element index (or ignored the step seed) fails;
* the codes and norms also equal the oracle's QSGD of the kept values at index base 0.
"""
import numpy as np
import pytest

import oracle

F32 = np.float32
S = 127


def planted(n, k, seed):
    """g, r with a known Top-K set: the kept positions carry c = +-1 (first 64 kept) or
    +-2 (next 64), split as g + r with both parts exact; everything else has |c| < 0.6."""
    assert k == 128
    rng = np.random.default_rng(seed)
    pos = np.sort(rng.choice(n, k, replace=False)).astype(np.int64)
    sign = np.where(rng.random(k) < 0.5, F32(-1.0), F32(1.0)).astype(F32)
    mag = np.where(np.arange(k) < 64, F32(1.0), F32(2.0)).astype(F32)
    g = rng.uniform(-0.5, 0.5, n).astype(F32)
    r = rng.uniform(-0.1, 0.1, n).astype(F32)
    g[pos] = sign * mag * F32(0.75)
    r[pos] = sign * mag * F32(0.25)
    return g, r, pos, sign, mag


def levels_from_words(words):
    """level = 15 + (U < 0.875) with U = (word >> 8) * 2^-24: up iff word >> 8 < 0.875 * 2^24."""
    return 15 + ((words >> np.uint64(8)) < np.uint64(14_680_064)).astype(np.int64)


def word_of(blocks, e):
    return blocks[np.arange(e.size), e & 3]


@pytest.mark.parametrize("seed,index_base", [(501, 0), (502, 0), (503, 2 ** 33 + 5)])
def test_kept_position_draw_against_rocrand(rocrand_ref, seed, index_base):
    n, k = 3001, 128
    g, r, pos, sign, mag = planted(n, k, seed)
    idx, codes, norms, new_r, val = oracle.ef_topk_qsgd(g, r, k, levels=S, group=64, seed=seed,
                                                        index_base=index_base)
    assert np.array_equal(idx, pos + index_base)
    assert np.array_equal(val, sign * mag)
    # group norms: sqrt(64 * 1) = 8 and sqrt(64 * 4) = 16, exact
    assert norms.tolist() == [8.0, 16.0]
    j = np.arange(k, dtype=np.int64)
    kept_words = word_of(rocrand_ref([(seed, int(c)) for c in j >> 2]), j)
    want = (sign.astype(np.int64) * levels_from_words(kept_words)).astype(np.int8)
    assert np.array_equal(codes, want)
    # the element-index draw would give other codes here, so the test tells the two apart
    e = pos + index_base
    global_words = word_of(rocrand_ref([(seed, int(c)) for c in e >> 2]), e)
    assert not np.array_equal(want, (sign.astype(np.int64) * levels_from_words(global_words)).astype(np.int8))
    # and so would the draw under another seed
    other = word_of(rocrand_ref([(seed + 1, int(c)) for c in j >> 2]), j)
    assert not np.array_equal(want, (sign.astype(np.int64) * levels_from_words(other)).astype(np.int8))
    # residual at the kept positions: c - g_hat with g_hat = sign * fl(nu * level / 127);
    # nu * level is exact and the subtraction is exact (Sterbenz), so fp64 gives it
    lev = np.abs(want.astype(np.float64))
    nu = np.where(np.arange(k) < 64, 8.0, 16.0)
    ghat = sign.astype(np.float64) * (nu * lev / S).astype(F32).astype(np.float64)
    assert np.array_equal(new_r[pos].astype(np.float64), sign * mag.astype(np.float64) - ghat)
    # off the kept set the residual is c itself
    off = np.ones(n, bool)
    off[pos] = False
    assert np.array_equal(new_r[off], (g + r).astype(F32)[off])


@pytest.mark.parametrize("levels,group", [(127, 64), (15, 64), (127, 128)])
def test_pipeline_is_topk_then_qsgd_of_kept_list(levels, group):
    rng = np.random.default_rng(levels + group)
    n, k = 20_011, 301
    g = rng.standard_t(3, n).astype(F32)
    r = (rng.standard_normal(n) * 0.1).astype(F32)
    idx, codes, norms, new_r, val = oracle.ef_topk_qsgd(g, r, k, levels=levels, group=group, seed=77,
                                                        index_base=1000)
    i2, v2, _ = oracle.ef_topk(g, r, k, 1000)
    assert np.array_equal(idx, i2) and np.array_equal(val.view(np.uint32), v2.view(np.uint32))
    c2, n2, gh, _ = oracle.qsgd(v2, group, levels, seed=77, index_base=0)
    assert np.array_equal(codes, c2)
    assert np.array_equal(norms.view(np.uint32), n2.view(np.uint32))
    assert np.array_equal(new_r[idx - 1000].view(np.uint32), (v2 - gh).astype(F32).view(np.uint32))
