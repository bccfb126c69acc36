"""Pins for the oracle's QSGD and TernGrad (CPU only).

* hand-worked fixtures whose outcome does not depend on the random draw;
* the pairwise tree order against a recursive halving written independently;
* the group norm against float64 np.linalg.norm;
* unbiasedness over many seeds against the exact expectation of the 24-bit draw;
* code sets, level bounds, sign agreement, packing and byte counts.
"""
import numpy as np
import pytest

import oracle
from golden_io import read_cases
import workloads

F32 = np.float32


def recursive_tree_sum(v):
    v = np.asarray(v, F32)
    if v.size == 1:
        return F32(v[0])
    h = v.size // 2
    return F32(recursive_tree_sum(v[:h]) + recursive_tree_sum(v[h:]))


@pytest.mark.parametrize("group", [4, 64, 256])
def test_tree_order_matches_recursive_halving(group):
    x = workloads.bucket(group * 50 + group // 2)
    got = oracle.pairwise_sum_of_squares(x, group)
    pad = np.zeros(got.size * group, F32)
    pad[:x.size] = x
    sq = (pad * pad).astype(F32)
    for j in range(got.size):
        assert got[j].view(np.uint32) == recursive_tree_sum(sq[j * group:(j + 1) * group]).view(np.uint32)


def test_norm_close_to_float64():
    x = workloads.bucket(64 * 2000)
    _, norms, _, _ = oracle.qsgd(x, 64, 15, seed=7)
    ref = np.linalg.norm(x.astype(np.float64).reshape(-1, 64), axis=1)
    assert np.max(np.abs(norms - ref) / ref) <= 2.0 ** -20


@pytest.mark.parametrize("name", ["qsgd_exact_levels", "qsgd_half_levels", "qsgd_zero_group"])
def test_qsgd_hand_worked(name):
    case = read_cases("qsgd_tern_hand.txt")[name]
    x = np.array([float(v) for v in case["x"]], F32)
    group, levels = int(case["group"][0]), int(case["levels"][0])
    for seed in (0, 1, 7, 12345):
        codes, norms, ghat, _ = oracle.qsgd(x, group, levels, seed)
        assert codes.tolist() == [int(v) for v in case["codes"]]
        assert norms.tolist() == [float(v) for v in case["norms"]]
        assert ghat.tolist() == [float(v) for v in case["ghat"]]


def test_qsgd_levels_bounds_and_signs():
    x = workloads.bucket(64 * 500 + 13)
    s = 15
    codes, norms, ghat, _ = oracle.qsgd(x, 64, s, seed=7)
    nu = norms[np.arange(x.size) // 64]
    u = (np.abs(x).astype(np.float64) / nu) * s
    lev = np.abs(codes.astype(np.int64))
    assert np.all(lev <= s)
    assert np.all((lev == np.floor(u)) | (lev == np.floor(u) + 1) | (lev == s))
    assert np.all((codes == 0) | (np.sign(codes) == np.sign(x)))
    assert np.array_equal(oracle.dequant_qsgd(codes, norms, 64, s), ghat)


def test_qsgd_unbiased_over_seeds():
    x = workloads.bucket(256, seed=21)
    s = 15
    _, norms, _, _ = oracle.qsgd(x, 64, s, seed=0)
    nu = norms[np.arange(x.size) // 64].astype(F32)
    u = ((np.abs(x) / nu).astype(F32) * F32(s)).astype(F32)
    l = np.floor(u)
    p = (u - l).astype(np.float64)
    # U takes values j / 2^24, so P(U < p) = ceil(p * 2^24) / 2^24 exactly
    exp_level = np.minimum(l + np.ceil(p * 2.0 ** 24) / 2.0 ** 24, s)
    seeds = 1500
    lev = np.zeros((seeds, x.size))
    for t in range(seeds):
        lev[t] = np.abs(oracle.qsgd(x, 64, s, seed=1000 + t)[0].astype(np.int64))
    mean = lev.mean(axis=0)
    sd = np.sqrt(np.maximum(p * (1 - p), 1e-12) / seeds)
    z = np.abs(mean - exp_level) / sd
    assert np.all((z < 5.5) | (p == 0))
    # and the expected value of g_hat is x up to the 2^-24 granularity of the draw
    exp_ghat = exp_level * nu.astype(np.float64) / s
    assert np.max(np.abs(exp_ghat - np.abs(x))) <= 1e-6 * np.max(np.abs(x)) + 2.0 ** -24 * nu.max()


def test_tern_pack_hand_worked():
    case = read_cases("qsgd_tern_hand.txt")["tern_pack"]
    codes = np.array([int(v) for v in case["codes"]], np.int8)
    packed = oracle.pack_ternary(codes)
    assert packed.tolist() == [int(v, 16) for v in case["packed"]]
    assert oracle.unpack_ternary(packed, codes.size).tolist() == codes.tolist()


def test_tern_extremes_any_seed():
    case = read_cases("qsgd_tern_hand.txt")["tern_extremes"]
    x = np.array([float(v) for v in case["x"]], F32)
    for seed in range(20):
        packed, scales, codes, ghat, _ = oracle.terngrad(x, [0, x.size], seed)
        assert codes.tolist() == [int(v) for v in case["codes"]]
        assert scales.tolist() == [float(v) for v in case["scale"]]


def test_tern_codes_bytes_and_patterns():
    x, off = workloads.layered(3, 3, 1001)       # lengths = 1 mod 4: ragged tails
    packed, scales, codes, ghat, _ = oracle.terngrad(x, off, seed=3)
    assert set(np.unique(codes).tolist()) <= {-1, 0, 1}
    two_bit = np.stack([(packed >> (2 * m)) & 3 for m in range(4)])
    assert not np.any(two_bit == 2)
    assert packed.size == 3 * ((1001 + 3) // 4)
    assert 4 * 1001 == 16 * 1001 // 4
    for s in range(3):
        seg = x[off[s]:off[s + 1]]
        assert scales[s] == np.abs(seg).max()
        nb = (1001 + 3) // 4
        assert oracle.unpack_ternary(packed[s * nb:(s + 1) * nb], 1001).tolist() == codes[off[s]:off[s + 1]].tolist()


def test_tern_unbiased_over_seeds():
    x = workloads.bucket(128, seed=8)
    sc = np.abs(x).max()
    p = (np.abs(x) / sc).astype(np.float64)
    exp_b = np.ceil(p * 2.0 ** 24) / 2.0 ** 24
    seeds = 1500
    acc = np.zeros(x.size)
    for t in range(seeds):
        acc += np.abs(oracle.terngrad(x, [0, x.size], seed=t)[2])
    mean = acc / seeds
    sd = np.sqrt(np.maximum(p * (1 - p), 1e-12) / seeds)
    assert np.all(np.abs(mean - exp_b) / sd < 5.5)


def test_tern_rng_index_is_global_position():
    x = workloads.bucket(400, seed=4)
    _, _, codes_all, _, _ = oracle.terngrad(x, [0, 150, 400], seed=9, index_base=1000)
    _, _, c2, _, _ = oracle.terngrad(x[150:], [0, 250], seed=9, index_base=1150)
    assert np.array_equal(codes_all[150:], c2)
