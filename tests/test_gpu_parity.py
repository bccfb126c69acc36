"""GPU parity: every entry point against the CPU oracle on the same seeded inputs.

Integer codes, indices and every float output are compared bit for bit (the library
and the oracle perform the same binary32 operations in the same order).  Sizes span
several tiles and ragged tails and finish in seconds on the CPU side.
"""
import numpy as np
import pytest

import oracle
import workloads
from gc_testlib import assert_bits_equal

pytestmark = pytest.mark.gpu

F32 = np.float32


@pytest.fixture(scope="module")
def gc():
    import torch  # noqa: F401
    import gradient_compression_ddp_amd as lib
    return lib


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.cpu().numpy()


# ---------------------------------------------------------------- calibration -------

@pytest.mark.parametrize("n", [1, 4, 4096 * 3 + 7, 16384, 1 << 20])
def test_stream_floor(gc, n):
    """The benchmark floor pass: out[i] = (x[i] > 0), ragged ends included, signed zeros
    and negative values giving 0."""
    x = workloads.bucket(n, seed=n)
    x[: min(n, 3)] = np.array([0.0, -0.0, 1e-45], F32)[: min(n, 3)]
    out = host(gc.stream_floor(dev(x)))
    assert out.dtype == np.uint8
    assert_bits_equal(out, (x > 0).astype(np.uint8), "floor bytes")


# ---------------------------------------------------------------- min-max ----------

MINMAX_CASES = [
    (64 * 300 + 37, 64, 8), (64 * 300 + 37, 64, 4), (1000, 4, 8), (1003, 16, 4), (5000, 256, 8),
    (5001, 128, 4), (70_001, 0, 8), (70_001, 0, 4), (300_000, 1000, 8), (300_003, 4097, 4),
    (3, 64, 8), (1, 4, 4), (257, 257, 8),
]


@pytest.mark.parametrize("n,group,bits", MINMAX_CASES)
@pytest.mark.parametrize("ef", [False, True])
def test_minmax(gc, n, group, bits, ef):
    x = workloads.bucket(n, seed=n % 97)
    r = (workloads.bucket(n, seed=5) * F32(0.01)).astype(F32) if ef else None
    codes, mins, scales, _, r_new = oracle.quant_minmax(x, group, bits, residual=r)
    rd = dev(r) if ef else None
    c_d, m_d, s_d = gc.quant_minmax(dev(x), group, bits, residual=rd)
    want_codes = codes if bits == 8 else oracle.pack_int4(codes)
    assert_bits_equal(host(c_d), want_codes, "codes")
    assert_bits_equal(host(m_d), mins, "mins")
    assert_bits_equal(host(s_d), scales, "scales")
    if ef:
        assert_bits_equal(host(rd), r_new, "residual")


def test_minmax_demo_per_tensor_int8(gc):
    g1, _ = workloads.ef_demo_gradients()
    codes, mins, scales, _, _ = oracle.quant_minmax(g1, 0, 8)
    c_d, m_d, s_d = gc.quant_minmax(dev(g1), 0, 8)
    assert_bits_equal(host(c_d), codes, "codes")
    assert_bits_equal(host(m_d), mins, "min")
    assert_bits_equal(host(s_d), scales, "scale")


@pytest.mark.parametrize("bits", [8, 4])
def test_minmax_bucket_full_size(gc, bits):
    x = workloads.bucket()
    codes, mins, scales, _, _ = oracle.quant_minmax(x, 64, bits)
    c_d, m_d, s_d = gc.quant_minmax(dev(x), 64, bits)
    assert_bits_equal(host(c_d), codes if bits == 8 else oracle.pack_int4(codes), "codes")
    assert_bits_equal(host(m_d), mins, "mins")
    assert_bits_equal(host(s_d), scales, "scales")


def test_minmax_signed_zero_and_constant_groups(gc):
    x = np.zeros(64 * 4, F32)
    x[0:64] = 0.0
    x[5] = -0.0
    x[64:128] = 3.5
    x[128:192] = np.linspace(-1, 1, 64, dtype=F32)
    x[192] = -0.0
    x[193:256] = 0.0
    for bits in (8, 4):
        codes, mins, scales, _, _ = oracle.quant_minmax(x, 64, bits)
        c_d, m_d, s_d = gc.quant_minmax(dev(x), 64, bits)
        assert_bits_equal(host(c_d), codes if bits == 8 else oracle.pack_int4(codes), "codes")
        assert_bits_equal(host(m_d), mins, "mins")
        assert_bits_equal(host(s_d), scales, "scales")


@pytest.mark.parametrize("bits,group", [(8, 64), (4, 64), (8, 0), (4, 0)])
@pytest.mark.parametrize("ef", [False, True])
def test_minmax_half_integer_quotients(gc, bits, group, ef):
    """Quotients (x - min) / scale exactly on, and one or two ulps either side of, k + 1/2
    (where the kernels leave the multiply-by-reciprocal estimate for the division), with
    scales 2^-20 .. 2^20 and one group of tiny values; codes bit-exact."""
    L = (1 << bits) - 1
    rng = np.random.default_rng(bits * 10 + (group > 0))
    G = 64
    ng = 512
    xs = []
    for g in range(ng):
        sc = F32(2.0 ** rng.integers(-20, 21))
        mn = F32(rng.integers(-5, 6)) * sc
        k = rng.integers(0, L, G).astype(F32)
        q = (k + F32(0.5)).astype(F32)
        d = rng.integers(-2, 3, G)
        q = np.array([np.nextafter(v, F32(np.inf) if dd > 0 else F32(0)) if dd else v
                      for v, dd in zip(q, d)], F32)
        for _ in range(1):
            q = np.where(np.abs(d) == 2, np.nextafter(q, np.where(d > 0, F32(np.inf), F32(0))), q).astype(F32)
        x = (mn + (q * sc).astype(F32)).astype(F32)
        x[0] = mn
        x[1] = (mn + F32(L) * sc).astype(F32)                 # the group's range is exactly L * scale
        xs.append(x)
    xs[7] = (rng.standard_normal(G) * F32(1e-41)).astype(F32)   # denormal group
    x = np.concatenate(xs).astype(F32)
    r = (rng.standard_normal(x.size) * F32(1e-7)).astype(F32) if ef else None
    codes, mins, scales, _, r_new = oracle.quant_minmax(x, group, bits, residual=r)
    rd = dev(r) if ef else None
    c_d, m_d, s_d = gc.quant_minmax(dev(x), group, bits, residual=rd)
    assert_bits_equal(host(c_d), codes if bits == 8 else oracle.pack_int4(codes), "codes")
    assert_bits_equal(host(m_d), mins, "mins")
    assert_bits_equal(host(s_d), scales, "scales")
    if ef:
        assert_bits_equal(host(rd), r_new, "residual")


# ---------------------------------------------------------------- QSGD -------------

@pytest.mark.parametrize("n,group,levels,base", [
    (64 * 500 + 13, 64, 15, 0), (10_000, 4, 1, 0), (10_003, 256, 127, 3), (777, 32, 7, 1 << 33),
    (5, 64, 15, 2), (64 * 64, 64, 127, 6), (64 * 300 + 5, 64, 6, 0), (20_001, 16, 12, 9),
    (64 * 200, 128, 126, 1 << 20),
])
@pytest.mark.parametrize("ef", [False, True])
def test_qsgd(gc, n, group, levels, base, ef):
    x = workloads.bucket(n, seed=n % 89)
    r = (workloads.bucket(n, seed=6) * F32(0.01)).astype(F32) if ef else None
    codes, norms, _, r_new = oracle.qsgd(x, group, levels, seed=7, index_base=base, residual=r)
    rd = dev(r) if ef else None
    c_d, n_d = gc.qsgd(dev(x), group, levels, 7, index_base=base, residual=rd)
    assert_bits_equal(host(c_d), codes, "codes")
    assert_bits_equal(host(n_d), norms, "norms")
    if ef:
        assert_bits_equal(host(rd), r_new, "residual")


def test_qsgd_bucket_full_size(gc):
    x = workloads.bucket()
    codes, norms, _, _ = oracle.qsgd(x, 64, 15, seed=7)
    c_d, n_d = gc.qsgd(dev(x), 64, 15, 7)
    assert_bits_equal(host(c_d), codes, "codes")
    assert_bits_equal(host(n_d), norms, "norms")


# ---------------------------------------------------------------- TernGrad ---------

@pytest.mark.parametrize("lens,base", [
    ([1001, 1001, 1001], 0), ([14_583, 14_583, 14_583, 14_583], 0), ([5, 0, 3, 250, 252, 1], 0),
    ([4096, 4096], 2), ([100_001, 7, 65_537], 1 << 33), ([1], 0),
])
@pytest.mark.parametrize("ef", [False, True])
def test_terngrad(gc, lens, base, ef):
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    n = int(off[-1])
    x = workloads.bucket(n, seed=len(lens)) if n else np.zeros(0, F32)
    # vary the scale per segment as in the layered workload
    for s in range(len(lens)):
        x[off[s]:off[s + 1]] *= F32(10.0 ** (s % 3))
    r = (workloads.bucket(n, seed=8) * F32(0.01)).astype(F32) if ef else None
    packed, scales, _, _, r_new = oracle.terngrad(x, off, seed=3, index_base=base, residual=r)
    rd = dev(r) if ef else None
    p_d, s_d = gc.terngrad(dev(x), off, 3, index_base=base, residual=rd)
    assert_bits_equal(host(p_d), packed, "packed codes")
    assert_bits_equal(host(s_d), scales, "scales")
    if ef:
        assert_bits_equal(host(rd), r_new, "residual")


@pytest.mark.parametrize("sc", [2.0, 2.0 ** -70, 3.0e30, 1e-40])
def test_terngrad_decision_boundaries(gc, sc):
    # |x| placed at U * s * (1 + d) for the element's own uniform U (taken from the oracle),
    # with d from 0 to +-2^-19, so that fl(|x|/s) lands on, just above and just below U
    # (inside the band where the kernel leaves its product estimate for the division);
    # scales far from 1 (2^-70, 3e30) and a subnormal one (1e-40, whose reciprocal
    # overflows); plus tiny values, denormals and zeros.  Codes must equal the oracle's
    # bit for bit.
    n, seed = 64 * 4096, 11
    u = oracle.uniform24(seed, np.arange(n, dtype=np.int64)).astype(np.float64)
    ds = np.array([0.0] + [sgn * 2.0 ** -e for e in range(19, 26) for sgn in (1, -1)])
    d = ds[np.arange(n) % ds.size]
    x = (u * sc * (1.0 + d)).astype(F32)
    x = np.minimum(np.abs(x), F32(sc)).astype(F32)
    x[::97] = F32(sc) * F32(2.0 ** -70) if sc > 1e-20 else F32(0.0)
    x[5::211] = np.float32(1e-45)
    x[7::389] = F32(0.0)
    sign = np.where(np.random.default_rng(3).random(n) < 0.5, -1.0, 1.0).astype(F32)
    x = (x * sign).astype(F32)
    x[0] = F32(sc)                                      # the segment's max
    packed, scales, _, _, _ = oracle.terngrad(x, [0, n], seed=seed)
    p_d, s_d = gc.terngrad(dev(x), np.array([0, n], np.int64), seed)
    assert_bits_equal(host(s_d), scales, "scale")
    assert_bits_equal(host(p_d), packed, "packed codes")


def test_terngrad_layers_scaled(gc):
    x, off = workloads.tern_layers(24, 145_833)        # lengths = 1 mod 4, as in the 350M case
    packed, scales, _, _, _ = oracle.terngrad(x, off, seed=3)
    p_d, s_d = gc.terngrad(dev(x), off, 3)
    assert_bits_equal(host(p_d), packed, "packed codes")
    assert_bits_equal(host(s_d), scales, "scales")


@pytest.mark.parametrize("ef,base", [(False, 0), (True, 3), (False, 1 << 35)])
def test_terngrad_many_segments(gc, ef, base):
    # 100 segments (more than one launch batch of 32): ragged lengths including empty and
    # one-element segments, starts at every offset mod 4, scales spread over 9 decades.
    rng = np.random.default_rng(21)
    lens = rng.integers(0, 30_000, 100)
    lens[::7] = 0
    lens[3::11] = 1
    lens[5::13] = rng.integers(4096, 70_000, lens[5::13].size)
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    n = int(off[-1])
    x = workloads.bucket(n, seed=22)
    for s in range(lens.size):
        x[off[s]:off[s + 1]] *= F32(10.0 ** (s % 9 - 4))
    r = (workloads.bucket(n, seed=23) * F32(1e-3)).astype(F32) if ef else None
    packed, scales, _, _, r_new = oracle.terngrad(x, off, seed=13, index_base=base, residual=r)
    rd = dev(r) if ef else None
    p_d, s_d = gc.terngrad(dev(x), off, 13, index_base=base, residual=rd)
    assert_bits_equal(host(s_d), scales, "scales")
    assert_bits_equal(host(p_d), packed, "packed codes")
    if ef:
        assert_bits_equal(host(rd), r_new, "residual")


@pytest.mark.parametrize("ef", [False, True])
def test_terngrad_batches_closed_by_size(gc, ef):
    # segments of 2^24 + 5, 9,000,001, 9,000,003, 2^23 + 7 and 3 elements: starts at four
    # different offsets mod 4, and batches of layers that close once they hold 2^24
    # elements (the first segment alone, then two, then two), so launches mix max tiles and
    # code tiles of segments of different sizes, as at 24 x 14,583,333
    lens = np.array([(1 << 24) + 5, 9_000_001, 9_000_003, (1 << 23) + 7, 3], dtype=np.int64)
    off = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    n = int(off[-1])
    x = workloads.bucket(n, seed=31)
    for s in range(lens.size):
        x[off[s]:off[s + 1]] *= F32(10.0 ** (s - 2))
    r = (workloads.bucket(n, seed=32) * F32(1e-2)).astype(F32) if ef else None
    packed, scales, _, _, r_new = oracle.terngrad(x, off, seed=17, index_base=5, residual=r)
    rd = dev(r) if ef else None
    p_d, s_d = gc.terngrad(dev(x), off, 17, index_base=5, residual=rd)
    assert_bits_equal(host(s_d), scales, "scales")
    assert_bits_equal(host(p_d), packed, "packed codes")
    if ef:
        assert_bits_equal(host(rd), r_new, "residual")


# ---------------------------------------------------------------- EF Top-K ---------

def run_topk(gc, g, r, k, base=0):
    rd = dev(r)
    idx, val = gc.ef_topk(dev(g), rd, k, index_base=base)
    return host(idx), host(val), host(rd)


def check_topk(gc, g, r, k, base=0):
    o_idx, o_val, o_res = oracle.ef_topk(g, r, k, index_base=base)
    idx, val, res = run_topk(gc, g, r, k, base)
    assert_bits_equal(idx, o_idx, "idx")
    assert_bits_equal(val, o_val, "values")
    assert_bits_equal(res, o_res, "residual")
    return res


def test_topk_demo_two_steps(gc):
    g1, g2 = workloads.ef_demo_gradients()
    r = np.zeros_like(g1)
    r = check_topk(gc, g1, r, workloads.DEMO_K)
    check_topk(gc, g2, r, workloads.DEMO_K)


@pytest.mark.parametrize("n,k", [(8192 * 3 + 77, 1), (8192 * 3 + 77, 100), (8192 * 3 + 77, 8192 * 3 + 77),
                                 (1, 1), (7, 3), (8192, 8192), (100_000, 50_000), (2_500_001, 25_000),
                                 (5_000_003, 4_000_000), (1 << 20, 10_000), ((1 << 20) + 1, 10_000)])
def test_topk_sizes(gc, n, k):
    g = workloads.bucket(n, seed=11)
    r = (workloads.bucket(n, seed=12) * F32(0.1)).astype(F32)
    check_topk(gc, g, r, k)


def test_topk_ties_and_specials(gc):
    n = 50_000
    g = np.full(n, 0.5, F32)                        # all ties: lowest indices win
    check_topk(gc, g, np.zeros(n, F32), 1234)
    g = np.zeros(n, F32)
    g[::7] = -0.0
    check_topk(gc, g, np.zeros(n, F32), 77)
    rng = np.random.default_rng(3)
    g = rng.choice(np.array([0.0, -0.0, 1.0, -1.0, 2.0, np.inf, -np.inf, np.nan, 1e-45], F32), n)
    check_topk(gc, g, np.zeros(n, F32), 10_000)


def test_topk_whole_input_select_all_ties(gc):
    # n = 2^20 (sampled) with every element, or all but five, tied with the k-th key:
    # every element reaches the bound, the pool overflows and the exact fallback over the
    # full c selects, ties to the lower index
    n = 1 << 20
    check_topk(gc, np.full(n, 0.5, F32), np.zeros(n, F32), 3)
    g = np.full(n, -0.25, F32)
    g[n - 5:] = 0.25
    check_topk(gc, g, np.zeros(n, F32), n - 2)


def test_topk_forced_fallback(gc):
    # a huge tie block defeats the candidate bound: the pool overflows and the exact
    # full-array path must still produce the oracle's answer
    n = 3_000_000
    g = np.full(n, 1.0, F32)
    g[1_000_000:1_000_010] = 2.0
    check_topk(gc, g, np.zeros(n, F32), 500_000)


def test_topk_index_base_and_zero_k(gc):
    g = workloads.bucket(40_000, seed=2)
    r = np.zeros_like(g)
    check_topk(gc, g, r, 400, base=(1 << 36) + 5)
    idx, val, res = run_topk(gc, g, r, 0)
    assert idx.size == 0
    assert_bits_equal(res, (g + r).astype(F32), "k=0 residual")


def test_topk_layered_three_steps_with_qsgd(gc):
    import torch
    n_layers, layer_len = 32, 65_537
    r = np.zeros(n_layers * layer_len, F32)
    rd = dev(r)
    for t in (1, 2, 3):
        g, _ = workloads.big_layers_host(n_layers, layer_len, step=t)
        k = g.size // 100
        o_idx, o_codes, o_norms, o_res, o_val = oracle.ef_topk_qsgd(g, r, k, levels=127, group=64,
                                                                     seed=500 + t)
        idx, codes, norms, val = gc.ef_topk(dev(g), rd, k, qsgd_levels=127, qsgd_group=64,
                                            qsgd_seed=500 + t)
        assert_bits_equal(host(idx), o_idx, f"step {t} idx")
        assert_bits_equal(host(val), o_val, f"step {t} values")
        assert_bits_equal(host(codes), o_codes, f"step {t} codes")
        assert_bits_equal(host(norms), o_norms, f"step {t} norms")
        assert_bits_equal(host(rd), o_res, f"step {t} residual")
        r = o_res


def test_topk_qsgd_without_values(gc):
    g, _ = workloads.big_layers_host(4, 30_001, step=1)
    r = np.zeros_like(g)
    k = 1_203
    o_idx, o_codes, o_norms, o_res, _ = oracle.ef_topk_qsgd(g, r, k, levels=15, group=16, seed=9)
    rd = dev(r)
    idx, codes, norms, val = gc.ef_topk(dev(g), rd, k, qsgd_levels=15, qsgd_group=16, qsgd_seed=9,
                                        want_values=False)
    assert val is None
    assert_bits_equal(host(idx), o_idx, "idx")
    assert_bits_equal(host(codes), o_codes, "codes")
    assert_bits_equal(host(norms), o_norms, "norms")
    assert_bits_equal(host(rd), o_res, "residual")


# ---------------------------------------------------------------- decompress -------

def test_decompress_all_kinds(gc):
    import torch
    x = workloads.bucket(64 * 40 + 9)
    n = x.size
    cases = []
    c8, m8, s8, _, _ = oracle.quant_minmax(x, 64, 8)
    cases.append((gc.KIND_MINMAX8, c8, m8, s8, 64, 0))
    c4, m4, s4, _, _ = oracle.quant_minmax(x, 64, 4)
    cases.append((gc.KIND_MINMAX4, oracle.pack_int4(c4), m4, s4, 64, 0))
    cq, nq, _, _ = oracle.qsgd(x, 64, 15, seed=7)
    cases.append((gc.KIND_QSGD, cq, nq, None, 64, 15))
    pk, sc, _, _, _ = oracle.terngrad(x, [0, n], seed=3)
    cases.append((gc.KIND_TERN, pk, sc, None, 0, 0))
    cases.append((gc.KIND_F32, x, None, None, 0, 0))
    base = np.linspace(-1, 1, 3 * n, dtype=F32)
    idx = np.sort(np.random.default_rng(1).choice(3 * n, n, replace=False)).astype(np.int64) + 1000
    for kind, codes, m0, m1, group, levels in cases:
        for alpha, acc in ((1.0, 0), (0.125, 1)):
            want = oracle.decompress_scatter(kind, None, n, 0, codes, m0, m1, group, levels, alpha, acc,
                                             np.zeros(n, F32) + F32(0.25))
            out = dev(np.zeros(n, F32) + F32(0.25))
            gc.decompress_scatter(kind, dev(codes), n, out, meta0=None if m0 is None else dev(m0),
                                  meta1=None if m1 is None else dev(m1), group=group, levels=levels,
                                  alpha=alpha, accumulate=bool(acc))
            assert_bits_equal(host(out), want, f"dense kind {kind}")
            want = oracle.decompress_scatter(kind, idx, n, 1000, codes, m0, m1, group, levels, alpha, acc,
                                             base.copy())
            out = dev(base)
            gc.decompress_scatter(kind, dev(codes), n, out, idx=dev(idx), index_base=1000,
                                  meta0=None if m0 is None else dev(m0), meta1=None if m1 is None else dev(m1),
                                  group=group, levels=levels, alpha=alpha, accumulate=bool(acc))
            assert_bits_equal(host(out), want, f"scatter kind {kind}")


def test_topk_small_k_on_large_n(gc):
    # k far below the sample's resolution: the candidate pool is sized from the bound
    n = 9_000_001
    g = workloads.bucket(n, seed=21)
    r = np.zeros(n, F32)
    for k in (1, 7, 1000):
        check_topk(gc, g, r, k)


@pytest.mark.parametrize("shift_out,shift_codes", [(0, 0), (1, 0), (0, 1)])
def test_decompress_dense_tiles_groups_alignment(gc, shift_out, shift_codes):
    """Dense decode over several 4096-entry tiles with a ragged tail, groups that are not
    powers of two, and buffers offset so that the vector path cannot be used."""
    n = 6 * 4100   # 24,600: six 4,096-entry tiles and a ragged tail; six TernGrad segments
    x = workloads.bucket(n, seed=11)
    cases = []
    c8, m8, s8, _, _ = oracle.quant_minmax(x, 1000, 8)
    cases.append((gc.KIND_MINMAX8, c8, m8, s8, 1000, 0))
    c4, m4, s4, _, _ = oracle.quant_minmax(x, 64, 4)
    cases.append((gc.KIND_MINMAX4, oracle.pack_int4(c4), m4, s4, 64, 0))
    cq, nq, _, _ = oracle.qsgd(x, 64, 127, seed=9)
    cases.append((gc.KIND_QSGD, cq, nq, None, 64, 127))
    seg = np.arange(0, n + 1, 4100, dtype=np.int64)
    pk, sc, _, _, _ = oracle.terngrad(x, seg, seed=5)
    cases.append((gc.KIND_TERN, pk, sc, None, 4100, 0))
    cases.append((gc.KIND_F32, x, None, None, 0, 0))
    for kind, codes, m0, m1, group, levels in cases:
        if shift_codes and kind != gc.KIND_MINMAX8:
            continue   # a one-byte offset is only meaningful for byte codes
        for alpha, acc in ((1.0, 0), (-0.5, 1)):
            init = np.linspace(-2, 2, n + shift_out, dtype=F32)
            want = oracle.decompress_scatter(kind, None, n, 0, codes, m0, m1, group, levels, alpha, acc,
                                             init[shift_out:].copy())
            out_full = dev(init)
            out = out_full[shift_out:]
            cbuf = dev(np.concatenate([np.zeros(shift_codes, codes.dtype), codes]))[shift_codes:]
            gc.decompress_scatter(kind, cbuf, n, out, meta0=None if m0 is None else dev(m0),
                                  meta1=None if m1 is None else dev(m1), group=group, levels=levels,
                                  alpha=alpha, accumulate=bool(acc))
            got = host(out_full)
            assert_bits_equal(got[shift_out:], want, f"kind {kind} shift {shift_out}/{shift_codes}")
            assert_bits_equal(got[:shift_out], init[:shift_out], "bytes before out untouched")
