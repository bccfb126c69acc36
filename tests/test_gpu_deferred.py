"""GPU parity of the deferred residual update (gc_ef_topk_deferred + gc_ef_flush).

Every call's indices, values, codes and norms are compared bit for bit with the oracle's
EF Top-K step; after gc_ef_flush the residual is compared bit for bit with the oracle's
residual.  Between calls the residual holds c = g + r at every position (the kept
entries' residuals sit in the pending record), which is checked too.  Cases cover the
whole-input select (n <= 2^15), the sampled candidate path, the exact fallback, k = 0,
and a 2^30-element bucket against the direct call.
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


def pure_steps(gc, grads, k, kmax=None):
    """Deferred pure Top-K over the given gradients; checks each step against the oracle
    and the flushed residual at the end."""
    n = grads[0].size
    rd = dev(np.zeros(n, F32))
    pend = gc.pending_record(n, kmax or k, "cuda")
    r = np.zeros(n, F32)
    for t, g in enumerate(grads):
        o_idx, o_val, o_res = oracle.ef_topk(g, r, k)
        idx, val = gc.ef_topk_deferred(dev(g), rd, k, pend)
        assert_bits_equal(host(idx), o_idx, f"step {t} idx")
        assert_bits_equal(host(val), o_val, f"step {t} values")
        # before the flush the residual holds c everywhere: the oracle's residual off the
        # kept set, the kept values on it
        want = o_res.copy()
        want[o_idx] = o_val
        assert_bits_equal(host(rd), want, f"step {t} unflushed residual")
        r = o_res
    gc.ef_flush(rd, pend)
    assert_bits_equal(host(rd), r, "flushed residual")
    return rd, pend


def test_deferred_demo_two_steps(gc):
    g1, g2 = workloads.ef_demo_gradients()
    pure_steps(gc, [g1, g2], workloads.DEMO_K)


@pytest.mark.parametrize("n,k", [(100_003, 1000), (1 << 20, 10_000), (2_500_001, 25_000), (8192 * 3 + 77, 245)])
def test_deferred_sizes_three_steps(gc, n, k):
    grads = [(workloads.bucket(n, seed=30 + t) * F32(1.0 + t)).astype(F32) for t in range(3)]
    pure_steps(gc, grads, k)


def test_deferred_forced_fallback_small_call(gc):
    # the same at 2^20 elements, where the one-block select runs over the full c
    n = 1 << 20
    g = np.full(n, 1.0, F32)
    g[300_000:300_007] = 2.0
    pure_steps(gc, [g, g], 100_000)


def test_deferred_forced_fallback(gc):
    # a huge tie block: the candidates overflow and the exact fallback records the kept
    # offsets and per-tile counts itself
    n = 3_000_000
    g = np.full(n, 1.0, F32)
    g[1_000_000:1_000_010] = 2.0
    pure_steps(gc, [g, g], 500_000)


def test_deferred_layered_three_steps_with_qsgd(gc):
    n_layers, layer_len = 32, 65_537
    n = n_layers * layer_len
    r = np.zeros(n, F32)
    rd = dev(r)
    pend = gc.pending_record(n, n // 100, "cuda")
    for t in (1, 2, 3):
        g, _ = workloads.big_layers_host(n_layers, layer_len, step=t)
        k = n // 100
        o_idx, o_codes, o_norms, o_res, o_val = oracle.ef_topk_qsgd(g, r, k, levels=127, group=64, seed=500 + t)
        idx, codes, norms, val = gc.ef_topk_deferred(dev(g), rd, k, pend, qsgd_levels=127, qsgd_group=64,
                                                     qsgd_seed=500 + t)
        assert_bits_equal(host(idx), o_idx, f"step {t} idx")
        assert_bits_equal(host(val), o_val, f"step {t} values")
        assert_bits_equal(host(codes), o_codes, f"step {t} codes")
        assert_bits_equal(host(norms), o_norms, f"step {t} norms")
        r = o_res
    gc.ef_flush(rd, pend)
    assert_bits_equal(host(rd), r, "flushed residual")
    gc.ef_flush(rd, pend)                      # the record is empty now: nothing changes
    assert_bits_equal(host(rd), r, "second flush")


def test_deferred_varying_k_and_zero_k(gc):
    n = 200_003
    grads = [workloads.bucket(n, seed=40 + t) for t in range(4)]
    ks = [2000, 500, 0, 3000]
    rd = dev(np.zeros(n, F32))
    pend = gc.pending_record(n, max(ks), "cuda")
    r = np.zeros(n, F32)
    for t, (g, k) in enumerate(zip(grads, ks)):
        o_idx, o_val, o_res = oracle.ef_topk(g, r, k)
        idx, val = gc.ef_topk_deferred(dev(g), rd, k, pend)
        assert_bits_equal(host(idx), o_idx, f"step {t} idx")
        assert_bits_equal(host(val), o_val, f"step {t} values")
        if k == 0:   # applies the record: the residual is exact and the record empty
            assert_bits_equal(host(rd), o_res, f"step {t} residual after k = 0")
        r = o_res
    gc.ef_flush(rd, pend)
    assert_bits_equal(host(rd), r, "flushed residual")


def test_deferred_matches_direct_on_a_2e30_bucket(gc):
    # the deferred and the direct call on the same 2^30-element inputs, two steps of
    # Top-1% + QSGD-127: outputs identical, residual identical after the flush (the
    # direct call is itself held to the oracle by the EF Top-K parity tests)
    import torch
    n, k = 1 << 30, (1 << 30) // 100
    gen = torch.Generator(device="cuda").manual_seed(9)
    r_a = torch.zeros(n, dtype=torch.float32, device="cuda")
    r_b = torch.zeros_like(r_a)
    pend = gc.pending_record(n, k, "cuda")
    for t in range(2):
        g = workloads.student_t_torch(n, gen, "cuda") * (1e-3 * (t + 1))
        a = gc.ef_topk(g, r_a, k, qsgd_levels=127, qsgd_group=64, qsgd_seed=7 + t)
        b = gc.ef_topk_deferred(g, r_b, k, pend, qsgd_levels=127, qsgd_group=64, qsgd_seed=7 + t)
        for x, y, what in zip(a, b, ("idx", "codes", "norms", "values")):
            assert torch.equal(x.view(torch.int32) if x.dtype == torch.float32 else x,
                               y.view(torch.int32) if y.dtype == torch.float32 else y), f"step {t} {what}"
        del g
    gc.ef_flush(r_b, pend)
    assert torch.equal(r_a.view(torch.int32), r_b.view(torch.int32))
