"""GPU parity of the gradient-norm-ratio monitor (gc_ef_compress with stats) and of the
options it combines with (Random-K, deferred residual).

The selection, codes, norms and residual are compared bit for bit with the oracle; the
monitor's float64 sums are compared within the float64 rounding of a sum of n
non-negative terms: every partial order gives a relative error of at most
(n - 1) * 2^-53 against the exact sum, so two orders differ by at most twice that; the
tests use 1e-9, above that bound for every n here (n <= 2.1e6 gives 4.7e-10).
"""
import numpy as np
import pytest

import oracle
import workloads
from gc_testlib import assert_bits_equal

pytestmark = pytest.mark.gpu

F32 = np.float32
REL = 1e-9


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


def stats_close(got, want, what):
    for i, name in enumerate(("sum c^2", "sum g_hat^2", "ratio")):
        g, w = float(got[i]), float(want[i])
        assert abs(g - w) <= REL * abs(w) + 1e-300, f"{what} {name}: {g!r} vs {w!r}"


def new_stats():
    import torch
    return torch.full((3,), float("nan"), dtype=torch.float64, device="cuda")


@pytest.mark.parametrize("select", ["topk", "randk"])
@pytest.mark.parametrize("levels", [0, 127])
def test_monitor_one_step(gc, select, levels):
    g, _ = workloads.big_layers_host(8, 65_537, step=1)
    r = (workloads.bucket(g.size, seed=19) * F32(1e-4)).astype(F32)
    k = g.size // 100
    want, o_idx, o_res = oracle.monitored_step(g, r, k, levels=levels, group=64, qsgd_seed=5, select=select,
                                               select_seed=77)
    rd = dev(r)
    st = new_stats()
    out = gc.ef_compress(dev(g), rd, k, select=select, select_seed=77, stats=st, qsgd_levels=levels,
                         qsgd_group=64, qsgd_seed=5)
    assert_bits_equal(host(out[0]), o_idx, "idx")
    assert_bits_equal(host(rd), o_res, "residual")
    stats_close(host(st), want, f"{select} levels={levels}")


def test_monitor_deferred_three_steps_with_qsgd(gc):
    n_layers, layer_len = 32, 65_537
    n = n_layers * layer_len
    k = n // 100
    r = np.zeros(n, F32)
    rd = dev(r)
    pend = gc.pending_record(n, k, "cuda")
    st = new_stats()
    for t in (1, 2, 3):
        g, _ = workloads.big_layers_host(n_layers, layer_len, step=t)
        want, o_idx, o_res = oracle.monitored_step(g, r, k, levels=127, group=64, qsgd_seed=500 + t)
        idx, codes, norms, val = gc.ef_compress(dev(g), rd, k, pending=pend, stats=st, qsgd_levels=127,
                                                qsgd_group=64, qsgd_seed=500 + t)
        assert_bits_equal(host(idx), o_idx, f"step {t} idx")
        stats_close(host(st), want, f"step {t}")
        r = o_res
    gc.ef_flush(rd, pend)
    assert_bits_equal(host(rd), r, "flushed residual")


@pytest.mark.parametrize("levels", [0, 127])
def test_monitor_randk_deferred(gc, levels):
    # Random-K with the deferred residual (only reachable through the options), pure and
    # with QSGD on the kept values
    n, k = 1_500_007, 15_000
    r = np.zeros(n, F32)
    rd = dev(r)
    pend = gc.pending_record(n, k, "cuda")
    st = new_stats()
    for t in range(3):
        g = workloads.bucket(n, seed=60 + t)
        want, o_idx, o_res = oracle.monitored_step(g, r, k, levels=levels, group=64, qsgd_seed=70 + t,
                                                   select="randk", select_seed=900 + t)
        out = gc.ef_compress(dev(g), rd, k, select="randk", select_seed=900 + t, pending=pend, stats=st,
                             qsgd_levels=levels, qsgd_group=64, qsgd_seed=70 + t)
        assert_bits_equal(host(out[0]), o_idx, f"step {t} idx")
        stats_close(host(st), want, f"step {t}")
        r = o_res
    gc.ef_flush(rd, pend)
    assert_bits_equal(host(rd), r, "flushed residual")


def test_monitor_special_cases(gc):
    n = 50_001
    g = workloads.bucket(n, seed=3)
    st = new_stats()
    gc.ef_compress(dev(g), dev(np.zeros(n, F32)), n, stats=st)          # keep everything
    s = host(st)
    assert abs(s[2] - 1.0) <= REL and abs(s[0] - s[1]) <= REL * s[0]
    st = new_stats()
    gc.ef_compress(dev(np.zeros(n, F32)), dev(np.zeros(n, F32)), 10, stats=st)
    assert list(host(st)) == [0.0, 0.0, 1.0]


def test_monitor_matches_float64_torch_on_a_2e28_bucket(gc):
    # at 2^28 elements: sum c^2 against torch's float64 sum of the same c, and sum g_hat^2
    # against the float64 sum of the kept values (pure Top-1%)
    import torch
    n, k = 1 << 28, (1 << 28) // 100
    gen = torch.Generator(device="cuda").manual_seed(17)
    g = workloads.student_t_torch(n, gen, "cuda")
    r = workloads.student_t_torch(n, gen, "cuda") * 0.01
    c64 = (g + r).double()
    st = new_stats()
    idx, val = gc.ef_compress(g, r, k, stats=st)
    sc = float((c64 * c64).sum())
    sg = float((val.double() ** 2).sum())
    del c64
    s = host(st)
    # torch's own summation order rounds too; both are within (n - 1) 2^-53 of the exact sum
    tol = 2.0 * n * 2.0 ** -53
    assert abs(s[0] / sc - 1.0) <= tol and abs(s[1] / sg - 1.0) <= tol
    assert abs(s[2] / np.sqrt(sg / sc) - 1.0) <= tol


def test_norm_ratio_monitor_reads_one_step_behind(gc):
    import torch
    from gradient_compression_ddp_amd.adaptive import NormRatioMonitor
    n = 100_000
    g = workloads.bucket(n, seed=8)
    st = new_stats()
    mon = NormRatioMonitor()
    assert mon.poll() is None
    gc.ef_compress(dev(g), dev(np.zeros(n, F32)), 1000, stats=st)
    mon.record(st)
    torch.cuda.synchronize()
    got = mon.poll()
    assert got is not None and got == tuple(float(x) for x in host(st))
