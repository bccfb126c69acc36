"""EF Top-K / Random-K on inputs of about 2^25 elements, bit for bit against the oracle.

The library bounds the k-th key from a sample, extracts candidates in the streaming
pass, selects over the candidate pool, and falls back to the full c when the
candidates cannot hold the answer.  The ordered emit finds each work item's output
position by look-back when the items are few (up to two per compute unit), and from a
separate count and scan when they are many.  With 256 compute units, 2^25 elements
make 512 items (look-back) and 2^25 + 1 make 513 (count and scan), so these sizes
straddle that switch.  Each case also reads back which source the selection used (the
candidates, or the full c of the fallback), so both are compared element by element
with the oracle.
"""
import numpy as np
import pytest

import oracle
import workloads
from gc_testlib import assert_bits_equal

pytestmark = pytest.mark.gpu

F32 = np.float32
N_LARGE = (1 << 25) + 28_693          # just above the switch; not a multiple of the 4096 tile


@pytest.fixture(scope="module")
def gc():
    import gradient_compression_ddp_amd as lib
    return lib


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def host(t):
    return t.cpu().numpy()


def workspace(gc, op, n, k, levels=0):
    import torch
    return torch.empty(gc.workspace_size(op, n, k, levels), dtype=torch.uint8, device="cuda:0")


def mode_of(ws):
    # the control block opens the workspace; its third 32-bit word is the source of the
    # selection: 0 the candidate pool, 1 the full c
    return int(host(ws[8:12]).view(np.uint32)[0])


def inputs(n, seed):
    g = workloads.bucket(n, seed=seed)
    r = (workloads.bucket(n, seed=seed + 1) * F32(0.1)).astype(F32)
    return g, r


@pytest.mark.parametrize("n,k", [(N_LARGE, N_LARGE // 100), (N_LARGE, 7), ((1 << 25) + 1, 1 << 18),
                                 (1 << 25, (1 << 25) // 100)])
def test_topk_two_steps_direct(gc, n, k):
    print(f"[large] direct n={n} k={k}", flush=True)
    g, r = inputs(n, 41)
    rd = dev(r)
    for step in (1, 2):
        if step == 2:
            g = (g * F32(0.9)).astype(F32)
        o_idx, o_val, o_res = oracle.ef_topk(g, r, k)
        ws = workspace(gc, gc.OP_EF_TOPK, n, k)
        idx, val = gc.ef_topk(dev(g), rd, k, workspace=ws)
        assert_bits_equal(host(idx), o_idx, f"step {step} idx")
        assert_bits_equal(host(val), o_val, f"step {step} values")
        assert_bits_equal(host(rd), o_res, f"step {step} residual")
        assert mode_of(ws) == 0
        r = o_res


def test_topk_deferred_with_qsgd_three_steps(gc):
    import torch
    n, k = N_LARGE, N_LARGE // 100
    print(f"[large] deferred qsgd n={n} k={k}", flush=True)
    g, r = inputs(n, 43)
    rd = dev(r)
    pend = gc.pending_record(n, k, torch.device("cuda:0"))
    for step in (1, 2, 3):
        gs = (g * F32(1.0 + 0.25 * step)).astype(F32)
        o_idx, o_codes, o_norms, o_res, o_val = oracle.ef_topk_qsgd(gs, r, k, levels=127, group=64, seed=500 + step)
        idx, codes, norms, val = gc.ef_topk_deferred(dev(gs), rd, k, pend, qsgd_levels=127, qsgd_group=64,
                                                     qsgd_seed=500 + step)
        assert_bits_equal(host(idx), o_idx, f"step {step} idx")
        assert_bits_equal(host(val), o_val, f"step {step} values")
        assert_bits_equal(host(codes), o_codes, f"step {step} codes")
        assert_bits_equal(host(norms), o_norms, f"step {step} norms")
        r = o_res
    gc.ef_flush(rd, pend)
    assert_bits_equal(host(rd), r, "flushed residual")


def test_topk_deferred_qsgd_without_values_three_steps(gc):
    # the call the metric path makes, at a size that takes the batch emit: no kept values
    # requested (they only pass through the staging array to the streaming QSGD pass);
    # codes, norms and the flushed residual must be the oracle's
    import torch
    n, k = N_LARGE, N_LARGE // 100
    print(f"[large] deferred qsgd, no values n={n} k={k}", flush=True)
    g, r = inputs(n, 47)
    rd = dev(r)
    pend = gc.pending_record(n, k, torch.device("cuda:0"))
    ws = workspace(gc, gc.OP_EF_TOPK, n, k, 127)
    for step in (1, 2, 3):
        gs = (g * F32(1.0 + 0.25 * step)).astype(F32)
        o_idx, o_codes, o_norms, o_res, _ = oracle.ef_topk_qsgd(gs, r, k, levels=127, group=64, seed=700 + step)
        idx, codes, norms, val = gc.ef_topk_deferred(dev(gs), rd, k, pend, qsgd_levels=127, qsgd_group=64,
                                                     qsgd_seed=700 + step, want_values=False, workspace=ws)
        assert val is None
        assert mode_of(ws) == 0
        assert_bits_equal(host(idx), o_idx, f"step {step} idx")
        assert_bits_equal(host(codes), o_codes, f"step {step} codes")
        assert_bits_equal(host(norms), o_norms, f"step {step} norms")
        r = o_res
    gc.ef_flush(rd, pend)
    assert_bits_equal(host(rd), r, "flushed residual")


def test_topk_deferred_qsgd_without_values_fallback(gc):
    # the same call when the selection falls back to the full c (the fallback emit stages
    # the kept values for the streaming QSGD pass)
    import torch
    n, k = N_LARGE, N_LARGE // 5
    print(f"[large] deferred qsgd fallback, no values n={n} k={k}", flush=True)
    g = np.full(n, -0.5, F32)
    g[::1001] = 0.75
    g[::7919] = 1.25
    r = np.zeros(n, F32)
    rd = dev(r)
    pend = gc.pending_record(n, k, torch.device("cuda:0"))
    ws = workspace(gc, gc.OP_EF_TOPK, n, k, 127)
    for step in (1, 2):
        o_idx, o_codes, o_norms, o_res, _ = oracle.ef_topk_qsgd(g, r, k, levels=127, group=64, seed=900 + step)
        idx, codes, norms, val = gc.ef_topk_deferred(dev(g), rd, k, pend, qsgd_levels=127, qsgd_group=64,
                                                     qsgd_seed=900 + step, want_values=False, workspace=ws)
        assert mode_of(ws) == 1
        assert_bits_equal(host(idx), o_idx, f"step {step} idx")
        assert_bits_equal(host(codes), o_codes, f"step {step} codes")
        assert_bits_equal(host(norms), o_norms, f"step {step} norms")
        r = o_res
    gc.ef_flush(rd, pend)
    assert_bits_equal(host(rd), r, "flushed residual")


def test_topk_forced_fallback(gc):
    # a huge tie block defeats the sampled bound: every element is a candidate, the pool
    # overflows, and the selection and the emit run over the full c
    n, k = N_LARGE, N_LARGE // 6
    print(f"[large] fallback n={n} k={k}", flush=True)
    g = np.full(n, 1.0, F32)
    g[10_000_000:10_000_010] = 2.0
    g[20_000_000:20_000_003] = -3.0
    r = np.zeros(n, F32)
    o_idx, o_val, o_res = oracle.ef_topk(g, r, k)
    rd = dev(r)
    ws = workspace(gc, gc.OP_EF_TOPK, n, k)
    idx, val = gc.ef_topk(dev(g), rd, k, workspace=ws)
    assert_bits_equal(host(idx), o_idx, "idx")
    assert_bits_equal(host(val), o_val, "values")
    assert_bits_equal(host(rd), o_res, "residual")
    assert mode_of(ws) == 1


def test_topk_forced_fallback_deferred(gc):
    import torch
    n, k = N_LARGE, N_LARGE // 5
    print(f"[large] fallback deferred n={n} k={k}", flush=True)
    g = np.full(n, -0.5, F32)
    g[::1001] = 0.75
    r = np.zeros(n, F32)
    rd = dev(r)
    pend = gc.pending_record(n, k, torch.device("cuda:0"))
    for step in (1, 2):
        o_idx, o_val, o_res = oracle.ef_topk(g, r, k)
        ws = workspace(gc, gc.OP_EF_TOPK, n, k)
        idx, val = gc.ef_topk_deferred(dev(g), rd, k, pend, workspace=ws)
        assert_bits_equal(host(idx), o_idx, f"step {step} idx")
        assert_bits_equal(host(val), o_val, f"step {step} values")
        assert mode_of(ws) == 1
        r = o_res
    gc.ef_flush(rd, pend)
    assert_bits_equal(host(rd), r, "flushed residual")


@pytest.mark.parametrize("fill", ["ones", "random"])
def test_topk_workspace_of_other_data(gc, fill):
    # The workspace holds whatever its memory held before (here all ones, or random
    # bytes): the control block, the counters and the pool are set by the call itself
    # before they are read, so both calls are exact and take the candidate path.
    import torch
    n, k = N_LARGE, N_LARGE // 100
    print(f"[large] workspace of other data ({fill}) n={n} k={k}", flush=True)
    g, r = inputs(n, 53)
    rd = dev(r)
    ws = workspace(gc, gc.OP_EF_TOPK, n, k)
    if fill == "ones":
        ws.fill_(255)
    else:
        gen = torch.Generator(device="cuda:0").manual_seed(5)
        ws.copy_(torch.randint(0, 256, ws.shape, generator=gen, device="cuda:0", dtype=torch.int32).to(torch.uint8))
    for step in (1, 2):
        if step == 2:
            g = (g * F32(0.9)).astype(F32)
        o_idx, o_val, o_res = oracle.ef_topk(g, r, k)
        idx, val = gc.ef_topk(dev(g), rd, k, workspace=ws)
        assert_bits_equal(host(idx), o_idx, f"step {step} idx")
        assert_bits_equal(host(val), o_val, f"step {step} values")
        assert_bits_equal(host(rd), o_res, f"step {step} residual")
        assert mode_of(ws) == 0
        r = o_res


@pytest.mark.parametrize("k,mode", [(N_LARGE // 100, 0), (N_LARGE, 1)])
def test_randk_with_qsgd(gc, k, mode):
    # k = n: some keys fall below the smallest of the 2^19 sampled keys, so the candidates
    # cannot hold all n and the selection runs over every key
    n = N_LARGE
    print(f"[large] randk n={n} k={k}", flush=True)
    g, r = inputs(n, 47)
    o_idx, o_codes, o_norms, o_res, o_val = oracle.ef_randk_qsgd(g, r, k, 77, levels=15, group=64, qsgd_seed=9,
                                                                 index_base=3)
    rd = dev(r)
    ws = workspace(gc, gc.OP_EF_RANDK, n, k, 15)
    idx, codes, norms, val = gc.ef_randk(dev(g), rd, k, 77, index_base=3, qsgd_levels=15, qsgd_group=64,
                                         qsgd_seed=9, workspace=ws)
    assert mode_of(ws) == mode
    assert_bits_equal(host(idx), o_idx, "idx")
    assert_bits_equal(host(val), o_val, "values")
    assert_bits_equal(host(codes), o_codes, "codes")
    assert_bits_equal(host(norms), o_norms, "norms")
    assert_bits_equal(host(rd), o_res, "residual")
