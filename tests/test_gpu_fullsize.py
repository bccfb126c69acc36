"""Parity at the full workload sizes, in the launch configuration bench.py times.

The oracle cannot sort 7e9 elements, so:
* the Top-K set is checked with the exact O(n) invariant, evaluated with torch on the
  GPU (an independent library), layer by layer;
* every QSGD code and norm of the 7e7 kept values, and the residual at every kept
  position, are compared bit for bit with the oracle on the host;
* TernGrad at 350M elements: scales against torch's max|x|, codes of sampled runs of
  every layer against the oracle.
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
    import gradient_compression_ddp_amd as lib
    return lib


def keys(t):
    import torch
    return t.view(torch.int32) & 0x7FFFFFFF


@pytest.mark.parametrize("mode", ["direct", "deferred"])
def test_metric_path_7e9_two_steps(gc, mode):
    # deferred: the call bench.py times (gc_ef_compress with a pending record); the true
    # residual before a step is rebuilt by flushing copies of the residual and the record
    import torch
    dev = torch.device("cuda:0")
    L, LL = workloads.BIG_LAYERS, workloads.BIG_LAYER_LEN
    n, k = L * LL, workloads.BIG_K
    g = torch.empty(n, dtype=torch.float32, device=dev)
    r = torch.zeros(n, dtype=torch.float32, device=dev)
    r_prev = torch.empty_like(r)
    out_idx = torch.empty(k, dtype=torch.int64, device=dev)
    out_codes = torch.empty(k, dtype=torch.int8, device=dev)
    out_norms = torch.empty((k + 63) // 64, dtype=torch.float32, device=dev)
    ws = torch.empty(gc.workspace_size(gc.OP_EF_TOPK, n, k, 127), dtype=torch.uint8, device=dev)
    pend = gc.pending_record(n, k, dev) if mode == "deferred" else None
    for t in (1, 2):
        workloads.layered_torch(L, LL, step=t, device=dev, out=g)
        r_prev.copy_(r)
        if pend is not None:
            gc.ef_flush(r_prev, pend.clone())
        gc.ef_compress(g, r, k, pending=pend, qsgd_levels=127, qsgd_group=64, qsgd_seed=500 + t,
                       out_idx=out_idx, out_codes=out_codes, out_norms=out_norms, want_values=False, workspace=ws)
        torch.cuda.synchronize()
        idx = out_idx
        assert int(idx[0]) >= 0 and int(idx[-1]) < n
        assert bool((idx[1:] > idx[:-1]).all()), "indices not strictly ascending"
        v = g[idx] + r_prev[idx]                       # c at the kept positions
        kv = keys(v)
        T = int(kv.min())
        i_star = int(idx[kv == T].max())
        kept_gt = int((kv > T).sum())
        kept_eq = int((kv == T).sum())
        # exact invariant over all n: nothing dropped is above T, and no dropped tie precedes i*
        gt = eq_before = 0
        for l in range(L):
            sl = slice(l * LL, (l + 1) * LL)
            c = g[sl] + r_prev[sl]
            kc = keys(c)
            gt += int((kc > T).sum())
            pos = torch.arange(l * LL, (l + 1) * LL, device=dev)
            eq_before += int(((kc == T) & (pos <= i_star)).sum())
            del c, kc, pos
        assert gt == kept_gt, f"step {t}: {gt - kept_gt} dropped entries exceed the threshold"
        assert eq_before == kept_eq, f"step {t}: a dropped tie precedes a kept one"
        # the residual equals c everywhere off the kept set (deferred: everywhere, the kept
        # set's residual waiting in the record)
        mask = torch.ones(n, dtype=torch.bool, device=dev)
        if pend is None:
            mask[idx] = False
        for l in range(L):
            sl = slice(l * LL, (l + 1) * LL)
            c = g[sl] + r_prev[sl]
            m = mask[sl]
            assert torch.equal(r[sl][m].view(torch.int32), c[m].view(torch.int32)), f"residual off the kept set, layer {l}"
            del c, m
        del mask
        # QSGD of every kept value and the residual at the kept positions, against the oracle
        v_h = v.cpu().numpy()
        codes, norms, ghat, _ = oracle.qsgd(v_h, 64, 127, seed=500 + t)
        assert_bits_equal(out_codes.cpu().numpy(), codes, f"step {t} codes")
        assert_bits_equal(out_norms.cpu().numpy(), norms, f"step {t} norms")
        if pend is None:
            kept_res = r[idx]
        else:
            r_chk = r.clone()
            gc.ef_flush(r_chk, pend.clone())
            kept_res = r_chk[idx]
            del r_chk
        assert_bits_equal(kept_res.cpu().numpy(), (v_h - ghat).astype(F32), f"step {t} kept residual")
        del v, kv


def test_terngrad_350m(gc):
    import torch
    dev = torch.device("cuda:0")
    L, LL = workloads.TERN_LAYERS, workloads.TERN_LAYER_LEN
    x = workloads.layered_torch(L, LL, step=0, device=dev, seed=3)
    off = np.arange(L + 1, dtype=np.int64) * LL
    packed, scales = gc.terngrad(x, off, 3)
    torch.cuda.synchronize()
    nb = (LL + 3) // 4
    assert packed.numel() == L * nb
    want_scales = torch.stack([x[l * LL:(l + 1) * LL].abs().max() for l in range(L)])
    assert_bits_equal(scales.cpu().numpy(), want_scales.cpu().numpy(), "scales")
    p = packed.cpu().numpy()
    assert not np.any(((p[:, None] >> np.array([0, 2, 4, 6], np.uint8)) & 3) == 2)
    rng = np.random.default_rng(0)
    sc = scales.cpu().numpy()
    for l in range(L):
        starts = np.concatenate([[0, nb - 64], rng.integers(0, nb - 64, 8)]) * 4
        for s0 in starts:
            lo = l * LL + int(s0)
            hi = min(lo + 256, (l + 1) * LL)
            xs = x[lo:hi].cpu().numpy()
            # a trailing +scale element pins the oracle's per-segment scale to the layer's
            probe = np.concatenate([xs, [sc[l]]]).astype(F32)
            _, _, codes, _, _ = oracle.terngrad(probe, [0, probe.size], seed=3, index_base=lo)
            want = oracle.pack_ternary(codes[:-1])
            b0 = int(s0) // 4
            got = p[l * nb + b0: l * nb + b0 + want.size]
            if hi == (l + 1) * LL:
                want = want[:got.size]
            assert_bits_equal(got, want, f"layer {l} bytes from {b0}")
