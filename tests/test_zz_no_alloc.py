"""gc_ef_compress_noalloc against gc_ef_compress (GPU, through the C ABI).

The no-allocation entry point runs the same pipeline in the library's fixed per-GPU
array instead of a caller workspace.  Its outputs (indices, values, QSGD codes and
norms, the residual, the pending record, the norm monitor) must equal the workspace
entry point's bit for bit, on two calls in a row whose second is smaller, so that the
second call runs over what the first left in the array.  Its host-side refusal of calls
beyond the array is tested without a GPU in test_capi.py.
"""
import numpy as np
import pytest

import workloads
from gc_testlib import assert_bits_equal

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gc():
    import gradient_compression_ddp_amd as lib
    return lib


def host(t):
    return t.cpu().numpy()


def run(gc, fn, g, r, k, pend, stats, **kw):
    import torch
    dev = g.device
    out_idx = torch.empty(k, dtype=torch.int64, device=dev)
    out_val = torch.empty(k, dtype=torch.float32, device=dev)
    levels = kw.get("qsgd_levels", 0)
    group = kw.get("qsgd_group", 64)
    extra = {}
    if levels:
        extra = dict(out_codes=torch.empty(k, dtype=torch.int8, device=dev),
                     out_norms=torch.empty((k + group - 1) // group, dtype=torch.float32, device=dev))
    outs = fn(g, r, k, out_idx=out_idx, out_val=out_val, pending=pend, stats=stats, **extra, **kw)
    torch.cuda.synchronize()
    return [host(t) for t in outs if t is not None]


CASES = [
    dict(select="topk", qsgd_levels=127, qsgd_group=64, qsgd_seed=501, deferred=True, monitor=False),
    dict(select="topk", qsgd_levels=0, deferred=False, monitor=True),
    dict(select="randk", select_seed=9, qsgd_levels=15, qsgd_group=64, qsgd_seed=7, deferred=False, monitor=False),
    dict(select="topk", qsgd_levels=127, qsgd_group=128, qsgd_seed=3, deferred=True, monitor=True),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_noalloc_matches_workspace_call(gc, case):
    import torch
    dev = torch.device("cuda:0")
    opt = dict(CASES[case])
    deferred = opt.pop("deferred")
    monitor = opt.pop("monitor")
    # first call: a 25 MiB bucket at k = 1%; second: a smaller, ragged one at k = 3%
    for n, k, seed in ((workloads.BUCKET_N, workloads.BUCKET_N // 100, 2), (1_000_003, 30_011, 5)):
        print(f"[noalloc] case {case} n={n} k={k}", flush=True)
        g = torch.from_numpy(workloads.bucket(n, seed=seed)).to(dev)
        r0 = torch.from_numpy((workloads.bucket(n, seed=seed + 100) * np.float32(1e-2)).astype(np.float32)).to(dev)
        results = []
        for fn in (gc.ef_compress, gc.ef_compress_noalloc):
            r = r0.clone()
            pend = gc.pending_record(n, k, dev) if deferred else None
            stats = torch.zeros(3, dtype=torch.float64, device=dev) if monitor else None
            outs = []
            for step in range(2):                  # two steps: the second applies the first's record
                outs += run(gc, fn, g, r, k, pend, stats, **opt)
            if pend is not None:
                outs.append(host(pend))
                gc.ef_flush(r, pend)
            outs.append(host(r))
            if stats is not None:
                outs.append(host(stats))
            results.append(outs)
        want, got = results
        assert len(want) == len(got)
        for j, (a, b) in enumerate(zip(got, want)):
            assert_bits_equal(a, b, f"case {case} n={n} output {j}")
