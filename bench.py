"""Benchmark: fused error-feedback Top-1% + 8-bit QSGD on a 7e9-element fp32 gradient.

One step = one deferred EF Top-K call (gc_ef_compress with a pending record, which is
gc_ef_topk_deferred) with QSGD (s = 127, groups of 64) over the whole flat gradient: c = g + r with the previous step's kept-set residuals applied in the same
pass, exact Top-k (k = 1% = 7e7), ordered compaction, QSGD of the kept values, and the
kept set's new residuals recorded for the next step.  The timed region ends with one
gc_ef_flush, so the K timed steps apply exactly K sets of kept-set residuals (the first
step applies the warm-up's) and the residual is exact when the clock stops.  --direct
times gc_ef_topk instead, which scatters the kept set's residuals inside each call;
--monitor adds the gradient-norm-ratio monitor to every step.
Inputs live in HBM before the timed region starts.

Workload (synthetic, generated on the GPU): 32 layers of 218,750,000 elements, each
t(3) times a per-layer lognormal(-7, 1) scale; three step gradients g_1..g_3 (step t
cycles through them), the residual carried from step to step starting at 0, QSGD seed
500 + t.

Printed: one JSON line.  value = input fp32 GB/s (4 n bytes per step / step time);
ms_per_step = the bracketed wall time of the K steps (and the final flush) / K, with each
step's own event time summarised as median, p10 and p90; roofline = the streaming pass
(the dominant kernel), 12 algorithmic bytes per element (read g and r, write c), timed with
HIP events recorded by the library on the launch stream inside the timed region, the
deferred record's bytes reported apart; cpu_baseline = the numpy oracle on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# Non-packed 32-bit VALU issue ceiling: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz.
VALU_PEAK_LANE_OPS = 256 * 4 * 16 * 2.4e9
# VALU lane-instructions per element of the quantizer kernels (SQ_INSTS_VALU x 64 /
# elements, rocprofv3 counters of bench.py --rows; profiles/compressor_rows_valu_and_traffic.md).
VALU_LANE_OPS_PER_ELEMENT = {"minmax8": 20.4, "minmax4": 20.7, "qsgd": 33.9, "terngrad": 23.0}
# Issue slots beyond one per instruction: v_mad_u64_u32 (the Philox4x32-10 multiplies, 20
# of the about 66 instructions of a block of 4 draws) occupies a SIMD for two full-rate
# slots (a kernel of Philox blocks alone measured 5.4 cycles per wave instruction against
# 4 for a full-rate one).  QSGD draws one block per quad; TernGrad one per quad in its
# pass and two per listed byte (3.7M of 87.5M) in the fix-up.
VALU_EXTRA_SLOTS_PER_ELEMENT = {"minmax8": 0.0, "minmax4": 0.0, "qsgd": 5.0, "terngrad": 5.4}

# HBM bytes per launch of the streaming pass on this workload, from two rocprofv3 counter
# runs per mode (FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0, factors from a plain 4 GiB device
# copy; the summary with its commands is profiles/k_ef_cand_7e9_hbm_traffic.md).  Valid
# only for the kernel source it was measured on: the digest covers the tile constants,
# the pending-record helpers, the block-rank helpers and the kernel itself, and a
# mismatch reports the traffic as null.
K1_TRAFFIC_BYTES = {"deferred": 8.5796e10, "direct": 8.4686e10}
K1_SOURCE_SHA256 = "35046b14518c4a6ace07d95c6b469706ed67610f0179bfc21cefd1f266233267"
METRIC = "EF-Top-1%+int8 compress GB/s of fp32 grad input; % of HBM peak"


def k1_source_digest():
    """SHA-256 of the text the streaming pass is built from: the tile constants it uses,
    the block-rank helpers and the kernel itself."""
    import hashlib
    import re
    src = open(os.path.join(ROOT, "gradient_compression_ddp_amd", "csrc", "ef_topk.hip")).read()
    parts = [m.group(0) for m in re.finditer(r"^constexpr \w+ (kBlock|kWaves|kRounds|kTile|kRegions) = .*$",
                                             src, re.M)]
    for start, end in (("struct PendHdr {", "// Block-level ordered ranking"),
                       ("__device__ __forceinline__ uint32_t rank_round", "// Kernels"),
                       ("void k_ef_cand(", "\n}\n")):
        a = src.index(start)
        parts.append(src[a:src.index(end, a)])
    return hashlib.sha256("\n".join(parts).encode()).hexdigest()


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=32)
    ap.add_argument("--layer-len", type=int, default=218_750_000)
    ap.add_argument("--ratio", type=float, default=0.01)
    ap.add_argument("--cpu-sample-log2", type=int, default=27,
                    help="elements in the oracle's sample (2^N, split over the same 32 layers)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calibration-gib", type=float, default=0.0,
                    help="run one device-to-device copy of this many GiB before the timed region "
                         "(a plain copy of known size for calibrating HBM byte counters)")
    ap.add_argument("--direct", action="store_true",
                    help="time gc_ef_topk (kept-set residuals scattered inside each call) instead of "
                         "gc_ef_topk_deferred + a final gc_ef_flush")
    ap.add_argument("--monitor", action="store_true",
                    help="also run the gradient-norm-ratio monitor in every step (gc_ef_compress stats)")
    ap.add_argument("--rows", action="store_true",
                    help="instead of the metric line, print one JSON line per compressor: each "
                         "timed on the GPU against the HBM roofline, with the oracle timed beside it")
    return ap.parse_args()


def cpu_baseline(args, n_layers):
    """Time the oracle (as it stands) on a bounded sample of the same workload."""
    import numpy as np
    import oracle
    import workloads
    n_s = 1 << args.cpu_sample_log2
    layer_len = n_s // n_layers
    g, _ = workloads.big_layers_host(n_layers, layer_len, step=1)
    r = np.zeros_like(g)
    k = int(g.size * args.ratio)
    t0 = time.perf_counter()
    oracle.ef_topk_qsgd(g, r, k, levels=127, group=64, seed=501)
    dt = time.perf_counter() - t0
    n_full = args.layers * args.layer_len
    return {
        "value": round(4.0 * g.size / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": 1,
        "cpus_usable": len(os.sched_getaffinity(0)),
        "cpus_host": os.cpu_count(),
        "kind": "oracle",
        "sample_fraction": round(g.size / n_full, 5),
        "sample": (f"{g.size} elements ({n_layers} layers x {layer_len}) of the same layered t(3) x "
                   f"lognormal recipe drawn on the host, k = {k} (1%), one EF-Top-k + QSGD-127 step; "
                   f"{dt:.2f} s in one thread (numpy elementwise work and sort run single-threaded)"),
    }

# ---------------------------------------------------------------------------
# Per-compressor lines (--rows).  Each op runs on its own workload from the
# seeded generators; the GPU side is timed with events on the launch stream
# (single calls eagerly, back-to-back throughput as a replayed HIP graph of
# several calls on distinct buffers, so that launch overhead does not hide the
# kernels), and the oracle is timed beside it on the same (or a sampled) input.
# ---------------------------------------------------------------------------

def _median(xs):
    xs = sorted(xs)
    return xs[len(xs) // 2]


def _eager_ms(torch, fn, reps=30, before=None):
    """Median over reps of one call bracketed by events (before() runs outside them)."""
    for _ in range(3):
        if before:
            before()
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        if before:
            before()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b))
    return _median(ts)


def _graph_ms(torch, fn_list, reps=7):
    """Capture the calls in one graph, replay it reps times; median ms per call."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for fn in fn_list:
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    try:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for fn in fn_list:
                fn()
        torch.cuda.synchronize()
        run = g.replay
    except RuntimeError as e:          # capture refused: time the same calls eagerly
        print(f"[rows] graph capture failed ({e}); timing eager back-to-back calls", file=sys.stderr)
        torch.cuda.synchronize()

        def run():
            for fn in fn_list:
                fn()
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        run()
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b))
    return _median(ts) / len(fn_list), run


def _oracle_s(fn):
    t0 = time.perf_counter()
    fn()
    return time.perf_counter() - t0


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max((i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"),
                   default=1)
    except Exception:
        return None


def _row(name, workload, unit_bytes, unit, gpu_ms, eager_ms, oracle_s=None, oracle_units=1.0,
         sample="", cores=1, extra=None, valu_ops=None):
    achieved = unit_bytes / (gpu_ms / 1e3) / 1e9
    line = {
        "row": name, "workload": workload, "unit": unit,
        "algorithmic_bytes_per_unit": unit_bytes,
        "ms_per_unit": round(gpu_ms, 5), "eager_call_ms": round(eager_ms, 5),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)},
    }
    if oracle_s is not None:
        per_unit = oracle_s / oracle_units
        line["cpu_oracle"] = {"s_per_unit": round(per_unit, 4), "cores": cores, "kind": "oracle",
                              "sample": sample, "gpu_speedup": round(per_unit * 1e3 / gpu_ms, 1)}
    if valu_ops is not None:
        # the counted VALU work of the unit against the issue ceiling (a utilisation figure
        # for the rows whose arithmetic, not HBM, sets the pace)
        rate = valu_ops / (gpu_ms / 1e3)
        line["valu_issue"] = {"lane_ops_per_unit": valu_ops, "achieved": round(rate / 1e12, 2),
                              "peak": round(VALU_PEAK_LANE_OPS / 1e12, 2), "unit": "1e12 lane-ops/s",
                              "frac": round(rate / VALU_PEAK_LANE_OPS, 4)}
    if extra:
        line.update(extra)
    print(json.dumps(line), flush=True)


def ddp_hook_row(torch, gc, dev, say):
    import socket
    import torch.distributed as dist
    from torch.nn.parallel import DistributedDataParallel as DDP
    from gradient_compression_ddp_amd.ddp_hook import CompressionHookState, ef_compress_hook
    say("DDP hook, world size 1")
    with socket.socket() as sk:
        sk.bind(("127.0.0.1", 0))
        port = sk.getsockname()[1]
    # the collective library prints a banner to stdout when its communicator starts: keep
    # stdout for the JSON lines by pointing fd 1 at stderr while the row runs
    sys.stdout.flush()
    saved_fd = os.dup(1)
    os.dup2(2, 1)
    dist.init_process_group("nccl", init_method=f"tcp://127.0.0.1:{port}", rank=0, world_size=1)
    try:
        def build(hook, overlap=True):
            torch.manual_seed(0)
            layers = []
            for _ in range(6):
                layers += [torch.nn.Linear(4096, 4096), torch.nn.ReLU()]
            m = DDP(torch.nn.Sequential(*layers).to(dev), device_ids=[0], bucket_cap_mb=25,
                    gradient_as_bucket_view=True)
            state = None
            if hook:
                state = CompressionHookState(ratio=0.01, qsgd_levels=127, deferred=True, overlap=overlap)
                m.register_comm_hook(state, ef_compress_hook)
            return m, state

        x = torch.randn(64, 4096, device=dev)

        def it_ms(m):
            def f():
                m.zero_grad(set_to_none=False)
                m(x).square().mean().backward()
            return _eager_ms(torch, f, reps=20)
        m0, _ = build(False)
        base = it_ms(m0)
        del m0
        m1, state = build(True)
        hooked = it_ms(m1)
        n = sum(p.numel() for p in m1.parameters())
        nb = len(state.buckets)
        k = sum(b.k for b in state.buckets.values())
        del m1, state
        m2, _ = build(True, overlap=False)
        serial = it_ms(m2)
        del m2
    finally:
        dist.destroy_process_group()
        sys.stdout.flush()
        os.dup2(saved_fd, 1)
        os.close(saved_fd)
    # per iteration: the EF pass (12 B per element, + the record), the kept set's outputs,
    # and the receive (payload read, 4 B per element written)
    ub = 12.0 * n + k * (8.0 + 1.0 + 4.0 / 64 + 4.0 + 4.0 + 16.0) + 4.0 * n + k * (8.0 + 1.0 + 4.0 / 64)
    extra = max(hooked - base, 1e-6)
    _row("next-4 DDP comm hook, world size 1 (EF Top-1% + QSGD-127, deferred)",
         f"6 x Linear(4096, 4096), {n:,} parameters in {nb} buckets of <= 25 MiB, batch 64", ub,
         "iteration (time over DDP's own hook)", extra, extra,
         extra={"iteration_ms_allreduce_hook": round(base, 4), "iteration_ms_compression_hook": round(hooked, 4),
                "iteration_ms_compression_hook_same_stream": round(serial, 4)})


def rows_mode(args):
    import numpy as np
    import torch
    import gradient_compression_ddp_amd as gc
    import workloads
    orc = None
    if not args.no_cpu:
        import oracle as orc
    dev = torch.device("cuda:0")
    say = lambda m: print(f"[rows] {m}", file=sys.stderr, flush=True)

    # c1: EF Top-K on the 1e6 demo gradient, k = 1e4 (cache-resident; latency).
    g1, _ = workloads.ef_demo_gradients()
    n, k = g1.size, workloads.DEMO_K
    say("EF Top-K demo")
    gd = torch.from_numpy(g1).to(dev)
    r0 = torch.zeros_like(gd)
    rs = [torch.zeros_like(gd) for _ in range(8)]
    ws = torch.empty(gc.workspace_size(gc.OP_EF_TOPK, n, k, 0), dtype=torch.uint8, device=dev)
    oi = [torch.empty(k, dtype=torch.int64, device=dev) for _ in range(8)]
    ov = [torch.empty(k, dtype=torch.float32, device=dev) for _ in range(8)]
    r = torch.zeros_like(gd)
    eager = _eager_ms(torch, lambda: gc.ef_topk(gd, r, k, out_idx=oi[0], out_val=ov[0], workspace=ws),
                      before=lambda: r.copy_(r0))
    gms, _ = _graph_ms(torch, [lambda i=i: gc.ef_topk(gd, rs[i], k, out_idx=oi[i], out_val=ov[i], workspace=ws)
                               for i in range(8)])
    osec = _oracle_s(lambda: orc.ef_topk(g1, np.zeros_like(g1), k)) if orc else None
    _row("a1-a3 EF Top-K (pure)", f"n=1,000,000 N(0,1), k=10,000", 12.0 * n + 12.0 * k, "call", gms, eager,
         osec, 1.0, "the same 1e6 input")

    # c1: per-tensor int8 min-max on the demo gradient.
    say("min-max per tensor")
    ws_m = gc.workspace_size(gc.OP_QUANT_MINMAX, n, 0, 0)
    wsm = torch.empty(max(ws_m, 1), dtype=torch.uint8, device=dev)
    cm = torch.empty(n, dtype=torch.uint8, device=dev)
    mn = torch.empty(1, dtype=torch.float32, device=dev)
    sc = torch.empty(1, dtype=torch.float32, device=dev)
    f = lambda: gc.quant_minmax(gd, 0, 8, codes=cm, mins=mn, scales=sc, workspace=wsm)
    eager = _eager_ms(torch, f)
    gms, _ = _graph_ms(torch, [f] * 8)
    osec = _oracle_s(lambda: orc.quant_minmax(g1, 0, 8)) if orc else None
    _row("a4 min-max int8, per tensor", "n=1,000,000 N(0,1)", 5.0 * n + 8, "call", gms, eager, osec, 1.0,
         "the same 1e6 input")

    # c2: one 25 MiB bucket; 40 distinct copies for back-to-back throughput.
    NB = 40
    xb = workloads.bucket()
    n = xb.size
    ng = n // 64
    x40 = torch.from_numpy(xb).to(dev).repeat(NB)
    xs = [x40[i * n:(i + 1) * n] for i in range(NB)]
    # the size's floor: a pass that only reads the 4-byte inputs and writes one byte each
    say("floor: read 4 B, write 1 B per element")
    fl = torch.empty(NB * n, dtype=torch.uint8, device=dev)
    fns = [lambda i=i: gc.stream_floor(xs[i], fl[i * n:(i + 1) * n]) for i in range(NB)]
    eager = _eager_ms(torch, fns[0])
    gms, _ = _graph_ms(torch, fns)
    floor_ms = gms
    _row("a4-a6 floor: plain pass reading 4 B and writing 1 B per element", "25 MiB bucket, 40 buckets",
         5.0 * n, "bucket", gms, eager, None, 1.0, "one bucket")
    del fl

    for bits in (8, 4):
        say(f"min-max int{bits} gs64")
        nc = n if bits == 8 else (n + 1) // 2
        codes = torch.empty(NB * nc, dtype=torch.uint8, device=dev)
        mins = torch.empty(NB * ng, dtype=torch.float32, device=dev)
        scales = torch.empty(NB * ng, dtype=torch.float32, device=dev)
        wsz = gc.workspace_size(gc.OP_QUANT_MINMAX, n, 64, 0)
        wsb = torch.empty(max(wsz, 1), dtype=torch.uint8, device=dev)
        fns = [lambda i=i: gc.quant_minmax(xs[i], 64, bits, codes=codes[i * nc:(i + 1) * nc],
                                           mins=mins[i * ng:(i + 1) * ng], scales=scales[i * ng:(i + 1) * ng],
                                           workspace=wsb) for i in range(NB)]
        eager = _eager_ms(torch, fns[0])
        gms, _ = _graph_ms(torch, fns)
        osec = _oracle_s(lambda: orc.quant_minmax(xb, 64, bits)) if orc else None
        ub = (5.0 if bits == 8 else 4.5) * n + 8.0 * ng
        _row(f"a4 min-max int{bits}, groups of 64", "25 MiB bucket: n=6,553,600 t(3)*1e-3, 40 buckets",
             ub, "bucket", gms, eager, osec, 1.0, "one bucket", extra={"vs_floor": round(gms / floor_ms, 3)},
             valu_ops=(VALU_LANE_OPS_PER_ELEMENT[f"minmax{bits}"] + VALU_EXTRA_SLOTS_PER_ELEMENT[f"minmax{bits}"]) * n)

    say("QSGD s=15 gs64")
    qc = torch.empty(NB * n, dtype=torch.int8, device=dev)
    qn = torch.empty(NB * ng, dtype=torch.float32, device=dev)
    fns = [lambda i=i: gc.qsgd(xs[i], 64, 15, 7, 0, codes=qc[i * n:(i + 1) * n], norms=qn[i * ng:(i + 1) * ng])
           for i in range(NB)]
    eager = _eager_ms(torch, fns[0])
    gms, _ = _graph_ms(torch, fns)
    osec = _oracle_s(lambda: orc.qsgd(xb, 64, 15, 7)) if orc else None
    _row("a5+a6 QSGD s=15, groups of 64 (Philox4x32-10)", "25 MiB bucket, 40 buckets",
         5.0 * n + 4.0 * ng, "bucket", gms, eager, osec, 1.0, "one bucket", extra={"vs_floor": round(gms / floor_ms, 3)},
         valu_ops=(VALU_LANE_OPS_PER_ELEMENT["qsgd"] + VALU_EXTRA_SLOTS_PER_ELEMENT["qsgd"]) * n)

    say("receive: 8 QSGD payloads of one bucket, averaged")
    W = 8
    hq = gc.payload_layout(gc.KIND_QSGD, n, n, 64, 15)
    pays = [torch.zeros(hq.bytes, dtype=torch.uint8, device=dev) for _ in range(W)]
    for w in range(W):
        gc.write_payload_header(pays[w], hq)
        sec = gc.payload_sections(pays[w], hq)
        gc.qsgd(xs[w], 64, 15, 7 + w, codes=sec["codes"], norms=sec["meta0"])
    outs = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(4)]
    fns = [lambda i=i: gc.decompress_payloads(pays, [hq] * W, outs[i]) for i in range(4)]
    eager = _eager_ms(torch, fns[0])
    gms, _ = _graph_ms(torch, fns)
    osec = None
    if orc:
        hcodes = [gc.payload_sections(pays[w], hq)["codes"].cpu().numpy() for w in range(W)]
        hnorms = [gc.payload_sections(pays[w], hq)["meta0"].cpu().numpy() for w in range(W)]

        def o_recv():
            acc = np.zeros(n, np.float32)
            for w in range(W):
                orc.decompress_scatter(orc.KIND_QSGD, None, n, 0, hcodes[w], hnorms[w], None, 64, 15,
                                       np.float32(1.0 / W), True, acc)
        osec = _oracle_s(o_recv)
    _row("a9 receive: average of W=8 dense QSGD payloads (one pass)", "8 x 25 MiB-bucket payloads, s = 15",
         W * (1.0 * n + 4.0 * ng) + 4.0 * n, "call", gms, eager, osec, 1.0, "the same 8 payloads")
    del pays, outs

    say("decompress QSGD / min-max int8 dense")
    outb = torch.empty(NB * n, dtype=torch.float32, device=dev)
    fns = [lambda i=i: gc.decompress_scatter(gc.KIND_QSGD, qc[i * n:(i + 1) * n], n, outb[i * n:(i + 1) * n],
                                             meta0=qn[i * ng:(i + 1) * ng], group=64, levels=15)
           for i in range(NB)]
    eager = _eager_ms(torch, fns[0])
    gms, _ = _graph_ms(torch, fns)
    qc0, qn0 = qc[:n].cpu().numpy(), qn[:ng].cpu().numpy()
    osec = _oracle_s(lambda: orc.decompress_scatter(orc.KIND_QSGD, None, n, 0, qc0, qn0, None, 64, 15, 1.0,
                                                    False, np.empty(n, np.float32))) if orc else None
    _row("a9 decompress QSGD, dense", "25 MiB bucket of codes, 40 buckets", 5.0 * n + 4.0 * ng, "bucket",
         gms, eager, osec, 1.0, "one bucket")
    del x40, xs, codes, mins, scales, qc, qn, outb

    # a9 scatter: the pure Top-K payload of the demo gradient, accumulated into a dense buffer.
    say("scatter f32 payload")
    idx, val = gc.ef_topk(gd, torch.zeros_like(gd), k)
    outs = torch.zeros_like(gd)
    f = lambda: gc.decompress_scatter(gc.KIND_F32, val, k, outs, idx=idx, accumulate=True)
    eager = _eager_ms(torch, f)
    gms, _ = _graph_ms(torch, [f] * 8)
    i0, v0 = idx.cpu().numpy(), val.cpu().numpy()
    osec = _oracle_s(lambda: orc.decompress_scatter(orc.KIND_F32, i0, k, 0, v0, None, None, 0, 0, 1.0, True,
                                                    np.zeros(g1.size, np.float32))) if orc else None
    _row("a9 scatter-accumulate f32", "k=10,000 of n=1,000,000", 8.0 * k + 4.0 * k + 8.0 * k, "call",
         gms, eager, osec, 1.0, "the same payload")
    del gd, r0, rs, r, ws

    # a9 receive, sparse: 8 workers' EF-Top-1% + QSGD-127 payloads into one 1e8 vector.
    say("receive: 8 sparse Top-1% + QSGD-127 payloads")
    W, ns, ks = 8, 100_000_000, 1_000_000
    hs = gc.payload_layout(gc.KIND_QSGD, ns, ks, 64, 127, sparse=True)
    pays = [torch.zeros(hs.bytes, dtype=torch.uint8, device=dev) for _ in range(W)]
    wsk = torch.empty(gc.workspace_size(gc.OP_EF_TOPK, ns, ks, 127), dtype=torch.uint8, device=dev)
    for w in range(W):
        gw = workloads.layered_torch(4, ns // 4, step=w, device=dev, seed=9)
        rw = torch.zeros_like(gw)
        gc.write_payload_header(pays[w], hs)
        sec = gc.payload_sections(pays[w], hs)
        gc.ef_topk(gw, rw, ks, qsgd_levels=127, qsgd_group=64, qsgd_seed=900 + w, out_idx=sec["idx"],
                   out_codes=sec["codes"], out_norms=sec["meta0"], want_values=False, workspace=wsk)
        del gw, rw
    del wsk
    outb = torch.empty(ns, dtype=torch.float32, device=dev)
    f = lambda: gc.decompress_payloads(pays, [hs] * W, outb)
    eager = _eager_ms(torch, f, reps=10)
    gms, _ = _graph_ms(torch, [f] * 2, reps=5)
    osec = None
    if orc:
        hp = [{k: v.cpu().numpy() for k, v in gc.payload_sections(pays[w], hs).items()} for w in range(W)]

        def o_recv_sparse():
            acc = np.zeros(ns, np.float32)
            for w in range(W):
                orc.decompress_scatter(orc.KIND_QSGD, hp[w]["idx"], ks, 0, hp[w]["codes"], hp[w]["meta0"], None,
                                       64, 127, np.float32(1.0 / W), True, acc)
        osec = _oracle_s(o_recv_sparse)
    _row("a9 receive: average of W=8 sparse Top-1% + QSGD-127 payloads", "8 payloads of k = 1e6 into n = 1e8",
         4.0 * ns + W * (ks * (8.0 + 1.0 + 8.0) + 4.0 * ks / 64), "call", gms, eager, osec, 1.0,
         "the same 8 payloads")
    del pays, outb

    # EF sparsification variants over 1e9 elements of the layered workload (32 layers),
    # k = 1%, QSGD-127 on the kept values: Random-K (direct and deferred residual) and the
    # norm monitor's cost on the deferred Top-K step.
    LR, LLR = 32, 31_250_000
    nr, kr = LR * LLR, LR * LLR // 100
    gr = workloads.layered_torch(LR, LLR, step=1, device=dev, seed=5)
    rr = torch.zeros_like(gr)
    oir = torch.empty(kr, dtype=torch.int64, device=dev)
    ocr = torch.empty(kr, dtype=torch.int8, device=dev)
    onr = torch.empty((kr + 63) // 64, dtype=torch.float32, device=dev)
    wsr = torch.empty(gc.workspace_size(gc.OP_EF_RANDK, nr, kr, 127), dtype=torch.uint8, device=dev)
    pend = gc.pending_record(nr, kr, dev)
    st = torch.zeros(3, dtype=torch.float64, device=dev)
    ns_o = 1 << 24
    h = gr[:ns_o].cpu().numpy() if orc else None
    kept_bytes = kr * (8.0 + 1.0 + 4.0 / 64 + 4.0 + 4.0)
    variants = [
        ("next-3 EF Random-K 1% + QSGD-127", dict(select="randk", select_seed=77), 12.0 * nr + kept_bytes,
         lambda: orc.ef_randk_qsgd(h, np.zeros_like(h), ns_o // 100, 77, levels=127, group=64, qsgd_seed=501)),
        ("next-3 EF Random-K 1% + QSGD-127, deferred residual", dict(select="randk", select_seed=77, pending=pend),
         12.0 * nr + kept_bytes + 16.0 * kr, None),
        ("a10 EF Top-K 1% + QSGD-127, deferred residual", dict(pending=pend), 12.0 * nr + kept_bytes + 16.0 * kr,
         lambda: orc.ef_topk_qsgd(h, np.zeros_like(h), ns_o // 100, levels=127, group=64, seed=501)),
        ("next-2 the same with the norm monitor", dict(pending=pend, stats=st), 12.0 * nr + kept_bytes + 16.0 * kr,
         lambda: orc.monitored_step(h, np.zeros_like(h), ns_o // 100, levels=127, group=64, qsgd_seed=501)),
    ]
    for name, opt, ub, ofn in variants:
        say(name)
        if "pending" in opt:
            gc.ef_flush(rr, pend)                  # each variant starts from an exact residual
        f = lambda opt=opt: gc.ef_compress(gr, rr, kr, qsgd_levels=127, qsgd_group=64, qsgd_seed=501, out_idx=oir,
                                           out_codes=ocr, out_norms=onr, want_values=False, workspace=wsr, **opt)
        eager = _eager_ms(torch, f, reps=10)
        gms, _ = _graph_ms(torch, [f] * 2, reps=5)
        osec = _oracle_s(ofn) if (orc and ofn) else None
        extra = {"norm_ratio": round(float(st[2]), 6)} if "stats" in opt else None
        _row(name, "n=1e9 (32 layers x 31,250,000, t(3) x lognormal scales), k=1e7", ub, "call", gms, eager, osec,
             ns_o / nr, "the first 2^24 elements, k = 1% of them", extra=extra)
    del gr, rr, oir, ocr, onr, wsr, pend, st

    # next-4: the DDP communication hook at world size 1 (NCCL on this GPU): forward and
    # backward of a 6 x Linear(4096, 4096) model (100.7M parameters, 16 buckets of 25 MiB)
    # with DDP's own all-reduce hook and with the compression hook (deferred EF Top-1% +
    # QSGD-127, all_gather of the payloads, receive).
    ddp_hook_row(torch, gc, dev, say)

    # c3: TernGrad over 24 layers of 14,583,333 (~350M parameters), one segmented call.
    say("TernGrad 24 layers")
    L3, LL3 = workloads.TERN_LAYERS, workloads.TERN_LAYER_LEN
    xt = workloads.layered_torch(L3, LL3, step=0, device=dev, seed=3)
    off = np.arange(L3 + 1, dtype=np.int64) * LL3
    n3 = L3 * LL3
    nbytes = L3 * ((LL3 + 3) // 4)
    pk = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    scl = torch.empty(L3, dtype=torch.float32, device=dev)
    wst = torch.empty(max(gc.workspace_size(gc.OP_TERNGRAD, n3, L3, 0), 1), dtype=torch.uint8, device=dev)
    f = lambda: gc.terngrad(xt, off, 3, 0, packed=pk, scales=scl, workspace=wst)
    eager = _eager_ms(torch, f, reps=10)
    gms, _ = _graph_ms(torch, [f] * 4, reps=5)
    osec = None
    if orc:
        h = xt[:LL3].cpu().numpy()
        osec = _oracle_s(lambda: orc.terngrad(h, [0, LL3], 3))
    _row("a5+a7 TernGrad, per-layer scale", "24 layers x 14,583,333 (t(3) x lognormal(-7,1) scales)",
         4.0 * n3 + nbytes + 4.0 * L3, "call (all 24 layers)", gms, eager, osec, 1.0 / L3,
         "one layer of 14,583,333, scaled by 24",
         valu_ops=(VALU_LANE_OPS_PER_ELEMENT["terngrad"] + VALU_EXTRA_SLOTS_PER_ELEMENT["terngrad"]) * n3)
    del xt, pk, wst

    # c4: PowerSGD rank 4 on the three matrix shapes, error feedback on.
    qs = workloads.psgd_initial_q()
    for j, (rows, cols) in enumerate(workloads.PSGD_SHAPES):
        say(f"PowerSGD {rows}x{cols}")
        G = torch.from_numpy(workloads.psgd_gradient(1, j, (rows, cols))).to(dev)
        Es = [torch.zeros_like(G) for _ in range(2)]
        Qs = [torch.from_numpy(qs[j]).to(dev) for _ in range(2)]
        Ps = [torch.empty((rows, 4), dtype=torch.float32, device=dev) for _ in range(2)]
        wsp = torch.empty(gc.workspace_size(gc.OP_POWERSGD, rows, cols, 4), dtype=torch.uint8, device=dev)
        fns = [lambda i=i: gc.powersgd_step(G, Es[i], Qs[i], P=Ps[i], workspace=wsp) for i in range(2)]
        eager = _eager_ms(torch, fns[0], reps=10)
        gms, _ = _graph_ms(torch, fns * 2, reps=5)
        osec, thr = None, None
        if orc:
            Gh = G.cpu().numpy()
            osec = _oracle_s(lambda: orc.powersgd_step(Gh, np.zeros_like(Gh), qs[j]))
            thr = _blas_threads()
        flops = 2.0 * rows * cols * 4 * 3
        _row(f"a8 PowerSGD rank 4", f"{rows}x{cols} N(0, 1e-4), E on", 24.0 * rows * cols, "step",
             gms, eager, osec, 1.0, "the same matrix, float64 BLAS", cores=thr,
             extra={"tflops_three_passes": round(flops / (gms / 1e3) / 1e12, 3)})
        del G, Es, Qs, Ps, wsp


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the compression kernels run per GPU; no collectives are built)", file=sys.stderr)
        sys.exit(2)
    if args.rows:
        rows_mode(args)
        return

    import torch
    import gradient_compression_ddp_amd as gc
    import workloads

    dev = torch.device("cuda:0")
    L, LL = args.layers, args.layer_len
    n = L * LL
    k = int(n * args.ratio)
    print(f"[bench] generating 3 step gradients of {n} elements on the GPU", file=sys.stderr, flush=True)
    grads = [workloads.layered_torch(L, LL, step=t, device=dev) for t in (1, 2, 3)]
    res = torch.zeros(n, dtype=torch.float32, device=dev)
    out_idx = torch.empty(k, dtype=torch.int64, device=dev)
    out_codes = torch.empty(k, dtype=torch.int8, device=dev)
    out_norms = torch.empty((k + 63) // 64, dtype=torch.float32, device=dev)
    ws = torch.empty(gc.workspace_size(gc.OP_EF_TOPK, n, k, 127), dtype=torch.uint8, device=dev)
    mode = "direct" if args.direct else "deferred"
    pend = None if args.direct else gc.pending_record(n, k, dev)
    stats = torch.zeros(3, dtype=torch.float64, device=dev) if args.monitor else None
    torch.cuda.synchronize()

    def step(i):
        t = i % 3
        gc.ef_compress(grads[t], res, k, pending=pend, stats=stats, qsgd_levels=127, qsgd_group=64,
                       qsgd_seed=501 + t, out_idx=out_idx, out_codes=out_codes, out_norms=out_norms,
                       want_values=False, workspace=ws)

    if args.copy_calibration_gib > 0:
        nb = int(args.copy_calibration_gib * (1 << 30)) // 4
        src = grads[0][:nb]
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] calibration copy of {4 * nb} bytes done", file=sys.stderr, flush=True)
        del dst
    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    gc.profile_collect()              # discard anything recorded before the timed region
    gc.profile_enable(True)
    torch.cuda.synchronize()
    # one event pair per step on the launch stream (the binding launches on torch's
    # current stream), so each step's own GPU time is known besides the bracketed total
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record()
    for j, i in enumerate(range(args.warmup, args.warmup + args.steps)):
        step(i)
        ev[j + 1].record()
    if pend is not None:
        gc.ef_flush(res, pend)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    step_ms = sorted(ev[j].elapsed_time(ev[j + 1]) for j in range(args.steps))
    gc.profile_enable(False)
    calls, ms_before, ms_pass, ms_after = gc.profile_collect()
    print(f"[bench] timed {args.steps} steps in {elapsed:.4f} s", file=sys.stderr, flush=True)

    ms_step = elapsed / args.steps * 1e3
    in_bytes = 4.0 * n
    alg_step = 12.0 * n + 8.0 * k + 1.0 * k + 4.0 * ((k + 63) // 64)
    value = in_bytes / (ms_step / 1e3) / 1e9
    pass_ms = ms_pass / max(calls, 1)
    # the method's own bytes: read g and r, write c.  Deferred mode also reads the record
    # of the previous step (a 4-byte offset and a 4-byte value per kept entry, 12 bytes of
    # tile table per tile): reported apart, as overhead of the design, not in the fraction
    pass_bytes = 12.0 * n
    record_bytes = 0.0 if args.direct else 8.0 * k + 12.0 * ((n + 4095) // 4096)
    achieved = pass_bytes / (pass_ms / 1e3) / 1e9

    def pct(q):
        return round(step_ms[min(len(step_ms) - 1, int(q * (len(step_ms) - 1) + 0.5))], 4)
    traffic = K1_TRAFFIC_BYTES[mode] if k1_source_digest() == K1_SOURCE_SHA256 else None
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "ef_topk_1pct_qsgd8_7e9",
            "elements": n, "layers": L, "layer_len": LL, "k": k, "residual_update": mode,
            "norm_monitor": bool(args.monitor),
            "qsgd_levels": 127, "qsgd_group": 64, "step_gradients": 3,
            "parallelism": "single GPU",
        },
        "step_ms_events": {"median": pct(0.5), "p10": pct(0.1), "p90": pct(0.9), "reps": len(step_ms)},
        "hbm_frac_step": round(alg_step / (ms_step / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": alg_step,
        "stage_ms_per_step": {"before_pass": round(ms_before / max(calls, 1), 4),
                              "streaming_pass": round(pass_ms, 4),
                              "after_pass": round(ms_after / max(calls, 1), 4)},
        "roofline": {
            "bound": "hbm",
            "kernel": ("k_ef_cand (fused c = g + r, write c, candidate extraction)" if args.direct else
                       "k_ef_cand (fused c = g + r with the previous step's kept-set residuals applied, "
                       "write c, candidate extraction)"),
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": round(traffic / 1e9 / (pass_ms / 1e3), 1) if traffic else None,
            "traffic_bytes_per_launch": traffic,
            "bytes_per_launch": pass_bytes,
            "record_bytes_per_launch": record_bytes,
            "avg_launch_ms": round(pass_ms, 4),
        },
    }
    if stats is not None:
        line["norm_ratio_last_step"] = round(float(stats[2]), 6)
    if not args.no_cpu:
        del grads, res, ws, pend
        torch.cuda.empty_cache()
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(args, L)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
