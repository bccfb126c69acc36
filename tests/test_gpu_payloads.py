"""GPU parity of the receive side (gc_decompress_payloads) and the wire format.

Each payload is produced on the GPU by the library's compressors writing straight into
the sections of one wire buffer; the expected result comes from the oracle alone: it
compresses the same inputs itself and adds the decoded payloads in order
(out = 0 or out, then out += alpha * g_hat_w for w = 0..W-1).  Bit-exact."""
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


def new_payload(gc, kind, n, count, group=0, levels=0, sparse=False, index_base=0):
    import torch
    h = gc.payload_layout(kind, n, count, group, levels, sparse, index_base)
    buf = torch.zeros(h.bytes, dtype=torch.uint8, device="cuda")
    gc.write_payload_header(buf, h)
    return buf, h


def dense_payload(gc, kind, x, group, levels, seed):
    """GPU payload of x, and the oracle's (codes, meta0, meta1) of the same x."""
    n = x.size
    buf, h = new_payload(gc, kind, n, n, group, levels)
    sec = gc.payload_sections(buf, h)
    xd = dev(x)
    if kind == gc.KIND_QSGD:
        gc.qsgd(xd, group, levels, seed, codes=sec["codes"], norms=sec["meta0"])
        c, nu, _, _ = oracle.qsgd(x, group, levels, seed)
        want = (c, nu, None)
    elif kind in (gc.KIND_MINMAX8, gc.KIND_MINMAX4):
        bits = 8 if kind == gc.KIND_MINMAX8 else 4
        gc.quant_minmax(xd, group, bits, codes=sec["codes"], mins=sec["meta0"], scales=sec["meta1"],
                        workspace=None)
        c, mn, sc, _, _ = oracle.quant_minmax(x, group, bits)
        want = (c if bits == 8 else oracle.pack_int4(c), mn, sc)
    elif kind == gc.KIND_TERN:
        gc.terngrad(xd, [0, n], seed, packed=sec["codes"], scales=sec["meta0"])
        pk, s, _, _, _ = oracle.terngrad(x, [0, n], seed)
        want = (pk, s, None)
    else:
        sec["codes"].copy_(xd)
        want = (x, None, None)
    return buf, h, want


def expected(kind, wants, count, group, levels, alpha, init, idx=None, index_base=0):
    out = init.copy()
    for w, (codes, m0, m1) in enumerate(wants):
        ix = None if idx is None else idx[w]
        oracle.decompress_scatter(kind, ix, count, index_base, codes, m0, m1, group, levels, alpha, True, out)
    return out


@pytest.mark.parametrize("kind,group,levels", [(3, 64, 15), (1, 1000, 0), (2, 64, 0), (4, 0, 0), (0, 0, 0)])
@pytest.mark.parametrize("W,accumulate", [(8, False), (3, True), (20, False)])
def test_dense_payloads_fused(gc, kind, group, levels, W, accumulate):
    n = 3 * 4096 + 1003
    bufs, hdrs, wants = [], [], []
    for w in range(W):
        x = workloads.bucket(n, seed=100 + w)
        b, h, want = dense_payload(gc, kind, x, group, levels, seed=7 + w)
        bufs.append(b); hdrs.append(h); wants.append(want)
    init = np.linspace(-1, 1, n, dtype=F32) if accumulate else np.zeros(n, F32)
    out = dev(init)
    alpha = F32(1.0) / F32(W)
    gc.decompress_payloads(bufs, hdrs, out, alpha=float(alpha), accumulate=accumulate)
    want = expected(kind, wants, n, group, levels, alpha, init)
    assert_bits_equal(host(out), want, f"kind {kind} W {W}")


@pytest.mark.parametrize("kind,group,levels,n", [(1, 64, 0, 3 * 4096 + 1003), (2, 128, 0, 3 * 4096 + 1003),
                                                  (3, 16, 127, 3 * 4096 + 1003), (4, 0, 0, 1 << 14)])
@pytest.mark.parametrize("W,accumulate", [(5, False), (17, True)])
def test_dense_payloads_sixteen_entry_path(gc, kind, group, levels, n, W, accumulate):
    """Packed codes in groups of a power of two >= 16 (TernGrad: one group of 2^14) take the
    path where a lane sums 16 entries of one group over chunks of payloads; ragged ends,
    a chunk cut short (W = 5), a second launch (W = 17) and accumulation included."""
    bufs, hdrs, wants = [], [], []
    for w in range(W):
        x = workloads.bucket(n, seed=500 + w)
        b, h, want = dense_payload(gc, kind, x, group, levels, seed=11 + w)
        bufs.append(b); hdrs.append(h); wants.append(want)
    init = np.linspace(-2, 2, n, dtype=F32) if accumulate else np.zeros(n, F32)
    out = dev(init)
    alpha = F32(1.0) / F32(W)
    gc.decompress_payloads(bufs, hdrs, out, alpha=float(alpha), accumulate=accumulate)
    want = expected(kind, wants, n, group, levels, alpha, init)
    assert_bits_equal(host(out), want, f"kind {kind} W {W}")


def test_dense_payloads_unaligned_out_takes_the_sequential_path(gc):
    import torch
    n, W = 5000, 4
    bufs, hdrs, wants = [], [], []
    for w in range(W):
        b, h, want = dense_payload(gc, gc.KIND_QSGD, workloads.bucket(n, seed=w), 64, 127, seed=w)
        bufs.append(b); hdrs.append(h); wants.append(want)
    full = torch.full((n + 1,), 3.0, dtype=torch.float32, device="cuda")
    gc.decompress_payloads(bufs, hdrs, full[1:])           # out offset by 4 bytes, not accumulating
    got = host(full)
    want = expected(gc.KIND_QSGD, wants, n, 64, 127, F32(1.0) / F32(W), np.zeros(n, F32))
    assert got[0] == F32(3.0)
    assert_bits_equal(got[1:], want, "unaligned out")


def test_sparse_topk_payloads(gc):
    """W Top-K payloads (values, and QSGD-coded kept values) from different gradients."""
    import torch
    n, k, W, base = 300_007, 3_000, 4, 1000
    for quant in (False, True):
        bufs, hdrs, idxs, wants = [], [], [], []
        for w in range(W):
            g = workloads.bucket(n, seed=40 + w)
            r = (workloads.bucket(n, seed=50 + w) * F32(0.1)).astype(F32)
            kind = gc.KIND_QSGD if quant else gc.KIND_F32
            b, h = new_payload(gc, kind, n, k, 64 if quant else 0, 127 if quant else 0, True, base)
            sec = gc.payload_sections(b, h)
            rd = dev(r)
            if quant:
                gc.ef_topk(dev(g), rd, k, index_base=base, qsgd_levels=127, qsgd_group=64, qsgd_seed=500 + w,
                           out_idx=sec["idx"], out_codes=sec["codes"], out_norms=sec["meta0"], want_values=False)
                oi, oc, onu, _, _ = oracle.ef_topk_qsgd(g, r, k, levels=127, group=64, seed=500 + w,
                                                        index_base=base)
                wants.append((oc, onu, None))
            else:
                gc.ef_topk(dev(g), rd, k, index_base=base, out_idx=sec["idx"], out_val=sec["codes"])
                oi, ov, _ = oracle.ef_topk(g, r, k, index_base=base)
                wants.append((ov, None, None))
            idxs.append(oi)
            bufs.append(b); hdrs.append(h)
        out = torch.zeros(n, dtype=torch.float32, device="cuda")
        gc.decompress_payloads(bufs, hdrs, out)
        kind = gc.KIND_QSGD if quant else gc.KIND_F32
        want = expected(kind, wants, k, 64 if quant else 0, 127 if quant else 0, F32(1.0) / F32(W),
                        np.zeros(n, F32), idx=idxs, index_base=base)
        assert_bits_equal(host(out), want, f"sparse quant={quant}")


def test_mixed_kinds_and_header_round_trip(gc):
    import torch
    n = 20_000
    specs = [(gc.KIND_MINMAX8, 64, 0), (gc.KIND_QSGD, 128, 15), (gc.KIND_TERN, 0, 0), (gc.KIND_F32, 0, 0)]
    bufs, hdrs, expect_out = [], [], np.zeros(n, F32)
    alpha = F32(0.25)
    for w, (kind, group, levels) in enumerate(specs):
        x = workloads.bucket(n, seed=200 + w)
        b, h, (c, m0, m1) = dense_payload(gc, kind, x, group, levels, seed=60 + w)
        h2 = gc.read_payload_header(b)                    # what a receiver would parse after a gather
        assert bytes(h2) == bytes(h)
        bufs.append(b); hdrs.append(h2)
        oracle.decompress_scatter(kind, None, n, 0, c, m0, m1, group, levels, alpha, True, expect_out)
    out = torch.full((n,), 9.0, dtype=torch.float32, device="cuda")
    gc.decompress_payloads(bufs, hdrs, out, alpha=float(alpha))
    assert_bits_equal(host(out), expect_out, "mixed kinds")


def test_bucket_full_size_eight_workers(gc):
    """Eight QSGD payloads of the 25 MiB bucket (s = 15, groups of 64), averaged."""
    import torch
    n, W = workloads.BUCKET_N, 8
    bufs, hdrs, wants = [], [], []
    for w in range(W):
        b, h, want = dense_payload(gc, gc.KIND_QSGD, workloads.bucket(n, seed=300 + w), 64, 15, seed=7 + w)
        bufs.append(b); hdrs.append(h); wants.append(want)
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    gc.decompress_payloads(bufs, hdrs, out)
    want = expected(gc.KIND_QSGD, wants, n, 64, 15, F32(1.0) / F32(W), np.zeros(n, F32))
    assert_bits_equal(host(out), want, "bucket W=8")


@pytest.mark.parametrize("levels", [6, 12, 126, 127])
def test_qsgd_decode_small_norms_even_levels(gc, levels):
    """QSGD codes with group norms from 1e-44 to 1e-28 (below and above 2^-100, where the
    decoders switch between the division and the multiply-and-correct quotient) and level
    counts with even factors, whose subnormal quotients can be exact rounding midpoints:
    the dense decode and the W-payload receive must equal the oracle bit for bit."""
    rng = np.random.default_rng(levels)
    n, group, W = 64 * 300 + 17, 64, 3
    ng = (n + group - 1) // group
    bufs, hdrs, wants = [], [], []
    for w in range(W):
        codes = rng.integers(-levels, levels + 1, n).astype(np.int8)
        nu = (10.0 ** rng.uniform(-44, -28, ng)).astype(F32)
        nu[::5] = F32(2.0 ** -100)
        nu[1::7] = np.nextafter(F32(2.0 ** -100), F32(0))
        buf, h = new_payload(gc, gc.KIND_QSGD, n, n, group, levels)
        sec = gc.payload_sections(buf, h)
        sec["codes"].copy_(dev(codes.view(np.uint8)).view(sec["codes"].dtype))
        sec["meta0"].copy_(dev(nu))
        bufs.append(buf); hdrs.append(h); wants.append((codes, nu, None))
    # dense decode of the first payload
    out = dev(np.zeros(n, F32))
    gc.decompress_scatter(gc.KIND_QSGD, gc.payload_sections(bufs[0], hdrs[0])["codes"], n, out,
                          meta0=gc.payload_sections(bufs[0], hdrs[0])["meta0"], group=group, levels=levels)
    want = oracle.decompress_scatter(gc.KIND_QSGD, None, n, 0, wants[0][0], wants[0][1], None, group, levels,
                                     1.0, 0, np.zeros(n, F32))
    assert_bits_equal(host(out), want, "dense decode")
    # the fused receive of all three
    out = dev(np.zeros(n, F32))
    alpha = F32(1.0) / F32(W)
    gc.decompress_payloads(bufs, hdrs, out, alpha=float(alpha))
    assert_bits_equal(host(out), expected(gc.KIND_QSGD, wants, n, group, levels, alpha, np.zeros(n, F32)),
                      "receive")


def _random_sparse_payload(gc, rng, kind, n_out, count, base, dense_span=None):
    """A hand-made sparse payload: strictly ascending idx (some positions below 0 or past
    n_out, which the receiver skips), random codes and metadata.  Returns the buffer, its
    header and what the oracle needs."""
    if dense_span is not None:
        pos = np.arange(*dense_span, dtype=np.int64)
        count = pos.size
    else:
        pos = np.sort(rng.choice(np.arange(-300, n_out + 300, dtype=np.int64), count, replace=False))
    group, levels = {gc.KIND_F32: (0, 0), gc.KIND_MINMAX8: (50, 0), gc.KIND_MINMAX4: (64, 0),
                     gc.KIND_QSGD: (64, 127), gc.KIND_TERN: (0, 0)}[kind]
    buf, h = new_payload(gc, kind, n_out, count, group, levels, True, base)
    sec = gc.payload_sections(buf, h)
    idx = pos + base
    ng = 0 if count == 0 else (count + (group or count) - 1) // (group or count)
    if kind == gc.KIND_F32:
        codes = rng.standard_normal(count).astype(F32)
    elif kind == gc.KIND_QSGD:
        codes = rng.integers(-127, 128, count).astype(np.int8)
    elif kind == gc.KIND_MINMAX8:
        codes = rng.integers(0, 256, count).astype(np.uint8)
    elif kind == gc.KIND_MINMAX4:
        codes = rng.integers(0, 256, (count + 1) // 2).astype(np.uint8)
    else:
        q = rng.choice(np.array([0, 1, 3], np.uint8), (count + 3) // 4 * 4)
        codes = (q[0::4] | (q[1::4] << 2) | (q[2::4] << 4) | (q[3::4] << 6)).astype(np.uint8)
    m0 = (rng.standard_normal(ng) * 0.1).astype(F32)
    m1 = np.abs(rng.standard_normal(ng) * 0.01).astype(F32) if kind in (gc.KIND_MINMAX8, gc.KIND_MINMAX4) else None
    if count:
        sec["idx"].copy_(dev(idx))
        sec["codes"].copy_(dev(codes).view(sec["codes"].dtype))
        if "meta0" in sec:
            sec["meta0"].copy_(dev(m0 if kind != gc.KIND_QSGD else np.abs(m0)))
        if "meta1" in sec:
            sec["meta1"].copy_(dev(m1))
    if kind == gc.KIND_QSGD:
        m0 = np.abs(m0)
    return buf, h, (kind, idx, count, base, codes, m0, m1, group, levels)


@pytest.mark.parametrize("W,accumulate", [(8, False), (17, True), (3, False)])
def test_sparse_merge_many_kinds(gc, W, accumulate):
    """All-sparse receive (the tile-by-tile merge): every payload kind, ragged output,
    positions outside [0, n_out) skipped, an empty payload, a dense run longer than the
    staging space, more payloads than one launch takes; order of the terms per element is
    payload order (the oracle adds them one payload at a time)."""
    rng = np.random.default_rng(W)
    n_out = 5 * 8 * 4096 + 1234
    kinds = [gc.KIND_F32, gc.KIND_QSGD, gc.KIND_MINMAX8, gc.KIND_MINMAX4, gc.KIND_TERN]
    bufs, hdrs, specs = [], [], []
    for w in range(W):
        kind = kinds[w % len(kinds)]
        base = int(rng.integers(0, 1 << 40))
        if w == 1:
            b, h, spec = _random_sparse_payload(gc, rng, kind, n_out, 0, base, dense_span=(2 * 4096 + 100, 4 * 4096 + 50))
        elif w == 2:
            b, h, spec = _random_sparse_payload(gc, rng, kind, n_out, 0, base)
        else:
            b, h, spec = _random_sparse_payload(gc, rng, kind, n_out, int(rng.integers(100, n_out // 20)), base)
        bufs.append(b); hdrs.append(h); specs.append(spec)
    init = np.linspace(-1, 1, n_out, dtype=F32) if accumulate else np.zeros(n_out, F32)
    alpha = F32(1.0) / F32(W)
    off = 1000
    big = np.concatenate([np.zeros(off, F32), init, np.zeros(off, F32)])
    for kind, idx, count, base, codes, m0, m1, group, levels in specs:
        oracle.decompress_scatter(kind, idx, count, base - off, codes, m0, m1, group, levels, alpha, True, big)
    out = dev(init)
    gc.decompress_payloads(bufs, hdrs, out, alpha=float(alpha), accumulate=accumulate)
    assert_bits_equal(host(out), big[off:off + n_out], f"W {W}")
