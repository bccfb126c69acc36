"""Pins for the oracle's decompression and the Top-K + 8-bit QSGD pipeline (CPU only):
decoded payloads reproduce each compressor's own g_hat, scatter matches dense decode,
and the pipeline keeps the exact Top-K set with the error-feedback split."""
import numpy as np

import oracle
import workloads

F32 = np.float32


def test_decode_matches_each_compressor():
    x = workloads.bucket(64 * 40 + 9)
    n = x.size
    c8, m8, s8, g8, _ = oracle.quant_minmax(x, 64, 8)
    out = oracle.decompress_scatter(oracle.KIND_MINMAX8, None, n, 0, c8, m8, s8, 64, 0, 1.0, 0,
                                    np.zeros(n, F32))
    assert np.array_equal(out, g8)
    c4, m4, s4, g4, _ = oracle.quant_minmax(x, 64, 4)
    out = oracle.decompress_scatter(oracle.KIND_MINMAX4, None, n, 0, oracle.pack_int4(c4), m4, s4,
                                    64, 0, 1.0, 0, np.zeros(n, F32))
    assert np.array_equal(out, g4)
    cq, nq, gq, _ = oracle.qsgd(x, 64, 15, seed=7)
    out = oracle.decompress_scatter(oracle.KIND_QSGD, None, n, 0, cq, nq, None, 64, 15, 1.0, 0,
                                    np.zeros(n, F32))
    assert np.array_equal(out, gq)
    pk, sc, ct, gt, _ = oracle.terngrad(x, [0, n], seed=3)
    out = oracle.decompress_scatter(oracle.KIND_TERN, None, n, 0, pk, sc, None, 0, 0, 1.0, 0,
                                    np.zeros(n, F32))
    assert np.array_equal(out, gt)


def test_scatter_accumulate():
    g = workloads.bucket(5000)
    idx, val, _ = oracle.ef_topk(g, np.zeros_like(g), 50, index_base=100)
    out = np.zeros(g.size, F32)
    oracle.decompress_scatter(oracle.KIND_F32, idx, 50, 100, val, None, None, 0, 0, 1.0, 1, out)
    oracle.decompress_scatter(oracle.KIND_F32, idx, 50, 100, val, None, None, 0, 0, 1.0, 1, out)
    dense = np.zeros(g.size, F32)
    dense[idx - 100] = val
    assert np.array_equal(out, (dense + dense).astype(F32))
    oracle.decompress_scatter(oracle.KIND_F32, idx, 50, 100, val, None, None, 0, 0, 0.5, 0, out)
    assert np.array_equal(out, (dense * F32(0.5)).astype(F32))


def test_pipeline_topk_then_qsgd8():
    g, off = workloads.big_layers_host(8, 4099, step=1)
    r = np.zeros_like(g)
    k = g.size // 100
    idx, codes, norms, r1, val = oracle.ef_topk_qsgd(g, r, k, seed=501)
    c = (g + r).astype(F32)
    assert oracle.topk_invariant_holds(c, idx, k)
    assert np.array_equal(val, c[idx])
    assert np.abs(codes.astype(np.int32)).max() <= 127
    assert norms.size == (k + 63) // 64
    ghat = oracle.dequant_qsgd(codes, norms, 64, 127)
    dropped = np.ones(g.size, bool)
    dropped[idx] = False
    assert np.array_equal(r1[dropped], c[dropped])
    # what is sent plus what is kept gives back c within half an ulp of the kept residual
    err = np.abs((ghat.astype(np.float64) + r1[idx]) - c[idx])
    assert np.all(err <= np.spacing(np.abs(r1[idx])) / 2)
