"""Pins for the oracle's min-max quantizer (CPU only): hand-worked fixtures, the
half-step error bound, the endpoints of every group, monotonicity, code-byte counts."""
import numpy as np
import pytest

import oracle
from golden_io import read_cases
import workloads

F32 = np.float32


@pytest.mark.parametrize("name", list(read_cases("minmax_hand.txt")))
def test_hand_worked_cases(name):
    case = read_cases("minmax_hand.txt")[name]
    x = np.array([float(v) for v in case["x"]], dtype=F32)
    bits, group = int(case["bits"][0]), int(case["group"][0])
    codes, mins, scales, ghat, _ = oracle.quant_minmax(x, group, bits)
    assert codes.tolist() == [int(v) for v in case["codes"]]
    assert mins.tolist() == [float(v) for v in case["mins"]]
    assert [int(s.view(np.uint32)) for s in scales] == [int(v, 16) for v in case["scale_bits"]]
    packed = codes if bits == 8 else oracle.pack_int4(codes)
    assert packed.tolist() == [int(v, 16) for v in case["packed"]]
    if bits == 4:
        assert oracle.unpack_int4(packed, x.size).tolist() == codes.tolist()


@pytest.mark.parametrize("bits,group", [(8, 64), (4, 64), (8, 0), (4, 0), (8, 256), (4, 1000)])
def test_error_bound_endpoints_monotone(bits, group):
    x = workloads.bucket(64 * 300 + 37)
    codes, mins, scales, ghat, _ = oracle.quant_minmax(x, group, bits)
    L = 2 ** bits - 1
    g = x.size if group == 0 else group
    for j in range(mins.size):
        seg = x[j * g:(j + 1) * g]
        q = codes[j * g:(j + 1) * g].astype(np.int64)
        if scales[j] > 0:
            assert q[np.argmin(seg)] == 0 and q[np.argmax(seg)] == L
        order = np.argsort(seg, kind="stable")
        assert np.all(np.diff(q[order]) >= 0)
        mag = max(abs(float(seg.min())), abs(float(seg.max())))
        slack = 3 * np.spacing(F32(mag))
        err = np.abs(seg.astype(np.float64) - ghat[j * g:(j + 1) * g].astype(np.float64))
        assert err.max() <= float(scales[j]) / 2 + float(slack)


def test_code_bytes_ratio():
    x = workloads.bucket(4096 * 3 + 1)
    c8, *_ = oracle.quant_minmax(x, 64, 8)
    c4, *_ = oracle.quant_minmax(x, 64, 4)
    assert x.nbytes == 4 * c8.nbytes
    assert oracle.pack_int4(c4).nbytes == (x.size + 1) // 2
    y = x[:-1]
    assert y.nbytes == 8 * oracle.pack_int4(oracle.quant_minmax(y, 64, 4)[0]).nbytes


def test_round_is_half_even_library_case():
    # np.rint is IEEE round-half-even, the rounding of np.round / torch.round on the pages
    v = np.array([0.5, 1.5, 2.5, -0.5, -1.5, 254.5], F32)
    assert np.rint(v).tolist() == [0.0, 2.0, 2.0, -0.0, -2.0, 254.0]


def test_error_feedback_residual():
    x = workloads.bucket(640)
    r0 = workloads.bucket(640, seed=9) * F32(0.1)
    codes, mins, scales, ghat, r1 = oracle.quant_minmax(x, 64, 8, residual=r0)
    xp = (x + r0).astype(F32)
    # the compensated value is split into what is sent and what is kept, within one rounding
    assert np.all(np.abs((ghat.astype(np.float64) + r1) - xp) <= np.spacing(np.abs(r1)) / 2 + 0)
    # and the codes are those of the compensated input
    assert np.array_equal(codes, oracle.quant_minmax(xp, 64, 8)[0])
