"""Pins for the oracle's PowerSGD step (CPU only): exact recovery of rank-r
matrices, orthonormality, agreement with LAPACK's QR, convergence to the SVD's
top-r subspace, and the error-feedback split."""
import numpy as np
import pytest

import oracle

F32 = np.float32


def test_rank_r_matrix_is_recovered():
    rng = np.random.default_rng(1)
    A = rng.standard_normal((300, 4)).astype(F32)
    B = rng.standard_normal((200, 4)).astype(F32)
    M = (A.astype(np.float64) @ B.T.astype(np.float64)).astype(F32)
    Q = rng.standard_normal((200, 4)).astype(F32)
    out = oracle.powersgd_step(M, None, Q)
    assert np.linalg.norm(out["E"]) / np.linalg.norm(out["M"]) < 1e-6
    assert np.allclose(out["Mhat"], out["M"], rtol=0, atol=1e-5 * np.abs(out["M"]).max())


def test_orthonormal_and_equal_to_lapack_qr():
    rng = np.random.default_rng(2)
    G = rng.normal(0, 1e-2, (257, 129)).astype(F32)
    Q = rng.standard_normal((129, 4)).astype(F32)
    out = oracle.powersgd_step(G, None, Q)
    P = out["P"]
    assert np.allclose(P.T @ P, np.eye(4), atol=1e-12)
    Pfull = G.astype(np.float64) @ Q.astype(np.float64)
    qr_q, qr_r = np.linalg.qr(Pfull)
    qr_q = qr_q * np.sign(np.diag(qr_r))       # make R's diagonal positive, as Gram-Schmidt does
    assert np.allclose(P, qr_q, atol=1e-10)


def test_power_iteration_converges_to_top_subspace():
    rng = np.random.default_rng(3)
    U, _ = np.linalg.qr(rng.standard_normal((120, 120)))
    V, _ = np.linalg.qr(rng.standard_normal((90, 90)))
    sv = np.concatenate([[10, 8, 6, 4], np.linspace(1, 0.1, 86)])
    M = (U[:, :90] * sv) @ V.T
    M = M.astype(F32)
    Q = rng.standard_normal((90, 4)).astype(F32)
    for _ in range(60):
        out = oracle.powersgd_step(M, None, Q)
        Q = out["Q"]
    u, s, vt = np.linalg.svd(M.astype(np.float64))
    best = (u[:, :4] * s[:4]) @ vt[:4]
    assert np.linalg.norm(out["Mhat"] - best) / np.linalg.norm(best) < 1e-6


def test_error_feedback_split():
    rng = np.random.default_rng(4)
    G = rng.normal(0, 1e-2, (64, 48)).astype(F32)
    E = rng.normal(0, 1e-3, (64, 48)).astype(F32)
    Q = rng.standard_normal((48, 4)).astype(F32)
    out = oracle.powersgd_step(G, E, Q)
    assert np.array_equal(out["M"], (G + E).astype(F32).astype(np.float64))
    assert np.allclose(out["Mhat"] + out["E"], out["M"], rtol=0, atol=1e-15)


def test_zero_column_stays_zero():
    G = np.zeros((16, 8), F32)
    G[:, 0] = 1.0
    Q = np.zeros((8, 2), F32)
    Q[0, 0] = 1.0
    Q[0, 1] = 2.0          # second column of P is parallel to the first -> zero after projection
    out = oracle.powersgd_step(G, None, Q)
    assert np.allclose(out["P"][:, 1], 0.0)
    assert np.allclose(out["Q"][:, 1], 0.0)


def test_numerically_dependent_column_becomes_zero():
    # p_1 = 2 p_0 exactly in exact arithmetic; the float64 projection leaves only rounding
    rng = np.random.default_rng(9)
    G = np.zeros((64, 16), F32)
    G[:, 0] = np.linspace(1, 2, 64, dtype=F32)
    G[:, 1] = rng.standard_normal(64).astype(F32)
    Q = np.zeros((16, 3), F32)
    Q[0, 0], Q[0, 1], Q[1, 2] = 1.0, 3.0, 1.0
    out = oracle.powersgd_step(G, None, Q)
    assert np.all(out["P"][:, 1] == 0.0)
    assert abs(np.linalg.norm(out["P"][:, 2]) - 1.0) < 1e-12      # an independent column survives
    assert abs(out["P"][:, 0] @ out["P"][:, 2]) < 1e-12
