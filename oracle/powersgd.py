"""PowerSGD rank-r step with error feedback (oracle, float64).

What the pages fix (hotdry.top "gradient-compression-quantization-sparsification",
section 3.1; aiqz.cc "梯度聚合通信优化实战方案", section "梯度压缩原理"): PowerSGD
approximates the gradient matrix by a low-rank product, sends only the two thin
factors, rebuilds the product at the receiver, costs extra computation, and is run
with error feedback.  The pages give no formula; we use one power-iteration step of
the PowerSGD paper the page cites (Vogels et al., NeurIPS 2019):

    M  = G + E                         (error feedback; fp32 add, as the GPU does)
    P  = M Q                           (rows x r)
    P^ = orthonormalize(P)             (modified Gram-Schmidt over the r columns)
    Q' = M^T P^                        (cols x r)
    M^ = P^ Q'^T,   E' = M - M^

Readings where the pages are open: modified Gram-Schmidt in column order 0..r-1
(for each j: subtract (p^_i . p_j) p^_i for i < j using the updated p_j, then divide
by its norm); only P is orthonormalized; Q' warm-starts the next step; matrices are
row-major.  A column that lies in the span of the previous ones becomes 0: in exact
arithmetic its projected norm is 0, and in floating point we take "numerically in the
span" to mean a projected norm of at most 1e-5 of the column's own norm (below that its
direction is set by rounding, not by the data).
"""
from __future__ import annotations

import numpy as np

F32 = np.float32
DEPENDENT_REL = 1e-5


def modified_gram_schmidt(P: np.ndarray) -> np.ndarray:
    P = np.array(P, dtype=np.float64, copy=True)
    rows, r = P.shape
    out = np.zeros_like(P)
    for j in range(r):
        v = P[:, j].copy()
        own = np.sqrt(v @ v)
        for i in range(j):
            v = v - (out[:, i] @ v) * out[:, i]
        nrm = np.sqrt(v @ v)
        out[:, j] = v / nrm if nrm > DEPENDENT_REL * own else 0.0
    return out


def powersgd_step(G: np.ndarray, E: np.ndarray | None, Q: np.ndarray):
    """One step.  Returns a dict with float64 results and float32-rounded carries.

    Keys: M (fp64 of the fp32 sum), P (P^), Q (Q'), Mhat, E (E'), and
    P32, Q32, E32 (the same rounded to float32, which a caller carries to the next
    step).
    """
    G = np.asarray(G, dtype=F32)
    M32 = (G + np.asarray(E, dtype=F32)).astype(F32) if E is not None else G.copy()
    M = M32.astype(np.float64)
    Q64 = np.asarray(Q, dtype=F32).astype(np.float64)
    P = M @ Q64
    Phat = modified_gram_schmidt(P)
    Qn = M.T @ Phat
    Mhat = Phat @ Qn.T
    En = M - Mhat
    return {
        "M": M, "P": Phat, "Q": Qn, "Mhat": Mhat, "E": En,
        "P32": Phat.astype(F32), "Q32": Qn.astype(F32), "E32": En.astype(F32),
    }
