"""Gradient-norm-ratio monitor of one compression step (oracle, float64).

What the pages fix (hotdry.top "gradient-compression-quantization-sparsification",
section 3.2, item 2): instrument the training step with the ratio of the gradient norm
after compression to the norm before it; a ratio that stays below 0.9 signals that the
compression is too strong.

Readings: "before" is the error-compensated gradient c = fl(g + r) that the compressor
sees, over all n elements; "after" is what the receiver decodes from the payload, g_hat
(the kept values for pure Top-K / Random-K, the QSGD reconstruction with QSGD), zero
off the kept set.  The monitor reports the two squared norms, summed in float64 from the
exact float64 squares of the float32 values, and ratio = sqrt(sum g_hat^2 / sum c^2),
with ratio = 1 when c is all zeros (then g_hat is all zeros too).  Summation order is
left open: this oracle uses numpy's float64 sum, and a compared result agrees within the
float64 rounding of a sum of n non-negative terms.
"""
from __future__ import annotations

import numpy as np

from .qsgd import qsgd
from .randk import ef_randk
from .topk import ef_topk

F32 = np.float32


def norm_stats(c: np.ndarray, g_hat: np.ndarray):
    """(sum c^2, sum g_hat^2, ratio) in float64."""
    c64 = np.asarray(c, dtype=F32).astype(np.float64)
    g64 = np.asarray(g_hat, dtype=F32).astype(np.float64)
    sc = float(np.sum(c64 * c64))
    sg = float(np.sum(g64 * g64))
    ratio = float(np.sqrt(sg / sc)) if sc > 0.0 else 1.0
    return sc, sg, ratio


def monitored_step(grad, residual, k, *, levels=0, group=64, qsgd_seed=0, index_base=0,
                   select="topk", select_seed=0):
    """One EF step (Top-K or Random-K, pure or with QSGD on the kept values) and its
    monitor.  Returns (stats, idx, new residual): stats = (sum c^2, sum g_hat^2, ratio).
    """
    grad = np.asarray(grad, dtype=F32)
    residual = np.asarray(residual, dtype=F32)
    c = (grad + residual).astype(F32)
    if select == "topk":
        idx, val, new_res = ef_topk(grad, residual, k, index_base)
    elif select == "randk":
        idx, val, new_res = ef_randk(grad, residual, k, select_seed, index_base)
    else:
        raise ValueError("select must be 'topk' or 'randk'")
    if levels > 0:
        _, _, g_hat, _ = qsgd(val, group, levels, qsgd_seed, index_base=0)
        new_res[idx - np.int64(index_base)] = (val - g_hat).astype(F32)
    else:
        g_hat = val
    return norm_stats(c, g_hat), idx, new_res


__all__ = ["norm_stats", "monitored_step"]
