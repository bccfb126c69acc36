"""Error-feedback Random-K sparsification (oracle).

What the pages fix (hotdry.top "gradient-compression-quantization-sparsification",
section 2.2: Random-K keeps a random K% of the gradient, a steadier communication
pattern than Top-K at some loss of retained information, and is run with the same error
feedback as Top-K, section 2.1; zyxy.net/archives/25733 "分布式训练中的梯度压缩算法",
section 二.2: random sparsification keeps each gradient with a probability and zeroes the
rest).

Reading: exactly k entries are kept (a fixed-size payload, like Top-K), chosen
uniformly at random without replacement by a counter-based draw, so that the choice is
reproducible and independent of the values:
    key_e = (Philox4x32-10 word of global index index_base + e under `seed`) >> 1
(a 31-bit key; the word is the one the quantizers draw, see philox.py).  The kept set is
the k largest keys, the lower index winning among equal keys; then, as for EF Top-K,
    c = fl(g + r),  idx ascending (plus index_base),  val = c[idx],
    r' = c with r'[idx] = +0.0.
With QSGD on the kept values (ef_randk_qsgd) the residual of a kept entry is
fl(val - g_hat) instead, as in the Top-K pipeline.
"""
from __future__ import annotations

import numpy as np

from .philox import random_words
from .qsgd import qsgd

F32 = np.float32


def randk_keys(seed: int, n: int, index_base: int = 0) -> np.ndarray:
    """The 31-bit selection key of each of the n elements (uint32)."""
    e = np.arange(n, dtype=np.int64) + np.int64(index_base)
    return (random_words(seed, e) >> np.uint32(1)).astype(np.uint32)


def select_largest(key: np.ndarray, k: int) -> np.ndarray:
    """Positions of the k largest keys, the lower position winning among equal keys,
    in ascending order (int64)."""
    n = key.size
    order = np.lexsort((np.arange(n, dtype=np.int64), -np.asarray(key).astype(np.int64)))
    return np.sort(order[:k]).astype(np.int64)


def ef_randk(grad: np.ndarray, residual: np.ndarray, k: int, seed: int, index_base: int = 0):
    """One error-feedback Random-K step.

    Returns (idx int64[k] ascending, offset by index_base; val float32[k] = c[idx];
    new residual float32[n]).
    """
    c = (np.asarray(grad, F32) + np.asarray(residual, F32)).astype(F32)
    n = c.size
    if not 0 <= k <= n:
        raise ValueError("k must lie in [0, n]")
    kept = select_largest(randk_keys(seed, n, index_base), k)
    new_res = c.copy()
    new_res[kept] = F32(0.0)
    return kept + np.int64(index_base), c[kept].copy(), new_res


def ef_randk_qsgd(grad, residual, k, seed, levels=127, group=64, qsgd_seed=0, index_base=0):
    """Random-K, then QSGD on the kept values (groups in kept order, RNG index = kept
    position).  Returns (idx, codes, norms, new residual, kept values)."""
    idx, val, new_res = ef_randk(grad, residual, k, seed, index_base)
    codes, norms, g_hat, _ = qsgd(val, group, levels, qsgd_seed, index_base=0)
    new_res[idx - np.int64(index_base)] = (val - g_hat).astype(F32)
    return idx, codes, norms, new_res, val
