"""Error-feedback Top-K sparsification (oracle).

What the pages fix:
* keep the K largest-magnitude entries of the flat gradient and drop the rest
  (hotdry.top "gradient-compression-quantization-sparsification", section 2;
  zyxy.net/archives/25733 "分布式训练中的梯度压缩算法", section 二.2 Top-K;
  5688vip.com "梯度累积与梯度压缩", section 4.2.1 ``topk_compress``, which sends
  int64 indices and the values at those indices);
* error feedback: add the residual left over from the previous round before
  selecting, and carry what was not sent into the next round
  (hotdry.top section 2.1; 5688vip.com section 4.2.1; aiqz.cc
  "梯度聚合通信优化实战方案", section "Python 演示", ``error_feedback_compress``).

Readings where the pages are open:
* exactly k entries are kept; among equal magnitudes the lower index wins; the
  output indices are in ascending order (``np.argpartition`` and the ``>=``
  threshold in the pages leave ties and order open);
* magnitude is compared on the IEEE bit pattern with the sign bit cleared (an
  unsigned 31-bit key).  +0 and -0 tie; NaNs rank above +Inf by their payload;
* the new residual is the compensated gradient with the kept entries set to +0.0
  (the demo's ``compensated - values`` read as subtracting the scattered values).
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def magnitude_key(c: np.ndarray) -> np.ndarray:
    """31-bit unsigned magnitude key of each float32: bit pattern with sign cleared."""
    return np.ascontiguousarray(c, dtype=F32).view(np.uint32) & np.uint32(0x7FFFFFFF)


def ef_topk(grad: np.ndarray, residual: np.ndarray, k: int, index_base: int = 0):
    """One error-feedback Top-K step.

    Returns (idx int64[k] ascending, offset by index_base; val float32[k] = c[idx];
    new residual float32[n]).
    """
    grad = np.asarray(grad, dtype=F32)
    residual = np.asarray(residual, dtype=F32)
    n = grad.size
    if not 0 <= k <= n:
        raise ValueError("k must lie in [0, n]")
    with np.errstate(over="ignore", invalid="ignore"):
        c = (grad + residual).astype(F32)             # compensated gradient, one fp32 add
    key = magnitude_key(c).astype(np.int64)
    # Sort by key descending, then by index ascending; keep the first k.
    order = np.lexsort((np.arange(n, dtype=np.int64), -key))
    kept = np.sort(order[:k]).astype(np.int64)
    val = c[kept].copy()
    new_residual = c.copy()
    new_residual[kept] = F32(0.0)
    return kept + np.int64(index_base), val, new_residual


def topk_invariant_holds(c: np.ndarray, idx: np.ndarray, k: int) -> bool:
    """O(n) check that ``idx`` is the exact Top-k set of ``c`` under the tie rule.

    Let T be the smallest key among the kept entries and i* the largest kept index
    whose key equals T.  The set is correct iff it has k distinct entries in
    ascending order, every dropped entry has key < T or (key == T and index > i*).
    """
    c = np.asarray(c, dtype=F32)
    idx = np.asarray(idx, dtype=np.int64)
    if idx.size != k:
        return False
    if k == 0:
        return True
    if np.any(np.diff(idx) <= 0) or idx[0] < 0 or idx[-1] >= c.size:
        return False
    key = magnitude_key(c).astype(np.int64)
    T = key[idx].min()
    i_star = idx[key[idx] == T].max()
    dropped = np.ones(c.size, dtype=bool)
    dropped[idx] = False
    kd = key[dropped]
    pos = np.nonzero(dropped)[0]
    ok_gt = not np.any(kd > T)
    ok_eq = not np.any((kd == T) & (pos < i_star))
    return bool(ok_gt and ok_eq)
