"""QSGD: stochastic rounding onto s levels of the group L2 norm (oracle).

What the pages fix (hotdry.top "gradient-compression-quantization-sparsification",
section 1.1): QSGD rounds each value up or down between discrete levels at random,
with probabilities set by its distance to the two levels, so that the quantized
gradient is unbiased in expectation; it is usually run with error feedback.
Grouping by 64 elements is the grouping strategy of section 1.2.  The pages give no
formula; we use the published QSGD scheme (Alistarh et al., NeurIPS 2017) that the
page names, per group of g elements:

    nu    = ||x_group||_2
    u     = (|x| / nu) * s,   l = floor(u),  p = u - l
    level = l + 1 with probability p, else l        (capped at s)
    code  = sign(x) * level                          (int8, |code| <= s <= 127)
    g_hat = sign(x) * (nu * level) / s

Readings where the pages are open:
* nu is fl(sqrt(sum of squares)) with the sum over a balanced pairwise tree in
  natural order (pairs (0,1),(2,3),..., then pairs of pairs); a partial last group
  is padded with +0.0;
* every step is one float32 operation: a = fl(|x|/nu), u = fl(a*s), p = u - l
  (exact), g_hat magnitude = fl(fl(nu*level)/s); "sign" means x < 0;
* the random draw for element i is the 24-bit Philox uniform U of element index
  index_base + i; "up" happens when U < p; nu == 0 gives all codes 0;
* with error feedback: x' = fl(x + e), and the new e = fl(x' - g_hat).
"""
from __future__ import annotations

import numpy as np

from .philox import uniform24

F32 = np.float32


def pairwise_sum_of_squares(x: np.ndarray, group: int) -> np.ndarray:
    """Per-group sum of squares over a balanced pairwise tree (group a power of two)."""
    if group < 1 or group & (group - 1):
        raise ValueError("group must be a power of two")
    x = np.asarray(x, dtype=F32)
    n = x.size
    ng = (n + group - 1) // group
    padded = np.zeros(ng * group, dtype=F32)
    padded[:n] = x
    sq = (padded * padded).astype(F32).reshape(ng, group)
    while sq.shape[1] > 1:
        sq = (sq[:, 0::2] + sq[:, 1::2]).astype(F32)
    return sq[:, 0].copy()


def qsgd(x: np.ndarray, group: int, levels: int, seed: int, index_base: int = 0,
         residual: np.ndarray | None = None):
    """Returns (codes int8[n], norms float32[ng], g_hat float32[n], new residual or None)."""
    if not 1 <= levels <= 127:
        raise ValueError("levels must lie in [1, 127]")
    x = np.asarray(x, dtype=F32)
    if residual is not None:
        x = (x + np.asarray(residual, dtype=F32)).astype(F32)
    n = x.size
    norms = np.sqrt(pairwise_sum_of_squares(x, group)).astype(F32)
    nu = norms[np.arange(n, dtype=np.int64) // group] if n else np.zeros(0, F32)
    s = F32(levels)
    ax = np.abs(x)
    neg = x < F32(0.0)
    live = nu > F32(0.0)
    with np.errstate(divide="ignore", invalid="ignore"):
        a = np.where(live, ax / np.where(live, nu, F32(1.0)), F32(0.0)).astype(F32)
    u = (a * s).astype(F32)
    l = np.floor(u).astype(F32)
    p = (u - l).astype(F32)
    U = uniform24(seed, np.int64(index_base) + np.arange(n, dtype=np.int64))
    up = (U < p).astype(F32)
    level = np.minimum(l + up, s).astype(F32)
    level = np.where(live, level, F32(0.0)).astype(F32)
    codes = np.where(neg, -level, level).astype(np.int8)
    g_hat = dequant_qsgd(codes, norms, group, levels)
    new_res = (x - g_hat).astype(F32) if residual is not None else None
    return codes, norms, g_hat, new_res


def dequant_qsgd(codes: np.ndarray, norms: np.ndarray, group: int, levels: int,
                 positions: np.ndarray | None = None) -> np.ndarray:
    """g_hat = sign * fl(fl(nu*|code|)/s), sign negative where code < 0."""
    codes = np.asarray(codes, dtype=np.int8)
    n = codes.size
    pos = np.arange(n, dtype=np.int64) if positions is None else np.asarray(positions, np.int64)
    nu = np.asarray(norms, dtype=F32)[pos // group] if n else np.zeros(0, F32)
    level = np.abs(codes.astype(np.int32)).astype(F32)
    mag = ((nu * level).astype(F32) / F32(levels)).astype(F32)
    return np.where(codes < 0, -mag, mag).astype(F32)
