"""The hybrid path: error-feedback Top-K followed by 8-bit QSGD on the kept values.

What the pages fix: combining Top-K at 1% with 8-bit quantization of what is sent
(5688vip.com "梯度累积与梯度压缩", section 4.3; hotdry.top
"gradient-compression-quantization-sparsification", section 3 on hybrid
compression), with the truncation error of both stages fed back (hotdry.top
section 1.1; 5688vip.com section 4.5).

Readings where the pages are open: the 8-bit stage is QSGD with s = 127 levels
(sign plus 7-bit level) over groups of 64 consecutive kept values in ascending index
order; the random draw of kept value j uses element index j (its position in the
kept list); the new residual is c everywhere except at the kept positions, where it
is fl(v - g_hat).
"""
from __future__ import annotations

import numpy as np

from .qsgd import qsgd
from .topk import ef_topk

F32 = np.float32


def ef_topk_qsgd(grad, residual, k, levels=127, group=64, seed=0, index_base=0):
    """Returns (idx int64[k], codes int8[k], norms float32[ceil(k/group)],
    new residual float32[n], kept values float32[k])."""
    idx, val, new_res = ef_topk(grad, residual, k, index_base)
    codes, norms, g_hat, _ = qsgd(val, group, levels, seed, index_base=0)
    new_res[idx - np.int64(index_base)] = (val - g_hat).astype(F32)
    return idx, codes, norms, new_res, val
