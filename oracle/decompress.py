"""Decompression at the receiver (oracle): dense decode or scatter of a payload.

What the pages fix (zyxy.net/archives/25733 "分布式训练中的梯度压缩算法", section 四:
each worker decompresses what it received before updating; section 二.2: the
sparsified gradient is the dense vector with the unkept entries set to 0).

For every payload kind the value of entry j is the dequantization formula of the
matching compressor (fp32, no FMA):
    F32      v_j
    MINMAX8  fl(fl(q_j * scale_g) + min_g)           q_j an 8-bit code
    MINMAX4  the same with 4-bit codes, two per byte (low nibble first)
    QSGD     sign * fl(fl(nu_g * |code_j|) / s)
    TERN     code_j * scale_g                         (2-bit codes, four per byte)
where g = j // group (group 0: one group).  The value is then multiplied by alpha
(fl) and either stored to or added (fl) into out[pos_j], pos_j = idx_j - index_base
for a scatter, or j for a dense decode.
"""
from __future__ import annotations

import numpy as np

from .minmax import dequant_minmax, unpack_int4
from .qsgd import dequant_qsgd
from .terngrad import unpack_ternary

F32 = np.float32
KIND_F32, KIND_MINMAX8, KIND_MINMAX4, KIND_QSGD, KIND_TERN = 0, 1, 2, 3, 4


def _values(kind, codes, count, meta0, meta1, group, levels):
    g = count if group == 0 else group
    if kind == KIND_F32:
        return np.asarray(codes, dtype=F32)[:count].copy()
    if kind == KIND_MINMAX8:
        return dequant_minmax(np.asarray(codes, np.uint8)[:count], meta0, meta1, g)
    if kind == KIND_MINMAX4:
        return dequant_minmax(unpack_int4(codes, count), meta0, meta1, g)
    if kind == KIND_QSGD:
        return dequant_qsgd(np.asarray(codes, np.int8)[:count], meta0, g, levels)
    if kind == KIND_TERN:
        c = unpack_ternary(codes, count)
        sc = np.asarray(meta0, dtype=F32)[np.arange(count, dtype=np.int64) // max(g, 1)]
        return np.where(c > 0, sc, np.where(c < 0, -sc, F32(0.0))).astype(F32)
    raise ValueError("unknown kind")


def decompress_scatter(kind, idx, count, index_base, codes, meta0, meta1, group, levels,
                       alpha, accumulate, out):
    """Apply one payload to ``out`` (float32, modified in place) and return it."""
    v = _values(kind, codes, count, meta0, meta1, group, levels)
    v = (v * F32(alpha)).astype(F32)
    pos = np.arange(count, dtype=np.int64) if idx is None else (
        np.asarray(idx, np.int64)[:count] - np.int64(index_base))
    if accumulate:
        out[pos] = (out[pos] + v).astype(F32)
    else:
        out[pos] = v
    return out
