"""Min-max (linear) quantization with deterministic rounding (oracle).

What the pages fix (zyxy.net/archives/25733 "分布式训练中的梯度压缩算法", section
二.1 "线性量化": formulas and ``linear_quantize``; section 三 error-compensation
example ``quantize_with_error_compensation``; aiqz.cc "梯度聚合通信优化实战方案",
section "Python 演示", ``quantize``):

    scale = (max - min) / (2^b - 1)
    q     = round((g - min) / scale)
    g_hat = q * scale + min
    with error compensation: g' = g + e, and the new e = g' - g_hat.

Per-group quantization (e.g. 64 elements per group) is the grouping strategy of
hotdry.top "gradient-compression-quantization-sparsification", section 1.2.

Readings where the pages are open:
* every step is one float32 operation: rng = fl(max - min), scale = fl(rng / L),
  q = rint(fl(fl(x - min) / scale)) clipped to [0, L], g_hat = fl(fl(q*scale) + min);
* divide by scale (the linear-quantization section and the demo), with no epsilon
  (the 5688vip.com page's ``+1e-8`` variant is not used); scale == 0 gives q = 0;
* codes are unsigned, 0..2^b-1 (the demo's cast to int8 overflows above 127);
  int4 codes pack two per byte, element 2j in the low nibble;
* metadata per group is (min, scale) in float32; the last group may be partial;
  group 0 means one group over the whole tensor;
* min and max follow the IEEE total order, in which -0 < +0, so the sign of a zero
  minimum is defined.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32


def _total_order_key(v: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(v, dtype=F32).view(np.uint32)
    return np.where(b & np.uint32(0x80000000), ~b, b | np.uint32(0x80000000))


def _groups(n: int, group: int):
    g = n if group == 0 else group
    if n == 0:
        return 0, max(g, 1)
    return (n + g - 1) // g, g


def quant_minmax(x: np.ndarray, group: int, bits: int, residual: np.ndarray | None = None):
    """Quantize x (plus residual, if given) per group.

    Returns (codes uint8[n] in 0..2^bits-1, mins float32[ng], scales float32[ng],
    g_hat float32[n], new residual float32[n] or None).
    """
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    x = np.asarray(x, dtype=F32)
    if residual is not None:
        x = (x + np.asarray(residual, dtype=F32)).astype(F32)
    n = x.size
    ng, g = _groups(n, group)
    L = F32(2 ** bits - 1)
    codes = np.zeros(n, dtype=np.uint8)
    mins = np.zeros(ng, dtype=F32)
    scales = np.zeros(ng, dtype=F32)
    g_hat = np.zeros(n, dtype=F32)
    for j in range(ng):
        seg = x[j * g:(j + 1) * g]
        key = _total_order_key(seg)
        mn = seg[np.argmin(key)]
        mx = seg[np.argmax(key)]
        rng = F32(mx - mn)
        scale = F32(rng / L)
        if scale == F32(0.0):
            q = np.zeros(seg.size, dtype=F32)
        else:
            q = np.clip(np.rint((seg - mn).astype(F32) / scale), F32(0.0), L).astype(F32)
        codes[j * g:(j + 1) * g] = q.astype(np.uint8)
        mins[j] = mn
        scales[j] = scale
        g_hat[j * g:(j + 1) * g] = ((q * scale).astype(F32) + mn).astype(F32)
    new_res = (x - g_hat).astype(F32) if residual is not None else None
    return codes, mins, scales, g_hat, new_res


def dequant_minmax(codes: np.ndarray, mins: np.ndarray, scales: np.ndarray, group: int,
                   positions: np.ndarray | None = None) -> np.ndarray:
    """g_hat = fl(fl(q*scale) + min) with the group of each code taken from its position."""
    codes = np.asarray(codes)
    n = codes.size
    pos = np.arange(n, dtype=np.int64) if positions is None else np.asarray(positions, np.int64)
    g = n if group == 0 else group
    gid = pos // max(g, 1)
    q = codes.astype(F32)
    return ((q * scales[gid]).astype(F32) + mins[gid]).astype(F32)


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Two 4-bit codes per byte: byte j = q[2j] | q[2j+1] << 4; an odd tail leaves 0 above."""
    codes = np.asarray(codes, dtype=np.uint8)
    n = codes.size
    out = np.zeros((n + 1) // 2, dtype=np.uint8)
    out[:] = codes[0::2]
    out[: n // 2] |= (codes[1::2] << 4).astype(np.uint8)
    return out


def unpack_int4(packed: np.ndarray, n: int) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(n, dtype=np.uint8)
    out[0::2] = packed[: (n + 1) // 2] & 0xF
    out[1::2] = packed[: n // 2] >> 4
    return out
