"""TernGrad: stochastic ternary codes with a per-layer scale (oracle).

What the pages fix (hotdry.top "gradient-compression-quantization-sparsification",
section 1.1): TernGrad maps every gradient value to one of -1, 0, +1, and normalizes
layer by layer to keep the variance under control.  The page gives no formula; we use
the scheme of the TernGrad paper it cites (Wen et al., NeurIPS 2017), per layer:

    s    = max |x|
    code = sign(x) * b,  b = 1 with probability |x| / s, else 0
    g_hat = code * s      (unbiased: E[g_hat] = x)

Readings where the pages are open:
* p = fl(|x| / s); the draw for element i is the 24-bit Philox uniform U of element
  index index_base + (global position of the element); b = (U < p); s == 0 gives 0;
* "sign" means x < 0;
* packing: 2 bits per element, 0 -> 00, +1 -> 01, -1 -> 11; element 4j+m of a layer
  sits in bits 2m..2m+1 of byte j of that layer's output; unused tail bits are 0;
  layers are packed one after another, layer s starting at byte sum_{j<s} ceil(len_j/4);
* with error feedback: x' = fl(x + e), and the new e = fl(x' - g_hat).

The page quotes "up to 32x" for ternary codes; at 2 bits per element the code bytes
are 1/16 of the fp32 bytes.
"""
from __future__ import annotations

import numpy as np

from .philox import uniform24

F32 = np.float32


def pack_ternary(codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.int8)
    n = codes.size
    bits = np.where(codes == 0, 0, np.where(codes > 0, 1, 3)).astype(np.uint8)
    padded = np.zeros(((n + 3) // 4) * 4, dtype=np.uint8)
    padded[:n] = bits
    q = padded.reshape(-1, 4)
    return (q[:, 0] | (q[:, 1] << 2) | (q[:, 2] << 4) | (q[:, 3] << 6)).astype(np.uint8)


def unpack_ternary(packed: np.ndarray, n: int) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(((n + 3) // 4) * 4, dtype=np.int8)
    for m in range(4):
        b = (packed >> (2 * m)) & 3
        out[m::4] = np.where(b == 0, 0, np.where(b == 1, 1, np.where(b == 3, -1, 99)))[: out[m::4].size]
    return out[:n]


def terngrad(x: np.ndarray, seg_offsets, seed: int, index_base: int = 0,
             residual: np.ndarray | None = None):
    """Returns (packed uint8[sum ceil(len/4)], scales float32[nseg], codes int8[n],
    g_hat float32[n], new residual or None)."""
    x = np.asarray(x, dtype=F32)
    if residual is not None:
        x = (x + np.asarray(residual, dtype=F32)).astype(F32)
    off = np.asarray(seg_offsets, dtype=np.int64)
    nseg = off.size - 1
    scales = np.zeros(nseg, dtype=F32)
    codes = np.zeros(x.size, dtype=np.int8)
    g_hat = np.zeros(x.size, dtype=F32)
    packed = []
    for s in range(nseg):
        a, b = int(off[s]), int(off[s + 1])
        seg = x[a:b]
        if seg.size:
            sc = F32(np.abs(seg).max())
        else:
            sc = F32(0.0)
        scales[s] = sc
        if sc > F32(0.0):
            p = (np.abs(seg) / sc).astype(F32)
            U = uniform24(seed, np.int64(index_base) + np.arange(a, b, dtype=np.int64))
            keep = (U < p)
            c = np.where(keep, np.where(seg < F32(0.0), -1, 1), 0).astype(np.int8)
        else:
            c = np.zeros(seg.size, dtype=np.int8)
        codes[a:b] = c
        g_hat[a:b] = dequant_terngrad(c, sc)
        packed.append(pack_ternary(c))
    packed = np.concatenate(packed) if packed else np.zeros(0, np.uint8)
    new_res = (x - g_hat).astype(F32) if residual is not None else None
    return packed, scales, codes, g_hat, new_res


def dequant_terngrad(codes: np.ndarray, scale) -> np.ndarray:
    """g_hat = code * s: +s, -s or +0.0 (exact)."""
    codes = np.asarray(codes, dtype=np.int8)
    sc = np.asarray(scale, dtype=F32)
    return np.where(codes > 0, sc, np.where(codes < 0, -sc, F32(0.0))).astype(F32)
