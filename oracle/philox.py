"""Counter-based RNG of the oracle: Philox4x32 with 10 rounds.

Definition: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel Random
Numbers: As Easy as 1, 2, 3", SC'11, section on the Philox family.  One block maps
a 128-bit counter (x0, x1, x2, x3) and a 64-bit key (k0, k1) to four 32-bit words.
Each round takes the two 32x32->64 products M0*x0 and M1*x2, and forms
    (hi(M1*x2) ^ x1 ^ k0,  lo(M1*x2),  hi(M0*x0) ^ x3 ^ k1,  lo(M0*x0));
between rounds the key is bumped by the Weyl constants (W0, W1) modulo 2^32.

Stochastic rounding needs one uniform per element, keyed on (seed, element index).
The pages only ask that stochastic rounding be unbiased (hotdry.top
"gradient-compression-quantization-sparsification", section 1.1 on QSGD) and
that it be reproducible from a seed; this layout is our reading:

    key     = (low 32 bits of seed, high 32 bits of seed)
    counter = (low 32 bits of e>>2, high 32 bits of e>>2, 0, 0)
    word    = output word number (e & 3) of that block
    U       = (word >> 8) * 2^-24        (24-bit uniform in [0, 1), exact in fp32)

Pinned in tests against rocRAND's host-callable Philox4x32-10 engine.
"""
from __future__ import annotations

import numpy as np

M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = np.uint64(0x9E3779B9)
W1 = np.uint64(0xBB67AE85)
MASK32 = np.uint64(0xFFFFFFFF)
SHIFT32 = np.uint64(32)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Apply ten Philox4x32 rounds.  Inputs are arrays/scalars of 32-bit values.

    Returns four uint32 arrays.  Arithmetic is done in uint64 so that each 32x32
    product is exact; every value is masked back to 32 bits.
    """
    x0 = np.asarray(c0, dtype=np.uint64) & MASK32
    x1 = np.asarray(c1, dtype=np.uint64) & MASK32
    x2 = np.asarray(c2, dtype=np.uint64) & MASK32
    x3 = np.asarray(c3, dtype=np.uint64) & MASK32
    ka = np.uint64(int(k0) & 0xFFFFFFFF)
    kb = np.uint64(int(k1) & 0xFFFFFFFF)
    x0, x1, x2, x3 = np.broadcast_arrays(x0, x1, x2, x3)
    for rnd in range(10):
        p0 = x0 * M0
        p1 = x2 * M1
        hi0, lo0 = p0 >> SHIFT32, p0 & MASK32
        hi1, lo1 = p1 >> SHIFT32, p1 & MASK32
        x0, x1, x2, x3 = hi1 ^ x1 ^ ka, lo1, hi0 ^ x3 ^ kb, lo0
        ka = (ka + W0) & MASK32
        kb = (kb + W1) & MASK32
    return (x0.astype(np.uint32), x1.astype(np.uint32),
            x2.astype(np.uint32), x3.astype(np.uint32))


def random_words(seed: int, e) -> np.ndarray:
    """The 32-bit Philox word assigned to each element index in ``e`` (int64 >= 0)."""
    e = np.asarray(e, dtype=np.int64).astype(np.uint64)
    ctr = e >> np.uint64(2)
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    w = philox4x32_10(ctr & MASK32, ctr >> SHIFT32, 0, 0, seed & 0xFFFFFFFF, seed >> 32)
    which = (e & np.uint64(3)).astype(np.int64)
    out = np.choose(which, w) if which.ndim else w[int(which)]
    return np.asarray(out, dtype=np.uint32)


def uniform24(seed: int, e) -> np.ndarray:
    """float32 uniform in [0, 1) with 24 random bits, for element indices ``e``."""
    w = random_words(seed, e)
    return ((w >> np.uint32(8)).astype(np.float32) * np.float32(2.0 ** -24)).astype(np.float32)
