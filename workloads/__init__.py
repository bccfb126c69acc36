"""Seeded synthetic inputs shared by the tests, the bench and the CPU oracle checks.

This module only draws random numbers and lays them out. It holds none of the
compression arithmetic, so both the HIP path and the oracle can be fed from it
without sharing any of the method's code.

Recipes (host side, numpy ``default_rng``; every multiply by a scale is fp32):

* ``ef_demo_gradients`` -- the 1,000,000-element N(0,1) gradient of the numpy demo
  on the aiqz.cc page "梯度聚合通信优化实战方案" (section "Python 演示", function
  ``simulate_gradients``: seed 42, float32), plus a second step drawn from seed 43
  and multiplied by float32(0.9), as the demo's second error-feedback call scales
  its gradient by 0.9.
* ``student_t`` -- Student-t with 3 degrees of freedom, drawn as
  Z0 / sqrt((Z1^2 + Z2^2 + Z3^2) / 3) from four independent standard normals in
  float64 and rounded once to float32.  This is the textbook construction of a
  t(3) variate; it is exact in distribution and about four times cheaper than
  ``Generator.standard_t`` in numpy.
* layered gradients: per-layer t(3) times a lognormal(-7, 1) per-layer scale.

Device-side recipes (``*_torch``) use torch's seeded CUDA generator with the same
constructions; they exist because a 7e9-element gradient takes tens of core-minutes
to draw on the host.  Device and host draws are different numbers; every test feeds
the same bytes to both sides.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32

# Sizes of the five workloads.
DEMO_N = 1_000_000
DEMO_K = 10_000
BUCKET_N = 6_553_600            # one 25 MiB DDP bucket of fp32
BUCKET_GROUP = 64
TERN_LAYERS = 24
TERN_LAYER_LEN = 14_583_333     # 24 x 14,583,333 = 349,999,992 (~350M parameters)
PSGD_SHAPES = ((4096, 4096), (4096, 11008), (11008, 4096))
PSGD_RANK = 4
BIG_LAYERS = 32
BIG_LAYER_LEN = 218_750_000     # 32 x 218,750,000 = 7e9
BIG_K = 70_000_000              # 1% of 7e9


def ef_demo_gradients(n: int = DEMO_N):
    """Step-1 and step-2 gradients of the 1M-element demo workload."""
    g1 = np.random.default_rng(42).standard_normal(n).astype(F32)
    g2 = F32(0.9) * np.random.default_rng(43).standard_normal(n).astype(F32)
    return g1, g2.astype(F32)


def student_t(rng: np.random.Generator, n: int) -> np.ndarray:
    """t(3) variates, float32, from four standard normals per value."""
    z = rng.standard_normal((4, n))
    chi2 = z[1] * z[1] + z[2] * z[2] + z[3] * z[3]
    return (z[0] / np.sqrt(chi2 / 3.0)).astype(F32)


def bucket(n: int = BUCKET_N, seed: int = 2) -> np.ndarray:
    """One DDP bucket: t(3) scaled by float32(1e-3)."""
    return (student_t(np.random.default_rng(seed), n) * F32(1e-3)).astype(F32)


def layer_scales(seed: int, n_layers: int) -> np.ndarray:
    return np.random.default_rng(seed).lognormal(-7.0, 1.0, n_layers).astype(F32)


def layered(seed: int, n_layers: int, layer_len: int, step: int | None = None):
    """Concatenated layers, each t(3) times its lognormal(-7,1) scale.

    Returns (flat float32 array, int64 offsets of length n_layers+1).
    Layer l is drawn from default_rng([seed, l]) (or [seed, step, l] when a step
    index is given), so a layer can be regenerated on its own.
    """
    scales = layer_scales(seed, n_layers)
    out = np.empty(n_layers * layer_len, dtype=F32)
    for l in range(n_layers):
        key = [seed, l] if step is None else [seed, step, l]
        out[l * layer_len:(l + 1) * layer_len] = (
            student_t(np.random.default_rng(key), layer_len) * scales[l])
    offsets = np.arange(n_layers + 1, dtype=np.int64) * layer_len
    return out, offsets


def tern_layers(n_layers: int = TERN_LAYERS, layer_len: int = TERN_LAYER_LEN, seed: int = 3):
    return layered(seed, n_layers, layer_len)


def psgd_gradient(step: int, j: int, shape) -> np.ndarray:
    """PowerSGD gradient matrix j at step t: entries N(0, variance 1e-4)."""
    rows, cols = shape
    return np.random.default_rng([4, step, j]).normal(0.0, 1e-2, (rows, cols)).astype(F32)


def psgd_initial_q(shapes=PSGD_SHAPES, rank: int = PSGD_RANK, seed: int = 11):
    """Initial Q for each matrix, drawn in order from one default_rng(11) stream."""
    rng = np.random.default_rng(seed)
    return [rng.standard_normal((cols, rank)).astype(F32) for (_, cols) in shapes]


def big_layers_host(n_layers: int, layer_len: int, step: int, seed: int = 5):
    """Scaled-down host version of the 7e9 workload (same recipe, smaller layers)."""
    return layered(seed, n_layers, layer_len, step=step)


# ---------------------------------------------------------------------------
# Device-side generators (torch).  Imported lazily so that CPU-only users of this
# module never need a GPU.
# ---------------------------------------------------------------------------

def student_t_torch(n: int, generator, device, out=None):
    """t(3) on the device: Z0 / sqrt((Z1^2+Z2^2+Z3^2)/3), computed in float32."""
    import torch
    z = torch.randn((4, n), generator=generator, device=device, dtype=torch.float32)
    chi2 = z[1] * z[1] + z[2] * z[2] + z[3] * z[3]
    t = z[0] / torch.sqrt(chi2 / 3.0)
    if out is None:
        return t
    out.copy_(t)
    return out


def layered_torch(n_layers: int, layer_len: int, step: int, device, seed: int = 5,
                  out=None, chunk: int = 1 << 26):
    """Device version of the layered workload.

    Layer l of step t is drawn from a torch CUDA generator seeded with
    seed * 1_000_003 + t * 1009 + l, in chunks, then multiplied by the host-drawn
    lognormal scale of layer l (float32 multiply).
    """
    import torch
    scales = layer_scales(seed, n_layers)
    n = n_layers * layer_len
    if out is None:
        out = torch.empty(n, dtype=torch.float32, device=device)
    gen = torch.Generator(device=device)
    for l in range(n_layers):
        gen.manual_seed(seed * 1_000_003 + step * 1009 + l)
        base = l * layer_len
        done = 0
        while done < layer_len:
            m = min(chunk, layer_len - done)
            view = out[base + done: base + done + m]
            student_t_torch(m, gen, device, out=view)
            view.mul_(float(scales[l]))
            done += m
    return out
