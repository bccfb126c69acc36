"""Shared helpers for the tests: building/loading the library and moving arrays."""
import os

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "gradient_compression_ddp_amd", "libgc.so")


def ensure_built():
    """Build libgc.so only if it is not there yet."""
    if not os.path.exists(LIB):
        # by path: importing the package would load the library that is missing
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_gc_build", os.path.join(ROOT, "gradient_compression_ddp_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()
    return LIB


def bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


def assert_bits_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    gb, wb = bits(got), bits(want)
    bad = np.nonzero(gb != wb)[0]
    assert bad.size == 0, (f"{what}: {bad.size} of {gb.size} entries differ; first at {bad[:5]}: "
                           f"got {got.ravel()[bad[:5]]} want {want.ravel()[bad[:5]]}")
