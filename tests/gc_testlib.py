"""Shared helpers for the tests: building/loading the library and moving arrays."""
import os

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "gradient_compression_ddp_amd", "libgc.so")


def ensure_built():
    """Build libgc.so only if it is not there yet.  GC_LIB_PATH, when set, names another
    build of the library to test instead (the host AddressSanitizer build)."""
    if os.environ.get("GC_LIB_PATH"):
        return os.environ["GC_LIB_PATH"]
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


def oracle_qsgd_threaded(v, group, levels, seed, chunks=16):
    """oracle.qsgd over v split at group boundaries into slices that run in threads
    (numpy releases the GIL in its array loops).  Slice [a, b) with a a multiple of the
    group is the oracle's own call at index_base a, so the result is the whole call's."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    ng = (v.size + group - 1) // group
    b = [min((ng * i // chunks) * group, v.size) for i in range(chunks + 1)]
    b[-1] = v.size
    with ThreadPoolExecutor(chunks) as ex:
        parts = list(ex.map(lambda i: oracle.qsgd(v[b[i]:b[i + 1]], group, levels, seed, index_base=b[i]),
                            range(chunks)))
    codes = np.concatenate([p[0] for p in parts])
    norms = np.concatenate([p[1] for p in parts])
    ghat = np.concatenate([p[2] for p in parts])
    return codes, norms, ghat


def oracle_terngrad_layers(x, layer_len, seed, residual=None, threads=8):
    """oracle.terngrad one layer at a time (layer l is the segment [l*L, (l+1)*L) of a
    call whose segments are the layers, so its draws use index_base l*L), in threads.
    Returns (packed per layer concatenated, scales, new residual or None)."""
    from concurrent.futures import ThreadPoolExecutor

    import oracle
    nl = x.size // layer_len

    def one(l):
        sl = slice(l * layer_len, (l + 1) * layer_len)
        res = None if residual is None else residual[sl]
        pk, sc, _, _, nr = oracle.terngrad(x[sl], [0, layer_len], seed, index_base=l * layer_len, residual=res)
        return pk, sc[0], nr

    with ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(one, range(nl)))
    packed = np.concatenate([p[0] for p in parts])
    scales = np.array([p[1] for p in parts], dtype=np.float32)
    new_r = None if residual is None else np.concatenate([p[2] for p in parts])
    return packed, scales, new_r
