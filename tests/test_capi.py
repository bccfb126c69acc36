"""The C ABI without a GPU: the library loads, exports every symbol include/gc.h declares,
and rejects bad arguments on the host before any HIP call (no compute is launched)."""
import ctypes
import os
import re

import pytest

from gc_testlib import ROOT, ensure_built

HEADER = os.path.join(ROOT, "include", "gc.h")


@pytest.fixture(scope="module")
def lib():
    path = ensure_built()
    lib = ctypes.CDLL(path)
    lib.gc_status_string.restype = ctypes.c_char_p
    lib.gc_last_error.restype = ctypes.c_char_p
    return lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gc_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"gc_ef_topk", "gc_quant_minmax", "gc_qsgd", "gc_terngrad", "gc_powersgd_step",
            "gc_decompress_scatter"} <= set(names)
    for name in names:
        assert hasattr(lib, name), f"libgc.so does not export {name}"


def test_status_strings_and_version(lib):
    lib.gc_status_string.restype = ctypes.c_char_p
    lib.gc_last_error.restype = ctypes.c_char_p
    assert lib.gc_status_string(0) == b"GC_OK"
    assert b"EINVAL" in lib.gc_status_string(1)
    assert b"unknown" in lib.gc_status_string(99)
    assert lib.gc_version() >= 100


def _ws(lib, op, n, k, aux):
    out = ctypes.c_size_t(7)
    st = lib.gc_workspace_size(op, ctypes.c_int64(n), ctypes.c_int64(k), ctypes.c_int64(aux), ctypes.byref(out))
    return st, out.value


def test_workspace_sizes(lib):
    st, b = _ws(lib, 1, 7_000_000_000, 70_000_000, 127)
    assert st == 0 and 1 << 30 < b < 8 << 30          # a few GB of candidate pool for the 7e9 case
    st, b = _ws(lib, 1, 1_000_000, 10_000, 0)
    assert st == 0 and b > 0
    assert _ws(lib, 1, 100, 0, 0) == (0, 0)
    assert _ws(lib, 1, 100, 101, 0)[0] == 1            # k > n
    assert _ws(lib, 2, 6_553_600, 64, 0) == (0, 0)     # small groups need no workspace
    st, b = _ws(lib, 2, 1_000_000, 0, 0)
    assert st == 0 and b >= 8
    assert _ws(lib, 2, 100, 3, 0)[0] == 1              # group < 4
    assert _ws(lib, 99, 1, 1, 1)[0] == 1


VP = ctypes.c_void_p
FAKE = VP(0x100000)     # never dereferenced: every call below fails validation first
MISALIGNED = VP(0x100004)


def test_ef_topk_rejects_bad_arguments(lib):
    lib.gc_last_error.restype = ctypes.c_char_p
    f = lib.gc_ef_topk
    f.argtypes = [VP, VP, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, VP, VP, ctypes.c_int,
                  ctypes.c_int64, ctypes.c_uint64, VP, VP, VP, ctypes.c_size_t, VP]
    assert f(FAKE, FAKE, 10, 11, 0, FAKE, FAKE, 0, 64, 0, None, None, FAKE, 1 << 20, None) == 1
    assert b"k must" in lib.gc_last_error()
    assert f(None, FAKE, 10, 1, 0, FAKE, FAKE, 0, 64, 0, None, None, FAKE, 1 << 20, None) == 1
    assert f(MISALIGNED, FAKE, 10, 1, 0, FAKE, FAKE, 0, 64, 0, None, None, FAKE, 1 << 20, None) == 1
    assert f(FAKE, FAKE, 10, 1, 0, FAKE, None, 0, 64, 0, None, None, FAKE, 1 << 20, None) == 1
    assert f(FAKE, FAKE, 10, 1, 0, FAKE, FAKE, 200, 64, 0, FAKE, FAKE, FAKE, 1 << 20, None) == 1
    assert f(FAKE, FAKE, 10, 1, 0, FAKE, FAKE, 127, 48, 0, FAKE, FAKE, FAKE, 1 << 20, None) == 1
    assert f(FAKE, FAKE, 10, 1, -1, FAKE, FAKE, 0, 64, 0, None, None, FAKE, 1 << 20, None) == 1
    assert f(FAKE, FAKE, 10, 1, 0, FAKE, FAKE, 0, 64, 0, None, None, None, 0, None) == 2
    assert f(FAKE, FAKE, 10, 1, 0, FAKE, FAKE, 0, 64, 0, None, None, FAKE, 16, None) == 2
    assert f(FAKE, FAKE, -1, 0, 0, FAKE, FAKE, 0, 64, 0, None, None, None, 0, None) == 1
    # n == 0 is a no-op that needs no pointers at all
    assert f(None, None, 0, 0, 0, None, None, 0, 64, 0, None, None, None, 0, None) == 0


def test_ef_randk_rejects_bad_arguments(lib):
    lib.gc_last_error.restype = ctypes.c_char_p
    f = lib.gc_ef_randk
    f.argtypes = [VP, VP, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_uint64, VP, VP, ctypes.c_int,
                  ctypes.c_int64, ctypes.c_uint64, VP, VP, VP, ctypes.c_size_t, VP]
    assert f(FAKE, FAKE, 10, 11, 0, 3, FAKE, FAKE, 0, 64, 0, None, None, FAKE, 1 << 20, None) == 1
    assert b"k must" in lib.gc_last_error()
    assert f(FAKE, MISALIGNED, 10, 1, 0, 3, FAKE, FAKE, 0, 64, 0, None, None, FAKE, 1 << 20, None) == 1
    assert f(FAKE, FAKE, 10, 1, 0, 3, None, FAKE, 0, 64, 0, None, None, FAKE, 1 << 20, None) == 1
    assert f(FAKE, FAKE, 10, 1, 0, 3, FAKE, FAKE, 127, 64, 0, None, FAKE, FAKE, 1 << 20, None) == 1
    assert f(FAKE, FAKE, 10, 1, 1 << 62, 3, FAKE, FAKE, 0, 64, 0, None, None, FAKE, 1 << 20, None) == 1
    assert f(FAKE, FAKE, 10, 1, 0, 3, FAKE, FAKE, 0, 64, 0, None, None, None, 0, None) == 2
    assert f(None, None, 0, 0, 0, 3, None, None, 0, 64, 0, None, None, None, 0, None) == 0
    # the Random-K candidate pool also keeps each candidate's value: more workspace than
    # Top-K of the same size, at every size
    for n, k in ((50_000_000, 500_000), (5_000_000, 50_000), (1000, 10)):
        st_t, b_t = _ws(lib, 1, n, k, 0)
        st_r, b_r = _ws(lib, 7, n, k, 0)
        assert st_t == 0 and st_r == 0 and b_r > b_t
    assert _ws(lib, 7, 100, 0, 0) == (0, 0)
    assert _ws(lib, 7, 100, 101, 0)[0] == 1


def test_deferred_calls_reject_bad_arguments(lib):
    f = lib.gc_ef_topk_deferred
    f.argtypes = [VP, VP, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, VP, VP, ctypes.c_int, ctypes.c_int64,
                  ctypes.c_uint64, VP, VP, VP, ctypes.c_size_t, VP, ctypes.c_size_t, VP]
    st, need = _ws(lib, 8, 100_000, 1000, 0)
    assert st == 0 and need > 0
    # the record grows by one 512-byte chunk per 64 entries of k
    assert _ws(lib, 8, 100_000, 1000 + 64 * 10, 0)[1] - need == 10 * 512
    assert _ws(lib, 8, 100, 101, 0)[0] == 1
    args = (FAKE, FAKE, 100_000, 1000, 0, FAKE, FAKE, 0, 64, 0, None, None)
    assert f(*args, None, need, FAKE, 1 << 30, None) == 1                       # no record
    assert f(*args, MISALIGNED, need, FAKE, 1 << 30, None) == 1                 # misaligned record
    assert f(*args, VP(0x200000), need - 1, FAKE, 1 << 30, None) == 2           # record too small
    assert f(*args, VP(0x200000), need, None, 0, None) == 2                     # no workspace
    assert f(FAKE, FAKE, 100_000, 100_001, 0, FAKE, FAKE, 0, 64, 0, None, None, FAKE, need, FAKE, 1 << 30,
             None) == 1                                                          # k > n
    fl = lib.gc_ef_flush
    fl.argtypes = [VP, ctypes.c_int64, VP, ctypes.c_size_t, VP]
    assert fl(MISALIGNED, 100_000, VP(0x200000), need, None) == 1
    assert fl(FAKE, 100_000, None, need, None) == 1
    assert fl(FAKE, 100_000, VP(0x200000), 16, None) == 2
    assert fl(None, 0, None, 0, None) == 0


def test_ef_compress_rejects_bad_options(lib):
    import gradient_compression_ddp_amd as gcm
    f = lib.gc_ef_compress
    f.argtypes = [VP, VP, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, VP, VP, ctypes.c_int, ctypes.c_int64,
                  ctypes.c_uint64, VP, VP, ctypes.POINTER(gcm.EfOptions), VP, ctypes.c_size_t, VP]
    assert ctypes.sizeof(gcm.EfOptions) == 40
    args = (FAKE, FAKE, 100_000, 1000, 0, FAKE, FAKE, 0, 64, 0, None, None)
    o = gcm.EfOptions(size=ctypes.sizeof(gcm.EfOptions), select=2)
    assert f(*args, ctypes.byref(o), FAKE, 1 << 30, None) == 1                     # unknown selector
    o = gcm.EfOptions(size=8)
    assert f(*args, ctypes.byref(o), FAKE, 1 << 30, None) == 1                     # struct too small
    o = gcm.EfOptions(size=ctypes.sizeof(gcm.EfOptions), stats=0x100004)
    assert f(*args, ctypes.byref(o), FAKE, 1 << 30, None) == 1                     # misaligned stats
    o = gcm.EfOptions(size=ctypes.sizeof(gcm.EfOptions), stats=0x100000)
    assert f(FAKE, FAKE, 100_000, 0, 0, FAKE, FAKE, 0, 64, 0, None, None, ctypes.byref(o), None, 0, None) == 1
    assert b"k > 0" in lib.gc_last_error()
    o = gcm.EfOptions(size=ctypes.sizeof(gcm.EfOptions), select=1)
    big = (FAKE, FAKE, 50_000_000, 500_000, 0, FAKE, FAKE, 0, 64, 0, None, None)
    need_t = _ws(lib, 1, 50_000_000, 500_000, 0)[1]
    assert f(*big, ctypes.byref(o), FAKE, need_t, None) == 2                       # Random-K needs more
    assert f(*big, ctypes.byref(o), FAKE, need_t - 256, None) == 2
    o = gcm.EfOptions(size=ctypes.sizeof(gcm.EfOptions), pending=0x200000, pending_bytes=64)
    assert f(*args, ctypes.byref(o), FAKE, 1 << 30, None) == 2                     # record too small


def test_other_calls_reject_bad_arguments(lib):
    q = lib.gc_quant_minmax
    q.argtypes = [VP, VP, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, VP, VP, VP, VP, ctypes.c_size_t, VP]
    assert q(FAKE, None, 100, 64, 7, FAKE, FAKE, FAKE, None, 0, None) == 1        # bits
    assert q(FAKE, None, 100, 48, 8, FAKE, FAKE, FAKE, None, 0, None) == 1        # group not a power of two
    assert q(FAKE, None, 100, 0, 8, FAKE, FAKE, FAKE, None, 0, None) == 2         # whole tensor needs workspace
    s = lib.gc_qsgd
    s.argtypes = [VP, VP, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_uint64, ctypes.c_int64, VP, VP, VP]
    assert s(FAKE, None, 100, 64, 0, 7, 0, FAKE, FAKE, None) == 1                 # levels
    assert s(FAKE, None, 100, 512, 15, 7, 0, FAKE, FAKE, None) == 1               # group too large
    t = lib.gc_terngrad
    t.argtypes = [VP, VP, ctypes.c_int, VP, ctypes.c_uint64, ctypes.c_int64, VP, VP, VP, ctypes.c_size_t, VP]
    bad = (ctypes.c_int64 * 3)(0, 10, 5)
    assert t(FAKE, None, 2, ctypes.cast(bad, VP), 3, 0, FAKE, FAKE, None, 0, None) == 1
    first = (ctypes.c_int64 * 2)(1, 10)
    assert t(FAKE, None, 1, ctypes.cast(first, VP), 3, 0, FAKE, FAKE, None, 0, None) == 1
    p = lib.gc_powersgd_step
    p.argtypes = [VP, VP, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, VP, VP, VP, ctypes.c_size_t, VP]
    assert p(FAKE, None, 64, 62, 4, FAKE, FAKE, FAKE, 1 << 20, None) == 1         # cols % 4
    assert p(FAKE, None, 64, 64, 5, FAKE, FAKE, FAKE, 1 << 20, None) == 1         # rank
    d = lib.gc_decompress_scatter
    d.argtypes = [ctypes.c_int, VP, ctypes.c_int64, ctypes.c_int64, VP, VP, VP, ctypes.c_int64, ctypes.c_int,
                  ctypes.c_float, ctypes.c_int, VP, ctypes.c_int64, VP]
    assert d(9, None, 10, 0, FAKE, FAKE, FAKE, 0, 0, 1.0, 0, FAKE, 10, None) == 1  # kind
    assert d(0, None, 11, 0, FAKE, None, None, 0, 0, 1.0, 0, FAKE, 10, None) == 1  # dense overrun
    assert d(3, None, 10, 0, FAKE, FAKE, None, 64, 0, 1.0, 0, FAKE, 10, None) == 1  # QSGD levels
    assert d(1, None, 10, 0, FAKE, FAKE, None, 64, 0, 1.0, 0, FAKE, 10, None) == 1  # min-max meta1


# ---- wire format and the receive side (host checks only) ---------------------------

def _hdr_mod():
    import gradient_compression_ddp_amd as gcm
    return gcm


def test_payload_layout_sections(lib):
    gcm = _hdr_mod()
    code_len = {gcm.KIND_F32: lambda c: 4 * c, gcm.KIND_MINMAX8: lambda c: c, gcm.KIND_MINMAX4: lambda c: (c + 1) // 2,
                gcm.KIND_QSGD: lambda c: c, gcm.KIND_TERN: lambda c: (c + 3) // 4}
    for kind in code_len:
        for count, group, sparse in ((0, 0, False), (1, 0, False), (1001, 64, False), (70_001, 1000, True),
                                     (12_345, 0, True)):
            h = gcm.payload_layout(kind, 10 ** 6, count, group, 15 if kind == gcm.KIND_QSGD else 0, sparse, 7)
            assert (h.magic, h.version, h.kind, h.count, h.group) == (gcm.PAYLOAD_MAGIC, 1, kind, count, group)
            g = group if group else max(count, 1)
            ng = 0 if count == 0 else -(-count // g)
            sections = []
            if sparse:
                sections.append((h.off_idx, 8 * count))
            else:
                assert h.off_idx == 0
            sections.append((h.off_codes, code_len[kind](count)))
            if kind == gcm.KIND_F32:
                assert h.off_meta0 == 0 and h.off_meta1 == 0
            else:
                sections.append((h.off_meta0, 4 * ng))
            if kind in (gcm.KIND_MINMAX8, gcm.KIND_MINMAX4):
                sections.append((h.off_meta1, 4 * ng))
            else:
                assert h.off_meta1 == 0
            end = 128
            for off, size in sections:          # aligned, in order, not overlapping
                assert off % 256 == 0 and off >= end
                end = off + size
            assert h.bytes >= end and h.bytes % 256 == 0 and h.bytes - end < 256
            assert bytes(h.reserved) == bytes(40)


def test_payload_layout_rejects(lib):
    gcm = _hdr_mod()
    h = gcm.PayloadHeader()
    f = gcm._lib.gc_payload_layout
    assert f(9, 10, 5, 0, 0, 0, 0, ctypes.byref(h)) == 1           # kind
    assert f(gcm.KIND_F32, 10, 11, 0, 0, 0, 0, ctypes.byref(h)) == 1   # count > n
    assert f(gcm.KIND_QSGD, 10, 5, 0, 0, 0, 0, ctypes.byref(h)) == 1   # QSGD levels
    assert f(gcm.KIND_F32, 10, 5, -1, 0, 0, 0, ctypes.byref(h)) == 1   # group
    assert f(gcm.KIND_F32, 10, 5, 0, 0, 0, 0, None) == 1               # no header


def test_decompress_payloads_rejects_before_any_launch(lib):
    gcm = _hdr_mod()
    good = gcm.payload_layout(gcm.KIND_QSGD, 1000, 1000, 64, 15)
    fake = 1 << 20                                    # never dereferenced: every call below is invalid
    out = ctypes.c_void_p(fake)

    def call(W, headers, ptrs, n_out=1000, out_ptr=out):
        P = (ctypes.c_void_p * max(W, 1))(*ptrs)
        H = (gcm.PayloadHeader * max(W, 1))(*headers)
        return gcm._lib.gc_decompress_payloads(W, ctypes.cast(P, ctypes.POINTER(ctypes.c_void_p)), H, 1.0, 0,
                                               out_ptr, n_out, None)
    assert call(0, [good], [fake]) == 1                              # W
    bad = gcm.PayloadHeader.from_buffer_copy(bytes(good)); bad.magic = 0
    assert call(1, [bad], [fake]) == 1                               # magic
    bad = gcm.PayloadHeader.from_buffer_copy(bytes(good)); bad.off_meta0 += 256
    assert call(1, [bad], [fake]) == 1                               # offsets differ from the layout
    bad = gcm.PayloadHeader.from_buffer_copy(bytes(good)); bad.flags = 2
    assert call(1, [bad], [fake]) == 1                               # unknown flag
    assert call(1, [good], [fake + 16]) == 1                         # payload not 256-byte aligned
    assert call(1, [good], [None]) == 1                              # payload NULL
    assert call(1, [good], [fake], n_out=999) == 1                   # n > n_out
    assert call(2, [good, bad], [fake, fake]) == 1                   # any bad header rejects the call
    assert call(1, [good], [fake], out_ptr=ctypes.c_void_p(fake + 2)) == 1   # out misaligned


def test_terngrad_workspace_is_sized_and_checked(lib):
    """gc_terngrad keeps two sets of 64 partial maxima per segment and the per-tile lists of
    unsettled bytes in the caller's workspace: the size query reports it, and a missing or
    short workspace is rejected before any launch."""
    size = lib.gc_workspace_size
    size.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t)]
    b = ctypes.c_size_t(0)
    assert size(4, 1000, 3, 0, ctypes.byref(b)) == 0 and b.value >= 2 * 3 * 64 * 4 + 128 * 20 and b.value % 256 == 0
    assert size(4, 0, 3, 0, ctypes.byref(b)) == 0 and b.value == 0        # nothing to do, no workspace
    t = lib.gc_terngrad
    t.argtypes = [VP, VP, ctypes.c_int, VP, ctypes.c_uint64, ctypes.c_int64, VP, VP, VP, ctypes.c_size_t, VP]
    off = (ctypes.c_int64 * 4)(0, 400, 700, 1000)
    assert t(FAKE, None, 3, ctypes.cast(off, VP), 3, 0, FAKE, FAKE, None, 0, None) == 2          # GC_EWORKSPACE
    assert t(FAKE, None, 3, ctypes.cast(off, VP), 3, 0, FAKE, FAKE, FAKE, 256, None) == 2        # too small
    assert b"workspace" in lib.gc_last_error()


def test_stream_floor_rejects_on_the_host(lib):
    f = lib.gc_stream_floor
    f.argtypes = [VP, VP, ctypes.c_int64, VP]
    lib.gc_last_error.restype = ctypes.c_char_p
    assert f(None, None, 0, None) == 0                      # nothing to do
    assert f(None, FAKE, 10, None) == 1
    assert f(MISALIGNED, FAKE, 10, None) == 1
    assert b"16-byte" in lib.gc_last_error()
    assert f(FAKE, VP(FAKE.value + 2), 10, None) == 1                 # out not 4-byte aligned
    assert f(FAKE, FAKE, -1, None) == 1


def test_noalloc_rejects_on_the_host(lib):
    # gc_ef_compress_noalloc validates like gc_ef_compress, then refuses any call whose
    # workspace would not fit its fixed array, all before its first HIP call
    lib.gc_last_error.restype = ctypes.c_char_p
    lib.gc_noalloc_scratch_bytes.restype = ctypes.c_size_t
    f = lib.gc_ef_compress_noalloc
    f.argtypes = [VP, VP, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, VP, VP, ctypes.c_int,
                  ctypes.c_int64, ctypes.c_uint64, VP, VP, VP, VP]
    cap = lib.gc_noalloc_scratch_bytes()
    assert cap == 32 << 20
    n = 1 << 28
    st, need = _ws(lib, 1, n, n // 100, 127)
    assert st == 0 and need > cap
    assert f(FAKE, FAKE, n, n // 100, 0, FAKE, None, 127, 64, 1, FAKE, FAKE, None, None) == 2   # GC_EWORKSPACE
    assert b"fixed scratch" in lib.gc_last_error()
    # bad arguments are reported as by gc_ef_compress, before the size check
    assert f(None, FAKE, 10, 1, 0, FAKE, FAKE, 0, 64, 0, None, None, None, None) == 1
    assert f(FAKE, FAKE, 10, 11, 0, FAKE, FAKE, 0, 64, 0, None, None, None, None) == 1
    assert b"k must" in lib.gc_last_error()
    assert f(FAKE, FAKE, n, n // 100, 0, FAKE, None, 127, 100, 1, FAKE, FAKE, None, None) == 1   # group
    # n == 0 and k == 0 need no workspace and touch nothing
    assert f(None, None, 0, 0, 0, None, None, 0, 64, 0, None, None, None, None) == 0


def test_prepared_calls_check_their_buffers(lib):
    # the prepared calls of the DDP hook check every buffer when they are set up, on the
    # host: host tensors, wrong dtypes and missing outputs raise before any library call
    import torch
    import gradient_compression_ddp_amd as gcm
    n, k = 10_000, 100
    cpu_res = torch.zeros(n)
    idx = torch.zeros(k, dtype=torch.int64)
    with pytest.raises(ValueError, match="GPU tensor"):
        gcm.PreparedEfCompress(n, cpu_res, k, out_idx=idx, out_val=torch.zeros(k))
    with pytest.raises(ValueError, match="GPU tensor"):
        gcm.PreparedDecompress([torch.zeros(256, dtype=torch.uint8)], [gcm.PayloadHeader()])
    with pytest.raises(ValueError, match="one header per payload"):
        gcm.PreparedDecompress([], [gcm.PayloadHeader()])
