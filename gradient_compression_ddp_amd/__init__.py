"""Python binding of libgc.so, the MI355X (gfx950) gradient-compression library.

Marshalling only: each function checks tensor dtypes/devices, allocates the outputs
and the workspace with torch when the caller does not pass them, and forwards raw
device pointers and the current HIP stream to the C ABI declared in include/gc.h.
Every step of the computation runs in the library's HIP kernels; there is no CPU
fallback.  Importing this package fails loudly if libgc.so has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "lib_path", "GCError", "workspace_size", "ef_compress", "ef_compress_noalloc", "noalloc_scratch_bytes",
    "EfOptions", "ef_topk", "ef_topk_deferred",
    "ef_flush", "pending_record",
    "ef_randk", "quant_minmax", "qsgd", "terngrad",
    "powersgd_step", "decompress_scatter", "KIND_F32", "KIND_MINMAX8", "KIND_MINMAX4",
    "KIND_QSGD", "KIND_TERN", "OP_EF_TOPK", "OP_QUANT_MINMAX", "OP_QSGD", "OP_TERNGRAD",
    "OP_POWERSGD", "OP_DECOMPRESS", "OP_EF_RANDK", "OP_EF_PENDING", "profile_enable", "profile_collect", "PayloadHeader",
    "PAYLOAD_MAGIC", "PAYLOAD_SPARSE", "payload_layout", "payload_sections", "write_payload_header",
    "read_payload_header", "decompress_payloads", "stream_floor", "PreparedEfCompress", "PreparedDecompress",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libgc.so")

GC_OK, GC_EINVAL, GC_EWORKSPACE, GC_EUNSUPPORTED, GC_EHIP = 0, 1, 2, 3, 4
OP_EF_TOPK, OP_QUANT_MINMAX, OP_QSGD, OP_TERNGRAD, OP_POWERSGD, OP_DECOMPRESS = 1, 2, 3, 4, 5, 6
OP_EF_RANDK, OP_EF_PENDING = 7, 8
KIND_F32, KIND_MINMAX8, KIND_MINMAX4, KIND_QSGD, KIND_TERN = 0, 1, 2, 3, 4

if not os.path.exists(lib_path):
    raise ImportError(
        f"{lib_path} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
        "or `python gradient_compression_ddp_amd/build.py` (needs hipcc for gfx950)")

_lib = ctypes.CDLL(lib_path)

PAYLOAD_MAGIC, PAYLOAD_VERSION, PAYLOAD_SPARSE = 0x31504347, 1, 1


class PayloadHeader(ctypes.Structure):
    """The 128-byte wire header of one payload (include/gc.h, gc_payload_header)."""
    _fields_ = [("magic", ctypes.c_uint32), ("version", ctypes.c_uint16), ("kind", ctypes.c_uint16),
                ("flags", ctypes.c_uint32), ("levels", ctypes.c_int32), ("n", ctypes.c_int64),
                ("count", ctypes.c_int64), ("index_base", ctypes.c_int64), ("group", ctypes.c_int64),
                ("off_idx", ctypes.c_uint64), ("off_codes", ctypes.c_uint64), ("off_meta0", ctypes.c_uint64),
                ("off_meta1", ctypes.c_uint64), ("bytes", ctypes.c_uint64), ("reserved", ctypes.c_uint8 * 40)]


assert ctypes.sizeof(PayloadHeader) == 128

SELECT_TOPK, SELECT_RANDK = 0, 1


class EfOptions(ctypes.Structure):
    """gc_ef_options (include/gc.h): selector, pending record, norm-monitor output."""
    _fields_ = [("size", ctypes.c_uint32), ("select", ctypes.c_uint32), ("select_seed", ctypes.c_uint64),
                ("pending", ctypes.c_void_p), ("pending_bytes", ctypes.c_size_t), ("stats", ctypes.c_void_p)]

_p, _i64, _u64, _i32, _f32, _sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint64, ctypes.c_int,
                                   ctypes.c_float, ctypes.c_size_t)
_SIGS = {
    "gc_status_string": ([_i32], ctypes.c_char_p),
    "gc_last_error": ([], ctypes.c_char_p),
    "gc_version": ([], _i32),
    "gc_workspace_size": ([_i32, _i64, _i64, _i64, ctypes.POINTER(_sz)], _i32),
    "gc_ef_topk": ([_p, _p, _i64, _i64, _i64, _p, _p, _i32, _i64, _u64, _p, _p, _p, _sz, _p], _i32),
    "gc_ef_compress": ([_p, _p, _i64, _i64, _i64, _p, _p, _i32, _i64, _u64, _p, _p, ctypes.POINTER(EfOptions),
                        _p, _sz, _p], _i32),
    "gc_ef_compress_noalloc": ([_p, _p, _i64, _i64, _i64, _p, _p, _i32, _i64, _u64, _p, _p,
                                ctypes.POINTER(EfOptions), _p], _i32),
    "gc_noalloc_scratch_bytes": ([], _sz),
    "gc_ef_topk_deferred": ([_p, _p, _i64, _i64, _i64, _p, _p, _i32, _i64, _u64, _p, _p, _p, _sz, _p, _sz, _p],
                            _i32),
    "gc_ef_flush": ([_p, _i64, _p, _sz, _p], _i32),
    "gc_ef_randk": ([_p, _p, _i64, _i64, _i64, _u64, _p, _p, _i32, _i64, _u64, _p, _p, _p, _sz, _p], _i32),
    "gc_quant_minmax": ([_p, _p, _i64, _i64, _i32, _p, _p, _p, _p, _sz, _p], _i32),
    "gc_qsgd": ([_p, _p, _i64, _i64, _i32, _u64, _i64, _p, _p, _p], _i32),
    "gc_stream_floor": ([_p, _p, _i64, _p], _i32),
    "gc_terngrad": ([_p, _p, _i32, _p, _u64, _i64, _p, _p, _p, _sz, _p], _i32),
    "gc_powersgd_step": ([_p, _p, _i64, _i64, _i32, _p, _p, _p, _sz, _p], _i32),
    "gc_decompress_scatter": ([_i32, _p, _i64, _i64, _p, _p, _p, _i64, _i32, _f32, _i32, _p, _i64, _p],
                              _i32),
    "gc_payload_layout": ([_i32, _i64, _i64, _i64, _i32, _i32, _i64, ctypes.POINTER(PayloadHeader)], _i32),
    "gc_decompress_payloads": ([_i32, ctypes.POINTER(_p), ctypes.POINTER(PayloadHeader), _f32, _i32, _p, _i64,
                                _p], _i32),
    "gc_profile_enable": ([_i32], _i32),
    "gc_profile_collect": ([ctypes.POINTER(_i64), ctypes.POINTER(ctypes.c_double),
                            ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)], _i32),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res


class GCError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = _lib.gc_last_error().decode(errors="replace")
        kind = _lib.gc_status_string(status).decode()
        super().__init__(f"{where}: {kind}: {msg}")
        self.status = status


def _check(status: int, where: str):
    if status != GC_OK:
        raise GCError(status, where)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t: torch.Tensor, dtype, name: str):
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def workspace_size(op: int, n: int, k: int = 0, aux: int = 0) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib.gc_workspace_size(op, n, k, aux, ctypes.byref(out)), "gc_workspace_size")
    return int(out.value)


def _workspace(op, n, k, aux, device, workspace):
    need = workspace_size(op, n, k, aux)
    if need == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    return workspace, workspace.numel()


def _sparsify(name, op, grad, residual, k, index_base, extra, qsgd_levels, qsgd_group, qsgd_seed,
              out_idx, out_val, out_codes, out_norms, want_values, workspace, stream, tail=()):
    _dev(grad, torch.float32, "grad")
    _dev(residual, torch.float32, "residual")
    n = grad.numel()
    if residual.numel() != n:
        raise ValueError("grad and residual differ in size")
    dev = grad.device
    if out_idx is None:
        out_idx = torch.empty(k, dtype=torch.int64, device=dev)
    quant = qsgd_levels > 0
    if out_val is None and (want_values or not quant):
        out_val = torch.empty(k, dtype=torch.float32, device=dev)
    if quant:
        if out_codes is None:
            out_codes = torch.empty(k, dtype=torch.int8, device=dev)
        if out_norms is None:
            out_norms = torch.empty((k + qsgd_group - 1) // qsgd_group, dtype=torch.float32, device=dev)
    if op is None:       # the entry point brings its own workspace
        ws_args = ()
    else:
        ws, ws_bytes = _workspace(op, n, k, qsgd_levels, dev, workspace)
        ws_args = (_ptr(ws), ws_bytes)
    _check(getattr(_lib, name)(_ptr(grad), _ptr(residual), n, k, index_base, *extra, _ptr(out_idx),
                               _ptr(out_val), qsgd_levels, qsgd_group, qsgd_seed, _ptr(out_codes),
                               _ptr(out_norms), *tail, *ws_args, _stream(stream)), name)
    if quant:
        return out_idx, out_codes, out_norms, out_val
    return out_idx, out_val


def ef_topk(grad, residual, k, index_base=0, *, qsgd_levels=0, qsgd_group=64, qsgd_seed=0,
            out_idx=None, out_val=None, out_codes=None, out_norms=None, want_values=True,
            workspace=None, stream=None):
    """Error-feedback Top-K; with qsgd_levels > 0 also QSGD on the kept values.

    Updates ``residual`` in place.  Returns ``(idx, val)`` for pure Top-K, or
    ``(idx, codes, norms, val)`` with QSGD (``val`` is None when ``want_values`` is False).
    """
    return _sparsify("gc_ef_topk", OP_EF_TOPK, grad, residual, k, index_base, (), qsgd_levels, qsgd_group,
                     qsgd_seed, out_idx, out_val, out_codes, out_norms, want_values, workspace, stream)


def ef_compress(grad, residual, k, index_base=0, *, select="topk", select_seed=0, pending=None, stats=None,
                qsgd_levels=0, qsgd_group=64, qsgd_seed=0, out_idx=None, out_val=None, out_codes=None,
                out_norms=None, want_values=True, workspace=None, stream=None):
    """One EF sparsification step with every option (gc_ef_compress).

    select: "topk" or "randk" (keys under ``select_seed``); pending: a record from
    :func:`pending_record` to defer the kept set's residual (apply with the next call or
    :func:`ef_flush`); stats: a float64 GPU tensor of 3 that receives the norm monitor
    (sum c^2, sum g_hat^2, ratio).  Outputs as :func:`ef_topk`.
    """
    opts = _ef_options(select, select_seed, pending, stats)
    op = OP_EF_RANDK if select == "randk" else OP_EF_TOPK
    return _sparsify("gc_ef_compress", op, grad, residual, k, index_base, (), qsgd_levels, qsgd_group, qsgd_seed,
                     out_idx, out_val, out_codes, out_norms, want_values, workspace, stream,
                     tail=(ctypes.byref(opts),))


def _ef_options(select, select_seed, pending, stats):
    if select not in ("topk", "randk"):
        raise ValueError("select must be 'topk' or 'randk'")
    opts = EfOptions(size=ctypes.sizeof(EfOptions), select=SELECT_RANDK if select == "randk" else SELECT_TOPK,
                     select_seed=select_seed)
    if pending is not None:
        _dev(pending, torch.uint8, "pending")
        opts.pending, opts.pending_bytes = pending.data_ptr(), pending.numel()
    if stats is not None:
        _dev(stats, torch.float64, "stats")
        if stats.numel() < 3:
            raise ValueError("stats must hold 3 doubles")
        opts.stats = stats.data_ptr()
    return opts


class PreparedEfCompress:
    """One gc_ef_compress call set up for repeated use on the same buffers (one DDP bucket
    every step): every argument but the gradient, the two seeds and the stream is checked
    and converted once, so a call costs the ctypes call and little else.  Same operation
    and outputs as :func:`ef_compress` with ``index_base = 0``."""

    def __init__(self, n, residual, k, *, select="topk", pending=None, stats=None, qsgd_levels=0, qsgd_group=64,
                 out_idx, out_val=None, out_codes=None, out_norms=None, workspace=None):
        _dev(residual, torch.float32, "residual")
        if residual.numel() != n:
            raise ValueError("residual differs in size from n")
        _dev(out_idx, torch.int64, "out_idx")
        quant = qsgd_levels > 0
        if quant:
            if out_codes is None or out_norms is None:
                raise ValueError("QSGD needs out_codes and out_norms")
        elif out_val is None:
            raise ValueError("pure selection needs out_val")
        self.n = n
        self._dev = residual.device
        self._opts = _ef_options(select, 0, pending, stats)
        op = OP_EF_RANDK if select == "randk" else OP_EF_TOPK
        ws, ws_bytes = _workspace(op, n, k, qsgd_levels, residual.device, workspace)
        self._keep = (residual, pending, stats, out_idx, out_val, out_codes, out_norms, ws)   # alive while prepared
        p = lambda t: None if t is None else t.data_ptr()
        self._head = (p(residual), n, k, 0, p(out_idx), p(out_val), qsgd_levels, qsgd_group)
        self._tail = (p(out_codes), p(out_norms), ctypes.byref(self._opts), p(ws), ws_bytes)
        self._fn = _lib.gc_ef_compress

    def __call__(self, grad, select_seed, qsgd_seed, stream_handle):
        """grad: float32 GPU tensor of n elements; stream_handle: the raw hipStream_t."""
        if grad.numel() != self.n or grad.dtype != torch.float32 or grad.device != self._dev:
            raise ValueError("grad must be a float32 tensor of n elements on the residual's device")
        self._opts.select_seed = select_seed
        _check(self._fn(grad.data_ptr(), *self._head, qsgd_seed, *self._tail, stream_handle), "gc_ef_compress")


class PreparedDecompress:
    """One gc_decompress_payloads call over fixed payload buffers, set up once: a call
    passes only the output and the stream.  Same operation as :func:`decompress_payloads`."""

    def __init__(self, payloads, headers, *, alpha=None, accumulate=False):
        W = len(payloads)
        if W != len(headers):
            raise ValueError("one header per payload")
        for b in payloads:
            _dev(b, torch.uint8, "payload")
        self._keep = list(payloads)
        self._ptrs = (ctypes.c_void_p * W)(*[b.data_ptr() for b in payloads])
        self._hdrs = (PayloadHeader * W)(*headers)
        self._W = W
        self._alpha = 1.0 / W if alpha is None else alpha
        self._acc = 1 if accumulate else 0
        self._pp = ctypes.cast(self._ptrs, ctypes.POINTER(ctypes.c_void_p))
        self._fn = _lib.gc_decompress_payloads

    def __call__(self, out, stream_handle):
        if out.dtype != torch.float32 or not out.is_contiguous():
            raise ValueError("out must be a contiguous float32 tensor")
        _check(self._fn(self._W, self._pp, self._hdrs, self._alpha, self._acc, out.data_ptr(), out.numel(),
                        stream_handle), "gc_decompress_payloads")


def noalloc_scratch_bytes() -> int:
    """Bytes of the fixed per-GPU array that :func:`ef_compress_noalloc` works in."""
    return int(_lib.gc_noalloc_scratch_bytes())


def ef_compress_noalloc(grad, residual, k, index_base=0, *, select="topk", select_seed=0, pending=None,
                        stats=None, qsgd_levels=0, qsgd_group=64, qsgd_seed=0, out_idx=None, out_val=None,
                        out_codes=None, out_norms=None, want_values=True, stream=None):
    """:func:`ef_compress` without a workspace (gc_ef_compress_noalloc): the library
    works in its own fixed per-GPU array and allocates nothing.  Pass every output
    tensor to keep this wrapper from allocating them; calls beyond the array's size
    raise GCError (GC_EWORKSPACE)."""
    opts = _ef_options(select, select_seed, pending, stats)
    return _sparsify("gc_ef_compress_noalloc", None, grad, residual, k, index_base, (), qsgd_levels, qsgd_group,
                     qsgd_seed, out_idx, out_val, out_codes, out_norms, want_values, None, stream,
                     tail=(ctypes.byref(opts),))


def pending_record(n, k_max, device):
    """A zero-filled (empty) pending record for :func:`ef_topk_deferred` on n elements."""
    return torch.zeros(max(workspace_size(OP_EF_PENDING, n, k_max), 1), dtype=torch.uint8, device=device)


def ef_topk_deferred(grad, residual, k, pending, index_base=0, *, qsgd_levels=0, qsgd_group=64, qsgd_seed=0,
                     out_idx=None, out_val=None, out_codes=None, out_norms=None, want_values=True,
                     workspace=None, stream=None):
    """:func:`ef_topk` whose kept-set residual update is recorded in ``pending`` (a
    uint8 tensor from :func:`pending_record`) and applied by the next call or by
    :func:`ef_flush`.  Outputs as :func:`ef_topk`."""
    _dev(pending, torch.uint8, "pending")
    return _sparsify("gc_ef_topk_deferred", OP_EF_TOPK, grad, residual, k, index_base, (), qsgd_levels,
                     qsgd_group, qsgd_seed, out_idx, out_val, out_codes, out_norms, want_values, workspace,
                     stream, tail=(_ptr(pending), pending.numel()))


def ef_flush(residual, pending, stream=None):
    """Apply ``pending`` to ``residual`` (which then equals what :func:`ef_topk` would
    have left) and empty the record."""
    _dev(residual, torch.float32, "residual")
    _dev(pending, torch.uint8, "pending")
    _check(_lib.gc_ef_flush(_ptr(residual), residual.numel(), _ptr(pending), pending.numel(), _stream(stream)),
           "gc_ef_flush")


def ef_randk(grad, residual, k, select_seed, index_base=0, *, qsgd_levels=0, qsgd_group=64, qsgd_seed=0,
             out_idx=None, out_val=None, out_codes=None, out_norms=None, want_values=True,
             workspace=None, stream=None):
    """Error-feedback Random-K (the k indices with the largest Philox keys under
    ``select_seed``); with qsgd_levels > 0 also QSGD on the kept values.  Outputs as
    :func:`ef_topk`."""
    return _sparsify("gc_ef_randk", OP_EF_RANDK, grad, residual, k, index_base, (select_seed,), qsgd_levels,
                     qsgd_group, qsgd_seed, out_idx, out_val, out_codes, out_norms, want_values, workspace,
                     stream)


def quant_minmax(x, group, bits, residual=None, *, codes=None, mins=None, scales=None,
                 workspace=None, stream=None):
    """Min-max quantization; returns (codes uint8, mins, scales).  int4 codes are packed."""
    _dev(x, torch.float32, "x")
    if residual is not None:
        _dev(residual, torch.float32, "residual")
    n = x.numel()
    g = n if group == 0 else group
    ng = 0 if n == 0 else (n + g - 1) // g
    dev = x.device
    if codes is None:
        codes = torch.empty(n if bits == 8 else (n + 1) // 2, dtype=torch.uint8, device=dev)
    if mins is None:
        mins = torch.empty(ng, dtype=torch.float32, device=dev)
    if scales is None:
        scales = torch.empty(ng, dtype=torch.float32, device=dev)
    ws, ws_bytes = _workspace(OP_QUANT_MINMAX, n, group, 0, dev, workspace)
    _check(_lib.gc_quant_minmax(_ptr(x), _ptr(residual), n, group, bits, _ptr(codes), _ptr(mins),
                                _ptr(scales), _ptr(ws), ws_bytes, _stream(stream)), "gc_quant_minmax")
    return codes, mins, scales


def qsgd(x, group, levels, seed, index_base=0, residual=None, *, codes=None, norms=None, stream=None):
    """QSGD; returns (codes int8, norms)."""
    _dev(x, torch.float32, "x")
    if residual is not None:
        _dev(residual, torch.float32, "residual")
    n = x.numel()
    dev = x.device
    if codes is None:
        codes = torch.empty(n, dtype=torch.int8, device=dev)
    if norms is None:
        norms = torch.empty((n + group - 1) // group, dtype=torch.float32, device=dev)
    _check(_lib.gc_qsgd(_ptr(x), _ptr(residual), n, group, levels, seed, index_base, _ptr(codes),
                        _ptr(norms), _stream(stream)), "gc_qsgd")
    return codes, norms


def stream_floor(x, out=None, *, stream=None):
    """Benchmark calibration: out[i] = (x[i] > 0) as uint8, nothing else (the bytes a
    one-pass 8-bit quantizer moves).  Returns out."""
    _dev(x, torch.float32, "x")
    if out is None:
        out = torch.empty(x.numel(), dtype=torch.uint8, device=x.device)
    _check(_lib.gc_stream_floor(_ptr(x), _ptr(out), x.numel(), _stream(stream)), "gc_stream_floor")
    return out


def terngrad(x, seg_offsets, seed, index_base=0, residual=None, *, packed=None, scales=None,
             workspace=None, stream=None):
    """TernGrad over segments; seg_offsets is a host sequence of nseg+1 int64 offsets.
    Returns (packed uint8, scales)."""
    import numpy as np
    _dev(x, torch.float32, "x")
    if residual is not None:
        _dev(residual, torch.float32, "residual")
    off = np.ascontiguousarray(np.asarray(seg_offsets, dtype=np.int64))
    nseg = off.size - 1
    lens = np.diff(off)
    nbytes = int(((lens + 3) // 4).sum()) if nseg > 0 else 0
    dev = x.device
    if packed is None:
        packed = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty(max(nseg, 0), dtype=torch.float32, device=dev)
    ws, ws_bytes = _workspace(OP_TERNGRAD, int(off[-1]) if nseg > 0 else 0, nseg, 0, dev, workspace)
    _check(_lib.gc_terngrad(_ptr(x), _ptr(residual), nseg, off.ctypes.data_as(ctypes.c_void_p), seed,
                            index_base, _ptr(packed), _ptr(scales), _ptr(ws), ws_bytes,
                            _stream(stream)), "gc_terngrad")
    return packed, scales


def powersgd_step(grad, residual, Q, *, P=None, workspace=None, stream=None):
    """One PowerSGD step on a rows x cols matrix; Q (cols x rank) is updated in place.
    Returns P (rows x rank)."""
    _dev(grad, torch.float32, "grad")
    if residual is not None:
        _dev(residual, torch.float32, "residual")
    _dev(Q, torch.float32, "Q")
    rows, cols = grad.shape
    rank = Q.shape[1]
    if P is None:
        P = torch.empty((rows, rank), dtype=torch.float32, device=grad.device)
    ws, ws_bytes = _workspace(OP_POWERSGD, rows, cols, rank, grad.device, workspace)
    _check(_lib.gc_powersgd_step(_ptr(grad), _ptr(residual), rows, cols, rank, _ptr(Q), _ptr(P), _ptr(ws),
                                 ws_bytes, _stream(stream)), "gc_powersgd_step")
    return P


def decompress_scatter(kind, codes, count, out, *, idx=None, index_base=0, meta0=None, meta1=None,
                       group=0, levels=0, alpha=1.0, accumulate=False, stream=None):
    """Decode `count` payload entries into `out` (dense, or scattered through idx)."""
    _dev(out, torch.float32, "out")
    _check(_lib.gc_decompress_scatter(kind, _ptr(idx), count, index_base, _ptr(codes), _ptr(meta0),
                                      _ptr(meta1), group, levels, alpha, 1 if accumulate else 0, _ptr(out),
                                      out.numel(), _stream(stream)), "gc_decompress_scatter")
    return out


def profile_enable(on: bool = True) -> None:
    """Record HIP events around the stages of every ef_topk call (see gc.h)."""
    _check(_lib.gc_profile_enable(1 if on else 0), "gc_profile_enable")


def profile_collect():
    """Wait for the recorded events; returns (calls, ms_before_pass, ms_pass, ms_after_pass)."""
    calls = ctypes.c_int64(0)
    a, b, c = ctypes.c_double(0), ctypes.c_double(0), ctypes.c_double(0)
    _check(_lib.gc_profile_collect(ctypes.byref(calls), ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)),
           "gc_profile_collect")
    return int(calls.value), a.value, b.value, c.value


# ---------------------------------------------------------------------------
# Wire format and the receive side
# ---------------------------------------------------------------------------

_CODE_DTYPE = {KIND_F32: torch.float32, KIND_MINMAX8: torch.uint8, KIND_MINMAX4: torch.uint8,
               KIND_QSGD: torch.int8, KIND_TERN: torch.uint8}


def payload_layout(kind, n, count, group=0, levels=0, sparse=False, index_base=0) -> PayloadHeader:
    """Header (section offsets and total size) of a payload of this shape."""
    h = PayloadHeader()
    _check(_lib.gc_payload_layout(kind, n, count, group, levels, 1 if sparse else 0, index_base,
                                  ctypes.byref(h)), "gc_payload_layout")
    return h


def _code_len(kind, count):
    return {KIND_F32: count, KIND_MINMAX8: count, KIND_MINMAX4: (count + 1) // 2,
            KIND_QSGD: count, KIND_TERN: (count + 3) // 4}[kind]


def payload_sections(buf, h: PayloadHeader) -> dict:
    """Typed views of the sections of payload `buf` (uint8 device tensor of h.bytes bytes)."""
    _dev(buf, torch.uint8, "payload")
    if buf.numel() < h.bytes:
        raise ValueError("payload buffer is smaller than the header says")
    g = h.group if h.group > 0 else max(h.count, 1)
    ng = 0 if h.count == 0 else (h.count + g - 1) // g
    out = {}
    if h.off_idx:
        out["idx"] = buf[h.off_idx:h.off_idx + 8 * h.count].view(torch.int64)
    dt = _CODE_DTYPE[h.kind]
    nbytes = _code_len(h.kind, h.count) * (4 if h.kind == KIND_F32 else 1)
    out["codes"] = buf[h.off_codes:h.off_codes + nbytes].view(dt)
    if h.off_meta0:
        out["meta0"] = buf[h.off_meta0:h.off_meta0 + 4 * ng].view(torch.float32)
    if h.off_meta1:
        out["meta1"] = buf[h.off_meta1:h.off_meta1 + 4 * ng].view(torch.float32)
    return out


def write_payload_header(buf, h: PayloadHeader) -> None:
    """Store the header in the first 128 bytes of the payload (a host-to-device copy)."""
    _dev(buf, torch.uint8, "payload")
    raw = torch.frombuffer(bytearray(bytes(h)), dtype=torch.uint8)
    buf[:128].copy_(raw)


def read_payload_header(buf) -> PayloadHeader:
    """Copy the first 128 bytes of a payload back to the host as a header."""
    return PayloadHeader.from_buffer_copy(bytes(buf[:128].cpu().numpy().tobytes()))


def decompress_payloads(payloads, headers, out, *, alpha=None, accumulate=False, stream=None):
    """out = (out if accumulate else 0) + sum_w alpha * decode(payload w), in payload order.

    payloads: list of uint8 device tensors (each 256-byte aligned); headers: their
    PayloadHeader objects.  alpha defaults to 1/W (the average)."""
    _dev(out, torch.float32, "out")
    W = len(payloads)
    if W != len(headers):
        raise ValueError("one header per payload")
    for b in payloads:
        _dev(b, torch.uint8, "payload")
    ptrs = (ctypes.c_void_p * W)(*[b.data_ptr() for b in payloads])
    hdrs = (PayloadHeader * W)(*headers)
    a = 1.0 / W if alpha is None else alpha
    _check(_lib.gc_decompress_payloads(W, ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p)), hdrs, a,
                                       1 if accumulate else 0, _ptr(out), out.numel(), _stream(stream)),
           "gc_decompress_payloads")
    return out
