"""DDP communication hook: error-feedback Top-K (or Random-K) + QSGD on every gradient bucket.

Sources: hotdry.top "gradient-compression-quantization-sparsification", section 3.2
(compress inside the framework's communication step, before the gradient leaves GPU
memory, overlapped with the backward pass); aiqz.cc "梯度聚合通信优化实战方案", section
"通信计算重叠" (gradient buckets: each bucket is sent as soon as the backward pass has
filled it) and "通信瓶颈分析" (the aggregate is the average over workers);
zyxy.net/archives/25733, section 四 (compress, exchange, decompress before the update).

Per bucket and step:
  1. gc_ef_compress: c = bucket + residual, exact Top-k (or Random-k) of c, QSGD of the
     kept values, written straight into this rank's payload (the 128-byte header and the
     idx / codes / norms sections of the wire format), the kept set's residual deferred
     to the bucket's next step by default;
  2. all_gather of the fixed-size payloads (every rank's k and layout are equal);
  3. gc_decompress_payloads: the bucket becomes the average of the W decoded payloads.
Every step is enqueued on one stream and nothing waits on the host: the stream waits
for the all_gather's work before the decode, and the hook returns a future that is
already complete, since whatever DDP runs next on that stream comes after the decode.
With `overlap` (the default) the three steps run on a side stream of the hook's own
(default priority), which first waits for an event recorded on DDP's stream (the bucket's
gradients are complete), so the backward pass of the earlier layers keeps running while
the bucket is compressed and exchanged; the returned future is device-aware and set on
the side stream, so DDP's stream waits for the decode only when DDP waits for the future.
Without it, every step runs on DDP's stream, which then also waits for the collective.

The iteration of a small model is bound by the host: each bucket's library calls are set
up once (PreparedEfCompress, PreparedDecompress: arguments checked and converted when the
bucket is created), so a step costs two ctypes calls, the collective and an event.

State per bucket (keyed by DDP's bucket index and size; DDP may regroup buckets after its
first iteration, and a bucket whose size changes starts from a zero residual): residual,
pending record, workspace, this rank's payload and the gathered payloads, and the
prepared calls over them.
"""
# No postponed annotations here: DDP checks the hook's annotations at run time.
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import torch
import torch.distributed as dist

from . import (KIND_F32, KIND_QSGD, OP_EF_RANDK, OP_EF_TOPK, PreparedDecompress, PreparedEfCompress, ef_flush,
               payload_layout, payload_sections, pending_record, workspace_size, write_payload_header)


def _align256(b: int) -> int:
    return (b + 255) & ~255


@dataclass
class _Bucket:
    n: int
    k: int
    header: object
    residual: torch.Tensor
    pending: Optional[torch.Tensor]
    workspace: torch.Tensor
    payload: torch.Tensor
    gathered: torch.Tensor
    stride: int
    stats: Optional[torch.Tensor]
    compress: PreparedEfCompress      # the bucket's library calls, set up once
    decode: PreparedDecompress
    ready: torch.cuda.Event           # side stream: the bucket's gradients are complete
    calls: int = 0


@dataclass
class CompressionHookState:
    """Options and per-bucket state of :func:`ef_compress_hook`."""
    process_group: Optional[dist.ProcessGroup] = None
    ratio: float = 0.01               # kept fraction k / n of every bucket
    qsgd_levels: int = 127            # 8-bit codes (sign + 7-bit level); 0 sends fp32 values
    qsgd_group: int = 64
    select: str = "topk"              # or "randk"
    deferred: bool = True             # kept-set residual applied by the bucket's next step
    monitor: bool = False             # keep the norm-ratio stats of every bucket
    seed: int = 0
    overlap: bool = True              # compress and exchange on a side stream
    buckets: Dict[int, _Bucket] = field(default_factory=dict)
    side_stream: Optional[torch.cuda.Stream] = None
    # tests: when a list, (bucket index, step, bucket before, bucket after) is appended
    capture: Optional[List[Tuple[int, int, torch.Tensor, torch.Tensor]]] = None

    def seeds(self, index: int, step: int) -> Tuple[int, int]:
        """(selection seed, QSGD seed) of a bucket's step; equal on every rank."""
        base = (self.seed * 1_000_003 + index) * 1_000_033 + step
        return base * 2 + 1, base * 2

    def k_for(self, n: int) -> int:
        return max(1, min(n, int(n * self.ratio)))

    def bucket(self, index: int, n: int, device) -> _Bucket:
        b = self.buckets.get(index)
        if b is not None and b.n == n:
            return b
        W = dist.get_world_size(self.process_group)
        k = self.k_for(n)
        if self.qsgd_levels > 0:
            h = payload_layout(KIND_QSGD, n, k, self.qsgd_group, self.qsgd_levels, sparse=True)
        else:
            h = payload_layout(KIND_F32, n, k, sparse=True)
        stride = _align256(h.bytes)
        payload = torch.zeros(stride, dtype=torch.uint8, device=device)
        write_payload_header(payload, h)
        op = OP_EF_RANDK if self.select == "randk" else OP_EF_TOPK
        ws = torch.empty(max(workspace_size(op, n, k, self.qsgd_levels), 1), dtype=torch.uint8, device=device)
        residual = torch.zeros(n, dtype=torch.float32, device=device)
        pending = pending_record(n, k, device) if self.deferred else None
        stats = torch.zeros(3, dtype=torch.float64, device=device) if self.monitor else None
        gathered = torch.empty(W * stride, dtype=torch.uint8, device=device)
        sec = payload_sections(payload, h)
        if self.qsgd_levels > 0:
            outs = dict(out_codes=sec["codes"], out_norms=sec["meta0"])
        else:
            outs = dict(out_val=sec["codes"])
        compress = PreparedEfCompress(n, residual, k, select=self.select, pending=pending, stats=stats,
                                      qsgd_levels=self.qsgd_levels, qsgd_group=self.qsgd_group, out_idx=sec["idx"],
                                      workspace=ws, **outs)
        decode = PreparedDecompress([gathered[w * stride:(w + 1) * stride] for w in range(W)], [h] * W)
        b = _Bucket(n=n, k=k, header=h, residual=residual, pending=pending, workspace=ws, payload=payload,
                    gathered=gathered, stride=stride, stats=stats, compress=compress, decode=decode,
                    ready=torch.cuda.Event())
        self.buckets[index] = b
        return b

    def flush(self) -> None:
        """Apply every bucket's pending record, so each residual is exact (e.g. before a
        checkpoint of the residuals), on the current stream, after the side stream's work."""
        if self.side_stream is not None:
            torch.cuda.current_stream().wait_stream(self.side_stream)
        for b in self.buckets.values():
            if b.pending is not None:
                ef_flush(b.residual, b.pending)


def _raw_stream(device_index: int) -> int:
    """The current stream's raw handle, without building a Stream object."""
    return torch._C._cuda_getCurrentRawStream(device_index)


def ef_compress_hook(state: CompressionHookState, bucket: dist.GradBucket) -> torch.futures.Future[torch.Tensor]:
    buf = bucket.buffer()
    if buf.dtype != torch.float32:
        raise TypeError("the compression hook handles float32 gradient buckets")
    index = bucket.index()
    b = state.bucket(index, buf.numel(), buf.device)
    step = b.calls
    b.calls += 1
    sel_seed, q_seed = state.seeds(index, step)
    if state.overlap:
        cur = torch.cuda.current_stream()
        if state.side_stream is None:
            state.side_stream = torch.cuda.Stream(device=buf.device)
        stream = state.side_stream
        b.ready.record(cur)              # the bucket's gradients are complete
        stream.wait_event(b.ready)
        with torch.cuda.stream(stream):  # the collective orders itself after the current stream
            _exchange(state, b, buf, index, step, sel_seed, q_seed, stream.cuda_stream)
            # a device-aware future set here records the side stream: DDP's stream waits
            # for the decode only when DDP waits for the future, at the end of backward,
            # so the backward of earlier layers is not held behind this bucket's exchange
            fut = torch.futures.Future(devices=[buf.device])
            fut.set_result(buf)
        return fut
    _exchange(state, b, buf, index, step, sel_seed, q_seed, _raw_stream(buf.device.index))
    # everything is ordered on DDP's stream, so the result is ready for what DDP runs next
    fut = torch.futures.Future()
    fut.set_result(buf)
    return fut


def _exchange(state, b, buf, index, step, sel_seed, q_seed, h):
    """Compress, all_gather and decode one bucket on the current stream (raw handle h)."""
    before = buf.clone() if state.capture is not None else None
    b.compress(buf, sel_seed, q_seed, h)
    work = dist.all_gather_into_tensor(b.gathered, b.payload, group=state.process_group, async_op=True)
    work.wait()                          # the stream waits for the gathered payloads; the host does not
    b.decode(buf, h)
    if state.capture is not None:
        state.capture.append((index, step, before, buf.clone()))
