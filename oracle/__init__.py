"""CPU oracle for the gradient-compression hot path -- TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously correct numpy implementation of what the HIP path computes.
Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the HIP library and imports
nothing from it; the product path never falls back to it.

Numeric contract (the HIP kernels follow the same one):

* every floating-point operation is a single IEEE binary32 operation with
  round-to-nearest-even: numpy float32 arrays, explicit ``np.float32`` scalars, no
  fused multiply-add, no flush-to-zero;
* division and square root are the correctly rounded ones (numpy float32 ``/`` and
  ``np.sqrt``);
* deterministic rounding is ``np.rint`` (round half to even), which is what the
  pages' ``np.round`` / ``torch.round`` do;
* group sums use an explicit balanced pairwise tree in natural index order, never
  ``np.sum`` (whose blocking order is unspecified);
* PowerSGD runs in float64 after the float32 error-feedback add.

Functions whose parity has no independent pin say "parity unpinned" in their own
docstring; at present every function has at least one pin in ``tests/``.
"""
from .philox import philox4x32_10, uniform24
from .topk import magnitude_key, ef_topk, topk_invariant_holds
from .minmax import quant_minmax, dequant_minmax, pack_int4, unpack_int4
from .qsgd import qsgd, dequant_qsgd, pairwise_sum_of_squares
from .terngrad import terngrad, dequant_terngrad, pack_ternary, unpack_ternary
from .powersgd import powersgd_step, modified_gram_schmidt
from .decompress import decompress_scatter, KIND_F32, KIND_MINMAX8, KIND_MINMAX4, KIND_QSGD, KIND_TERN
from .pipeline import ef_topk_qsgd
from .randk import randk_keys, ef_randk, ef_randk_qsgd
from .monitor import norm_stats, monitored_step

__all__ = [
    "philox4x32_10", "uniform24", "magnitude_key", "ef_topk", "topk_invariant_holds",
    "quant_minmax", "dequant_minmax", "pack_int4", "unpack_int4", "qsgd", "dequant_qsgd",
    "pairwise_sum_of_squares", "terngrad", "dequant_terngrad", "pack_ternary",
    "unpack_ternary", "powersgd_step", "modified_gram_schmidt", "decompress_scatter",
    "KIND_F32", "KIND_MINMAX8", "KIND_MINMAX4", "KIND_QSGD", "KIND_TERN", "ef_topk_qsgd",
    "randk_keys", "ef_randk", "ef_randk_qsgd", "norm_stats", "monitored_step",
]
