"""Adaptive compression hooks driven by the gradient-norm-ratio monitor.

Sources: hotdry.top "gradient-compression-quantization-sparsification", section 3.2,
item 2 (watch the ratio of the gradient norm after compression to the norm before it;
a ratio that stays below 0.9 signals compression that is too strong) and item 3 (compress
harder when the network is congested, back off when it is idle); zyxy.net/archives/25733,
section 三 (use a small compression ratio early in training and a larger one later).

The pages give the signals, not a control law.  This module's reading:

* The settings form a ladder from the weakest compression (rung 0) to the strongest.
  A setting is the kept fraction k/n and the QSGD levels of the kept values (0: values
  sent as fp32).
* During the first ``warmup_steps`` observations the weakest rung is used.
* Norm alarm: ``patience`` consecutive ratios below ``alarm`` move one rung weaker and
  fire the ``on_alarm`` hooks.  The alarm has priority over the network signal.
* Network signal: the caller passes the share of the step spent in communication.
  Above ``congested`` the controller moves one rung stronger, below ``idle`` one rung
  weaker.  After any move it holds for ``patience`` observations, so one slow step
  does not make it oscillate.
* Every change fires the ``on_change`` hooks with (old, new) settings.

NormRatioMonitor moves the device-side stats of gc_ef_compress (sum c^2, sum g_hat^2,
ratio) to pinned host memory on the compression stream and hands them over once that
copy has completed, so reading the ratio of step t never stalls step t + 1.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, List, Optional, Sequence, Tuple

import torch


@dataclass(frozen=True)
class Setting:
    ratio: float        # kept fraction k / n
    qsgd_levels: int    # QSGD levels of the kept values (0: fp32 values)

    def k_for(self, n: int) -> int:
        return max(1, min(n, int(n * self.ratio)))


# Weakest to strongest: Top-10% int8, Top-1% int8, Top-1% with 7 levels (4 bits with the
# sign), Top-0.1% with 7 levels.
DEFAULT_LADDER: Tuple[Setting, ...] = (Setting(0.10, 127), Setting(0.01, 127), Setting(0.01, 7),
                                       Setting(0.001, 7))


class AdaptiveController:
    def __init__(self, ladder: Sequence[Setting] = DEFAULT_LADDER, start: int = 1, alarm: float = 0.9,
                 patience: int = 3, congested: float = 0.5, idle: float = 0.1, warmup_steps: int = 0):
        if not ladder:
            raise ValueError("the ladder needs at least one setting")
        if not 0 <= start < len(ladder):
            raise ValueError("start must index the ladder")
        if patience < 1:
            raise ValueError("patience must be >= 1")
        if not idle < congested:
            raise ValueError("idle must be below congested")
        self.ladder = tuple(ladder)
        self.rung = start
        self.alarm = alarm
        self.patience = patience
        self.congested = congested
        self.idle = idle
        self.warmup_steps = warmup_steps
        self.steps = 0
        self.low_streak = 0
        self.hold = 0
        self.on_alarm: List[Callable[[int, float], None]] = []
        self.on_change: List[Callable[[Setting, Setting], None]] = []

    @property
    def setting(self) -> Setting:
        if self.steps < self.warmup_steps:
            return self.ladder[0]
        return self.ladder[self.rung]

    def _move(self, delta: int) -> None:
        new = min(max(self.rung + delta, 0), len(self.ladder) - 1)
        if new != self.rung:
            old = self.ladder[self.rung]
            self.rung = new
            for hook in self.on_change:
                hook(old, self.ladder[new])
        self.hold = self.patience

    def observe(self, ratio: Optional[float] = None, comm_fraction: Optional[float] = None) -> Setting:
        """Feed one step's signals (either may be None) and get the setting for the next."""
        self.steps += 1
        if self.steps <= self.warmup_steps:
            return self.setting
        if ratio is not None:
            self.low_streak = self.low_streak + 1 if ratio < self.alarm else 0
            if self.low_streak >= self.patience:
                for hook in self.on_alarm:
                    hook(self.steps, ratio)
                self.low_streak = 0
                self._move(-1)
                return self.setting
        if self.hold > 0:
            self.hold -= 1
            return self.setting
        if comm_fraction is not None:
            if comm_fraction > self.congested:
                self._move(+1)
            elif comm_fraction < self.idle:
                self._move(-1)
        return self.setting


class NormRatioMonitor:
    """Host view of the norm-monitor stats, one step behind, without synchronizing."""

    def __init__(self):
        self.host = torch.zeros(3, dtype=torch.float64, pin_memory=True)
        self.event: Optional[torch.cuda.Event] = None
        self.last: Optional[Tuple[float, float, float]] = None

    def record(self, stats: torch.Tensor, stream: Optional[torch.cuda.Stream] = None) -> None:
        """Queue the copy of a device float64[3] stats tensor on `stream` (default: current)."""
        stream = stream or torch.cuda.current_stream()
        with torch.cuda.stream(stream):
            self.host.copy_(stats[:3], non_blocking=True)
            self.event = torch.cuda.Event()
            self.event.record(stream)

    def poll(self) -> Optional[Tuple[float, float, float]]:
        """The newest stats whose copy has completed (None before the first one)."""
        if self.event is not None and self.event.query():
            self.last = tuple(float(x) for x in self.host.tolist())
            self.event = None
        return self.last
