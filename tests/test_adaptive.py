"""Host logic of the adaptive compression hooks (no GPU)."""
import pytest

from gradient_compression_ddp_amd.adaptive import DEFAULT_LADDER, AdaptiveController, Setting


def test_alarm_after_patience_moves_weaker_and_fires_hooks():
    c = AdaptiveController(start=2, alarm=0.9, patience=3)
    alarms, changes = [], []
    c.on_alarm.append(lambda step, r: alarms.append((step, r)))
    c.on_change.append(lambda old, new: changes.append((old, new)))
    assert c.observe(0.5) == DEFAULT_LADDER[2]
    assert c.observe(0.95) == DEFAULT_LADDER[2]       # a good step resets the streak
    c.observe(0.5)
    c.observe(0.5)
    assert c.observe(0.5) == DEFAULT_LADDER[1]       # third low ratio in a row
    assert alarms == [(5, 0.5)]
    assert changes == [(DEFAULT_LADDER[2], DEFAULT_LADDER[1])]


def test_network_signal_moves_with_hold_and_bounds():
    c = AdaptiveController(start=1, patience=2, congested=0.5, idle=0.1)
    assert c.observe(comm_fraction=0.7) == DEFAULT_LADDER[2]   # congested: stronger
    assert c.observe(comm_fraction=0.7) == DEFAULT_LADDER[2]   # held
    assert c.observe(comm_fraction=0.7) == DEFAULT_LADDER[2]   # held
    assert c.observe(comm_fraction=0.7) == DEFAULT_LADDER[3]
    for _ in range(10):
        c.observe(comm_fraction=0.9)
    assert c.setting == DEFAULT_LADDER[-1]                     # clamped at the strongest
    for _ in range(20):
        c.observe(comm_fraction=0.01)
    assert c.setting == DEFAULT_LADDER[0]                      # idle: back to the weakest
    assert c.observe(comm_fraction=0.3) == DEFAULT_LADDER[0]   # in between: stay


def test_alarm_has_priority_over_congestion():
    c = AdaptiveController(start=2, patience=1, congested=0.5)
    assert c.observe(ratio=0.2, comm_fraction=0.9) == DEFAULT_LADDER[1]


def test_warmup_uses_the_weakest_setting():
    c = AdaptiveController(start=3, warmup_steps=2)
    assert c.setting == DEFAULT_LADDER[0]
    assert c.observe(ratio=0.1, comm_fraction=0.9) == DEFAULT_LADDER[0]
    assert c.observe(ratio=0.1, comm_fraction=0.9) == DEFAULT_LADDER[3]   # warm-up over: the start rung
    assert c.steps == 2


def test_k_for_and_validation():
    assert Setting(0.01, 127).k_for(7_000_000_000) == 70_000_000
    assert Setting(0.001, 7).k_for(10) == 1
    with pytest.raises(ValueError):
        AdaptiveController(ladder=())
    with pytest.raises(ValueError):
        AdaptiveController(start=9)
    with pytest.raises(ValueError):
        AdaptiveController(idle=0.6, congested=0.5)
