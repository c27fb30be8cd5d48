"""Host logic of the sequence driver (no GPU): which scheme each step uses."""
import pytest

from activation_residual_compression_amd.session import MODES, Schedule


def test_schedule_full_steps_then_phases():
    s = Schedule([(3, "lr"), (1, "q2"), (10, "q1")], full_steps=1)
    assert [s.at(t) for t in range(12)] == (["full", "q2", "q2", "lr", "lr", "lr", "lr", "lr", "lr",
                                              "lr", "q1", "q1"])
    s = Schedule([(0, "q1")], full_steps=3)
    assert [s.at(t) for t in range(5)] == ["full", "full", "full", "q1", "q1"]


def test_schedule_rejects_gaps_and_empty_warmup():
    with pytest.raises(ValueError):
        Schedule([(2, "q1")], full_steps=1)      # step 1 has no scheme
    with pytest.raises(ValueError):
        Schedule([(0, "q1")], full_steps=0)      # step 0 is always sent in full
    with pytest.raises(ValueError):
        Schedule([], full_steps=1)
    assert MODES == ("closed", "noef", "direct")
