"""GPU smoke test of the calibration's timing path (the calibration itself is
a measurement, run by `python -m decode_attention_prefix_amd.calibrate`)."""
import math

import pytest

from test_gpu_parity import _torch

pytestmark = pytest.mark.gpu


def test_step_timer_times_both_schedules():
    _torch()
    from decode_attention_prefix_amd import calibrate as cal
    tm = cal.StepTimer(steps=3, warmup=1)
    t = cal.family_tree(64, 2, subtrees=4)
    for mode in (0, 1):
        us = tm.time_tree(t, share_mode=mode)
        assert math.isfinite(us) and us > 0
    assert tm.read_rate() > 1e11
