"""bench.py's live clock reading on the device: on the 192-atom stack it
returns a fully busy interval's per-XCD clocks, a mean between idle and the
spec clock, and the socket power (skipped where amdsmi is not importable)."""
import os
import sys

import pytest

from gpu_helpers import say

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_clock_reading_under_load():
    pytest.importorskip("amdsmi")
    import torch

    import bench
    import emulated_fp32_matrix_amd as emu
    import synth

    dev = torch.device("cuda:0")
    gemms = synth.gemms(2)
    tensors = bench.make_inputs(torch, dev, gemms)
    clock = bench.clock_under_load(torch, emu, gemms, tensors, "BF16X9")
    say(f"clock reading: {clock}")
    assert clock is not None, "no fully busy interval within the time limit"
    assert len(clock["xcd_ghz"]) >= 1
    assert 0.5 < clock["sclk_ghz"] <= 2.6
    assert all(0.1 < x <= 2.6 for x in clock["xcd_ghz"])
    assert abs(clock["sclk_ghz"] - sum(clock["xcd_ghz"]) / len(clock["xcd_ghz"])) < 0.002
    assert clock["gfx_activity_pct"] >= 95
    assert clock["after_s"] <= 4.5
