"""The matrix-unit rate probe (emulated_fp32_matrix_amd/ceiling): its entry
point refuses bad arguments before any HIP call (host), and on the device
a short run gives a rate and a clock in the range the hardware allows."""
import ctypes

import pytest

from emulated_fp32_matrix_amd import ceiling


@pytest.mark.parametrize("which,seconds", [(2, 1.0), (-1, 1.0), (0, 0.0), (1, -1.0), (0, 31.0)])
def test_bad_arguments_are_refused_before_any_hip_call(which, seconds):
    lib = ceiling._lib()
    d = ctypes.c_double()
    assert lib.emu_ceiling_run(which, seconds, ctypes.byref(d), ctypes.byref(d), ctypes.byref(d)) != 0
    assert lib.emu_ceiling_run(0, 1.0, None, ctypes.byref(d), ctypes.byref(d)) != 0


@pytest.mark.gpu
@pytest.mark.parametrize("kind", ["bf16", "f32"])
def test_short_run_is_in_range(kind):
    r = ceiling.run(kind, 0.3)
    spec = ceiling.SPEC[kind]
    assert 0.3 * spec < r["tflops"] <= 1.02 * spec, r
    assert 0.5 < r["sclk_ghz"] <= 2.5, r
    # the rate follows the clock: at least 80 % of the peak at the measured clock
    assert 0.8 < r["frac_of_peak_at_that_clock"] <= 1.01, r
