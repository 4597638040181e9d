"""The GPU tests' bf16 output check (tests/gpu_util.check_bf16_output), run
on hand-made values on the CPU: it accepts what bf16 storage of the exact
value allows and refuses one ulp more."""

import numpy as np
import pytest

from tests.gpu_util import bf16_ulp, check_bf16_output

PAD = np.zeros(100)  # exact elements, so that a few errors keep the mean low


def padded(x):
    return np.concatenate([np.asarray(x, dtype=np.float64), PAD])


def test_small_values_hold_the_absolute_bar():
    ref = padded([0.5, -1.25, 3.9])
    check_bf16_output(ref + padded([9e-3, -9e-3, 0.0]), ref, "within 1e-2")
    with pytest.raises(AssertionError):
        check_bf16_output(ref + padded([1.1e-2, 0.0, 0.0]), ref, "above 1e-2")


def test_mean_bar():
    ref = np.zeros(10)
    with pytest.raises(AssertionError):
        check_bf16_output(ref + 2e-3, ref, "mean above 1e-3")


def test_large_values_must_be_faithfully_rounded():
    # |O| >= 4: bf16 spacing is 1/32 on [4, 8), so 1e-2 cannot be asked for
    ref = padded([4.2933, 5.0 + 1.0 / 64])  # the second one is a tie
    lo = padded([4.28125, 5.0])             # the bf16 number below each
    hi = padded([4.3125, 5.03125])          # and above
    assert np.all(bf16_ulp(ref[:2]) == 1.0 / 32)
    check_bf16_output(lo, ref, "round down")
    check_bf16_output(hi, ref, "round up")
    with pytest.raises(AssertionError):
        check_bf16_output(padded([4.25, 5.0]), ref, "two ulps below")


def test_non_finite_output_fails():
    with pytest.raises(AssertionError):
        check_bf16_output(np.array([np.nan]), np.array([0.0]), "nan")
