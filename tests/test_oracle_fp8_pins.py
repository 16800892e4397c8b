"""The fp8 part of the CPU oracle against its pins (torch's CPU E4M3 codec, ties-to-even
midpoints, numpy float32 division, exact rational sums, the binary16 oracle, closed forms
and invariants). No GPU."""
import numpy as np
import pytest

import oracle
from oracle_fp8_pins import FP8_PINS


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.Oracle(oracle.LIBRARY)


@pytest.mark.parametrize("pin", FP8_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_fp8_tolerance_checker_known_vectors():
    ref = np.array([[1.0, -2.0, 0.0, 100.0]])
    bound = np.array([[0.0, 0.0, 256.0, 0.0]])         # abs term 2^-8 * 256 = 1 at (0, 2)
    ok = np.array([[1.0, -2.0, 0.99, 100.0]], np.float16).view(np.uint16)
    assert oracle.compare_fp8(ok, ref, bound)["fails"] == 0
    bad = np.array([[1.0, -2.0, 1.02, 100.5]], np.float16).view(np.uint16)
    rep = oracle.compare_fp8(bad, ref, bound)
    assert rep["fails"] == 2 and rep["first_fail"] == (0, 2)
    nan = np.array([[np.nan, -2.0, 0.0, 100.0]], np.float16).view(np.uint16)
    assert oracle.compare_fp8(nan, ref, bound)["fails"] == 1
