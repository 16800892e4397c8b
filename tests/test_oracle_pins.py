"""The CPU oracle against its pins (exact arithmetic, closed forms, invariants, numpy's
binary16 codec, IEEE 754 golden values). No GPU."""
import pytest

import oracle
from oracle_pins import ALL_PINS


@pytest.fixture(scope="module")
def orc():
    oracle.build()
    return oracle.Oracle(oracle.LIBRARY)


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_tolerance_checker_known_vectors():
    import numpy as np
    ref = np.array([[1.0, -2.0, 0.0, 100.0]])
    K = 100  # abs term 1e-2
    ok = np.array([[1.0, -2.0, 0.0, 100.0]], np.float16).view(np.uint16)
    rep = oracle.compare(ok, ref, K)
    assert rep["fails"] == 0
    # 100 +- (0.4 + 0.01) is the edge; 100.5 is representable in fp16 (spacing 0.0625)
    bad = np.array([[1.0, -2.0, 0.0, 100.5]], np.float16).view(np.uint16)
    rep = oracle.compare(bad, ref, K)
    assert rep["fails"] == 1 and rep["first_fail"] == (0, 3)
    nan = np.array([[np.nan, -2.0, 0.0, 100.0]], np.float16).view(np.uint16)
    assert oracle.compare(nan, ref, K)["fails"] == 1
    near = np.array([[1.0, -2.0, 0.0098, 100.0]], np.float16).view(np.uint16)
    assert oracle.compare(near, ref, K)["fails"] == 0
