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


def test_fp8_tolerance_catches_typical_mistakes():
    """The fp8 tolerance is not vacuous: results with one k-block's scale doubled, with B's
    k order shuffled inside a block, or with the last k-block dropped fail it."""
    import tgemm_workloads as W
    M, N, K = 64, 256, 1040
    A, SA, B, SB = W.make_fp8_inputs(M, N, K, seed=5)
    ref = oracle.gemm_fp8(A, SA, B, SB, relu=False)
    E = oracle.fp8_bound(A, SA, B, SB)
    ok = oracle.f16_encode(ref)
    assert oracle.compare_fp8(ok, ref, E)["fails"] == 0
    SA2 = SA.copy()
    SA2[:, 3] *= 2
    B2 = B.copy()
    rng = np.random.default_rng(6)
    B2[:, 256:384] = B2[:, 256 + rng.permutation(128)]
    SA3 = SA.copy()
    SA3[:, -1] = 0
    for what, args in [("scale doubled", (A, SA2, B, SB)), ("k shuffled in B", (A, SA, B2, SB)),
                       ("last block dropped", (A, SA3, B, SB))]:
        bad = oracle.f16_encode(oracle.gemm_fp8(*args, relu=False))
        rep = oracle.compare_fp8(bad, ref, E)
        assert rep["fails"] > M * N // 4, (what, rep)
