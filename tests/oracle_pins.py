"""Pins for the CPU oracle: checks against facts that do not come from the oracle.

Each pin takes an ``oracle.Oracle`` instance and raises AssertionError when the
instance disagrees with something the mathematics or an independent implementation
fixes. The same list runs against the real oracle (test_oracle_pins.py) and against
deliberately broken copies of its source (test_oracle_mutants.py), which must each
fail at least one pin.

Independent facts used:
  * exact rational arithmetic (Python ``fractions``) on tiny shapes;
  * numpy's binary16 codec (an independent implementation of IEEE 754 binary16);
  * IEEE 754 values and ties-to-even roundings written in tests/golden/;
  * closed forms: ones @ ones = K, A @ I = A, I @ B = B;
  * sign symmetry of round-to-nearest: ReLU(A @ (-B)) = max(-(A @ B), +0) bit for bit.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
U = Fraction(1, 2 ** 53)  # unit roundoff of float64


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def _finite_f16_bits(rng, shape, frac_special=0.1):
    """Arbitrary finite binary16 bit patterns, with extra weight on subnormals and +-65504."""
    bits = rng.integers(0, 1 << 16, size=shape, dtype=np.uint32).astype(np.uint16)
    bad = ((bits >> 10) & 31) == 31
    while bad.any():
        bits[bad] = rng.integers(0, 1 << 16, size=int(bad.sum()), dtype=np.uint32).astype(np.uint16)
        bad = ((bits >> 10) & 31) == 31
    special = rng.random(shape) < frac_special
    choices = np.array([0x0001, 0x03FF, 0x8001, 0x7BFF, 0xFBFF, 0x0000, 0x8000, 0x0400], np.uint16)
    bits[special] = rng.choice(choices, size=int(special.sum()))
    return bits


def _exact(bits):
    """binary16 bits -> exact Fractions, via numpy's codec (float16 -> float is exact)."""
    vals = bits.view(np.float16).astype(np.float64)
    return [[Fraction(float(v)) for v in row] for row in vals]


# --------------------------------------------------------------------------------------
# codec pins
# --------------------------------------------------------------------------------------
def pin_decode_all_patterns(orc):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.f16_decode(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "NaN patterns decode differently from numpy"
    assert np.array_equal(got[~nan].view(np.uint64), ref[~nan].view(np.uint64)), \
        "decode differs from numpy's binary16 codec"


def pin_decode_golden(orc):
    for hx, val in _read_golden("binary16_points.txt"):
        h = int(hx, 16)
        got = float(orc.f16_decode(np.array([h], np.uint16))[0])
        if val == "nan":
            assert got != got, hx
        elif val in ("inf", "-inf"):
            assert got == float(val), hx
        elif val == "-0":
            assert got == 0.0 and np.signbit(got), hx
        else:
            assert Fraction(got) == Fraction(val), (hx, got, val)
            if val == "0":
                assert not np.signbit(got), hx


def pin_encode_roundtrip(orc):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    keep = ~np.isnan(vals)
    back = orc.f16_encode(vals[keep])
    assert np.array_equal(back, bits[keep]), "encode(decode(h)) != h"


def pin_encode_vs_numpy(orc):
    rng = np.random.default_rng(11)
    # random magnitudes over the whole binary16 range, plus exact midpoints (ties)
    x = rng.standard_normal(200000) * np.exp2(rng.uniform(-26, 17, 200000))
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = bits.view(np.float16).astype(np.float64)
    v = v[np.isfinite(v)]
    v = np.sort(v)
    mids = (v[1:] + v[:-1]) / 2.0  # exact in float64
    x = np.concatenate([x, mids, -mids, [65519.99, 65520.0, 1e6, -1e6, 0.0, -0.0]])
    got = orc.f16_encode(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref), "encode differs from numpy's round-to-nearest-even"


def pin_encode_golden(orc):
    for val, hx in _read_golden("rne_points.txt"):
        x = float(Fraction(val))
        got = int(orc.f16_encode(np.array([x]))[0])
        assert got == int(hx, 16), (val, hex(got), hx)


# --------------------------------------------------------------------------------------
# contraction pins
# --------------------------------------------------------------------------------------
def pin_bruteforce_exact(orc):
    """Tiny shapes, arbitrary finite inputs: the oracle is within the float64 summation
    bound gamma_{K-1} * sum|a b| of the exact rational sum."""
    rng = np.random.default_rng(5)
    for trial in range(40):
        M, N = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        K = int(rng.integers(1, 41))
        A = _finite_f16_bits(rng, (M, K))
        B = _finite_f16_bits(rng, (K, N))
        relu = bool(trial % 2)
        got = orc.gemm(A, B, relu=relu)
        Ae, Be = _exact(A), _exact(B)
        n = K - 1
        gamma = (n * U) / (1 - n * U)
        for i in range(M):
            for j in range(N):
                terms = [Ae[i][k] * Be[k][j] for k in range(K)]
                s = sum(terms, Fraction(0))
                bound = gamma * sum(abs(t) for t in terms)
                ref = s if (not relu or s > 0) else Fraction(0)
                err = abs(Fraction(float(got[i, j])) - ref)
                # ReLU can only shrink the error: |relu(x) - relu(s)| <= |x - s|
                assert err <= bound, (trial, i, j, float(err), float(bound))


def pin_bruteforce_exact_integers(orc):
    """Small-integer inputs keep every partial sum exact: the oracle equals the exact sum."""
    rng = np.random.default_rng(6)
    for trial in range(40):
        M, N = int(rng.integers(1, 8)), int(rng.integers(1, 8))
        K = int(rng.integers(1, 65))
        A = rng.integers(-16, 17, size=(M, K)).astype(np.float16)
        B = rng.integers(-16, 17, size=(K, N)).astype(np.float16)
        relu = bool(trial % 2)
        got = orc.gemm(A, B, relu=relu)
        ref = A.astype(np.int64) @ B.astype(np.int64)
        if relu:
            ref = np.maximum(ref, 0)
        assert np.array_equal(got, ref.astype(np.float64)), trial


def pin_ones(orc):
    for (M, N, K) in [(3, 5, 1), (4, 3, 1000), (2, 7, 2051), (5, 2, 4095), (1, 1, 4096)]:
        A = np.ones((M, K), np.float16)
        B = np.ones((K, N), np.float16)
        for relu in (False, True):
            got = orc.gemm(A, B, relu=relu)
            assert np.all(got == K), (M, N, K, relu)
        got = orc.gemm(A, -B, relu=False)
        assert np.all(got == -K), (M, N, K)


def pin_identity(orc):
    rng = np.random.default_rng(7)
    M, K, N = 13, 29, 17
    A = _finite_f16_bits(rng, (M, K))
    B = _finite_f16_bits(rng, (K, N))
    IK = np.eye(K, dtype=np.float16)
    IM = np.eye(M, dtype=np.float16)
    a = A.view(np.float16).astype(np.float64)
    b = B.view(np.float16).astype(np.float64)
    assert np.array_equal(orc.gemm(A, IK, relu=False), a)
    assert np.array_equal(orc.gemm(IK, B, relu=False), b)
    assert np.array_equal(orc.gemm(A, IK, relu=True), np.where(a > 0, a, 0.0))
    # a permutation matrix selects columns: A @ P = A[:, perm]
    perm = rng.permutation(K)
    P = np.zeros((K, K), np.float16)
    P[perm, np.arange(K)] = 1
    assert np.array_equal(orc.gemm(A, P, relu=False), a[:, perm])
    assert np.array_equal(orc.gemm(IM, A, relu=False), a)


def pin_relu_sign_invariants(orc):
    rng = np.random.default_rng(8)
    A = rng.standard_normal((37, 53)).astype(np.float16)
    B = rng.standard_normal((53, 41)).astype(np.float16)
    Bn = (B.view(np.uint16) ^ np.uint16(0x8000)).view(np.float16)
    plain = orc.gemm(A, B, relu=False)
    r_pos = orc.gemm(A, B, relu=True)
    r_neg = orc.gemm(A, Bn, relu=True)
    assert not np.any(np.signbit(r_pos)) and np.all(r_pos >= 0)
    assert not np.any(np.signbit(r_neg)) and np.all(r_neg >= 0)
    flipped = np.where(-plain > 0, -plain, 0.0)
    assert np.array_equal(r_neg.view(np.uint64), flipped.view(np.uint64))
    assert np.array_equal(r_pos - r_neg, plain)
    assert np.any(plain < 0) and np.any(plain > 0)


def pin_transpose(orc):
    rng = np.random.default_rng(9)
    A = rng.standard_normal((23, 71)).astype(np.float16)
    B = rng.standard_normal((71, 19)).astype(np.float16)
    c = orc.gemm(A, B, relu=False)
    ct = orc.gemm(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T), relu=False)
    assert np.array_equal(c.T.view(np.uint64), ct.view(np.uint64))


def pin_threads(orc):
    rng = np.random.default_rng(10)
    A = rng.standard_normal((64, 300)).astype(np.float16)
    B = rng.standard_normal((300, 48)).astype(np.float16)
    c1 = orc.gemm(A, B, relu=True, nthreads=1)
    c4 = orc.gemm(A, B, relu=True, nthreads=4)
    assert np.array_equal(c1.view(np.uint64), c4.view(np.uint64))


def pin_entries_match_full(orc):
    rng = np.random.default_rng(12)
    A = rng.standard_normal((40, 90)).astype(np.float16)
    B = rng.standard_normal((90, 30)).astype(np.float16)
    for relu in (False, True):
        full = orc.gemm(A, B, relu=relu)
        rows = rng.integers(0, 40, 200)
        cols = rng.integers(0, 30, 200)
        ent = orc.gemm_entries(A, B, rows, cols, relu=relu)
        assert np.array_equal(ent.view(np.uint64), full[rows, cols].view(np.uint64))


def pin_entries_exact(orc):
    """The one-by-one path against exact integer sums (independent of the full path)."""
    rng = np.random.default_rng(13)
    A = rng.integers(-16, 17, size=(9, 50)).astype(np.float16)
    B = rng.integers(-16, 17, size=(50, 11)).astype(np.float16)
    ref = A.astype(np.int64) @ B.astype(np.int64)
    rows, cols = np.meshgrid(np.arange(9), np.arange(11), indexing="ij")
    for relu in (False, True):
        ent = orc.gemm_entries(A, B, rows.ravel(), cols.ravel(), relu=relu)
        r = np.maximum(ref, 0) if relu else ref
        assert np.array_equal(ent.reshape(9, 11), r.astype(np.float64)), relu


def pin_strided(orc):
    """Leading dimensions larger than the row length give the same result."""
    rng = np.random.default_rng(14)
    Abig = rng.standard_normal((21, 64)).astype(np.float16)
    Bbig = rng.standard_normal((40, 33)).astype(np.float16)
    A, B = Abig[:, :40], Bbig[:, :25]
    c = orc.gemm(A, B, relu=True)
    c2 = orc.gemm(np.ascontiguousarray(A), np.ascontiguousarray(B), relu=True)
    assert np.array_equal(c.view(np.uint64), c2.view(np.uint64))
    ref = A.astype(np.float64) @ B.astype(np.float64)
    assert np.allclose(c, np.maximum(ref, 0), rtol=1e-12, atol=1e-12)
    rows = rng.integers(0, 21, 50)
    cols = rng.integers(0, 25, 50)
    e = orc.gemm_entries(A, B, rows, cols, relu=True)
    assert np.array_equal(e.view(np.uint64), c[rows, cols].view(np.uint64))


def pin_degenerate(orc):
    A = np.zeros((4, 0), np.float16)
    B = np.zeros((0, 6), np.float16)
    for relu in (False, True):
        c = orc.gemm(A, B, relu=relu)
        assert c.shape == (4, 6) and np.all(c == 0) and not np.any(np.signbit(c))
    assert orc.gemm(np.zeros((0, 3), np.float16), np.zeros((3, 5), np.float16), relu=True).shape == (0, 5)
    assert orc.gemm(np.zeros((2, 3), np.float16), np.zeros((3, 0), np.float16), relu=True).shape == (2, 0)


def pin_float64_product(orc):
    """Against numpy's float64 matmul (BLAS order differs: equal within the float64
    summation bound, which is ~1e-13 relative here)."""
    rng = np.random.default_rng(15)
    A = rng.standard_normal((70, 130)).astype(np.float16)
    B = rng.standard_normal((130, 50)).astype(np.float16)
    ref = A.astype(np.float64) @ B.astype(np.float64)
    absref = np.abs(A.astype(np.float64)) @ np.abs(B.astype(np.float64))
    got = orc.gemm(A, B, relu=False)
    assert np.all(np.abs(got - ref) <= 2 * 130 * 2.0 ** -53 * absref)


ALL_PINS = [
    pin_decode_all_patterns, pin_decode_golden, pin_encode_roundtrip, pin_encode_vs_numpy,
    pin_encode_golden, pin_bruteforce_exact, pin_bruteforce_exact_integers, pin_ones,
    pin_identity, pin_relu_sign_invariants, pin_transpose, pin_threads,
    pin_entries_match_full, pin_entries_exact, pin_strided, pin_degenerate,
    pin_float64_product,
]
