"""Pins for the fp8 part of the CPU oracle (E4M3 codec, block quantizer, block-scaled GEMM).

Each pin takes an ``oracle.Oracle`` instance and raises AssertionError when the instance
disagrees with something that does not come from the oracle:
  * code points and roundings taken from the OCP 8-bit floating point specification's
    definition of E4M3 (tests/golden/e4m3_points.txt);
  * torch's CPU float8_e4m3fn codec (an independent implementation of OCP E4M3) over all
    256 codes and on random float32 values below the saturation point;
  * ties-to-even at every midpoint between neighbouring E4M3 values (a property of the
    rounding, checked on values built from torch's decoded codes);
  * numpy's IEEE float32 division for the block scales and the scaled values;
  * exact rational arithmetic (Python ``fractions``) for the block-scaled sum;
  * the binary16 oracle (pinned on its own) when every scale is 1: E4M3 values are exact
    binary16 values, so the two definitions coincide up to float64 rounding;
  * closed forms (all-ones codes with block-varying scales), scale linearity, the block
    structure (a zero scale removes exactly its k-block), ReLU and thread invariance.
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

BLOCK = 128
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def pin_e4m3_golden(orc):
    """Decode and encode the code points and roundings of tests/golden/e4m3_points.txt."""
    n = 0
    with open(os.path.join(GOLDEN, "e4m3_points.txt")) as f:
        for line in f:
            row = line.split("#", 1)[0].split()
            if not row:
                continue
            kind, a, b = row
            if kind == "decode":
                got = float(orc.e4m3_decode(np.array([int(a, 16)], np.uint8))[0])
                if b == "nan":
                    assert got != got, (a, got)
                else:
                    assert Fraction(got) == Fraction(b), (a, got, b)
                    assert np.signbit(got) == b.startswith("-"), (a, got, b)
            else:
                got = int(orc.e4m3_encode(np.array([float(Fraction(a))]))[0])
                assert got == int(b, 16), (a, hex(got), b)
            n += 1
    assert n >= 30, n


def _torch():
    import torch
    return torch


def _torch_decode(codes: np.ndarray) -> np.ndarray:
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_encode(x32: np.ndarray) -> np.ndarray:
    torch = _torch()
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _finite_codes(rng, shape, frac_special=0.1):
    """Arbitrary finite E4M3 codes, with extra weight on subnormals, zeros and +-448."""
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    nan = (c & 0x7F) == 0x7F
    c[nan] = rng.integers(0, 0x7F, size=int(nan.sum())).astype(np.uint8)
    special = rng.random(shape) < frac_special
    choices = np.array([0x01, 0x07, 0x81, 0x7E, 0xFE, 0x00, 0x80, 0x08], np.uint8)
    c[special] = rng.choice(choices, size=int(special.sum()))
    return c


def _scales(rng, shape):
    """float32 scales of mixed sizes: powers of two and values with full significands."""
    s = (2.0 ** rng.integers(-12, 4, size=shape)) * rng.uniform(0.5, 1.0, size=shape)
    s = s.astype(np.float32)
    s[rng.random(shape) < 0.2] = np.float32(1.0)
    return s


# --------------------------------------------------------------------------------------
# codec pins
# --------------------------------------------------------------------------------------
def pin_e4m3_decode_all_codes(orc):
    codes = np.arange(256, dtype=np.uint8)
    got = orc.e4m3_decode(codes)
    ref = _torch_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref)), "NaN codes differ from torch"
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok]), "decoded values differ from torch"
    assert np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok])), "signed zeros differ"


def pin_e4m3_encode_roundtrip(orc):
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    back = orc.e4m3_encode(_torch_decode(codes))
    assert np.array_equal(back, codes), "encode(decode(c)) != c"


def pin_e4m3_encode_ties_even(orc):
    v = _torch_decode(np.arange(0x7F, dtype=np.uint8))   # +0 .. 448, increasing
    assert np.all(np.diff(v) > 0)
    lo, hi = v[:-1], v[1:]
    mid = (lo + hi) / 2                                   # exact in float64
    want = np.where(np.arange(0x7E) % 2 == 0, np.arange(0x7E), np.arange(1, 0x7F)).astype(np.uint8)
    assert np.array_equal(orc.e4m3_encode(mid), want), "ties not to the even code"
    assert np.array_equal(orc.e4m3_encode(-mid), want | 0x80), "negative ties"
    eps = (hi - lo) * 2.0 ** -20
    assert np.array_equal(orc.e4m3_encode(mid - eps), np.arange(0x7E, dtype=np.uint8)), "below midpoint"
    assert np.array_equal(orc.e4m3_encode(mid + eps), np.arange(1, 0x7F, dtype=np.uint8)), "above midpoint"


def pin_e4m3_encode_vs_torch(orc):
    rng = np.random.default_rng(81)
    x = np.concatenate([rng.uniform(-464, 464, 20000), rng.normal(0, 1, 20000),
                        rng.uniform(-2.0 ** -5, 2.0 ** -5, 20000)]).astype(np.float32)
    assert np.array_equal(orc.e4m3_encode(x.astype(np.float64)), _torch_encode(x)), "differs from torch"


def pin_e4m3_saturation(orc):
    big = np.array([448.0, 448.5, 463.99, 464.0, 479.9, 480.0, 1e6, np.inf])
    assert np.all(orc.e4m3_encode(big) == 0x7E) and np.all(orc.e4m3_encode(-big) == 0xFE)
    assert orc.e4m3_encode(np.array([np.nan]))[0] & 0x7F == 0x7F


# --------------------------------------------------------------------------------------
# quantizer pins
# --------------------------------------------------------------------------------------
def _f16_blocks(rng, R, K):
    x = rng.normal(0.0, 1.0, size=(R, K)) * (2.0 ** rng.integers(-6, 6, size=(R, 1)))
    x = x.astype(np.float16)
    x[rng.random((R, K)) < 0.02] = 0
    return x


def _blocks(R, K, br):
    for r0 in range(0, R, br):
        for k0 in range(0, K, BLOCK):
            yield r0 // br, k0 // BLOCK, slice(r0, min(R, r0 + br)), slice(k0, min(K, k0 + BLOCK))


def pin_quant_scales_numpy(orc):
    rng = np.random.default_rng(82)
    for R, K, br in [(5, 300, 1), (300, 260, 128), (129, 128, 128), (3, 1, 1), (7, 129, 1)]:
        x = _f16_blocks(rng, R, K)
        x[:, :min(K, BLOCK)][0] = 0                       # a zero block in row 0 (br = 1)
        Q, S = orc.quant_fp8(x, br)
        assert S.shape == (-(-R // br), -(-K // BLOCK)) and Q.shape == (R, K)
        for rb, kb, rs, ks in _blocks(R, K, br):
            amax = np.float32(np.abs(x[rs, ks].astype(np.float32)).max())
            s = np.float32(1.0) if amax == 0 else np.float32(amax) / np.float32(448.0)
            assert S[rb, kb] == s, (R, K, br, rb, kb)
            y = x[rs, ks].astype(np.float32) / s              # float32 division, IEEE
            assert np.array_equal(Q[rs, ks], _torch_encode(y)), (R, K, br, rb, kb)


def pin_quant_dequant_error(orc):
    rng = np.random.default_rng(83)
    x = _f16_blocks(rng, 64, 384)
    Q, S = orc.quant_fp8(x, 1)
    deq = _torch_decode(Q) * np.repeat(S.astype(np.float64), BLOCK, axis=1)[:, :384]
    # half a spacing of E4M3 at |x|/s (relative 2^-4 for normals, 2^-10 absolute below 2^-6)
    y = np.abs(x.astype(np.float64)) / np.repeat(S.astype(np.float64), BLOCK, axis=1)[:, :384]
    half = np.where(y >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(y, 1e-300))) - 4), 2.0 ** -10)
    bound = half * np.repeat(S.astype(np.float64), BLOCK, axis=1)[:, :384] * (1 + 2.0 ** -20)
    assert np.all(np.abs(deq - x.astype(np.float64)) <= bound + 1e-30)
    # the largest element of every block lands on +-448
    for rb, kb, rs, ks in _blocks(64, 384, 1):
        blk = np.abs(x[rs, ks].astype(np.float64))
        if blk.max() > 0:
            j = int(np.argmax(blk))
            assert Q[rs, ks].reshape(-1)[j] & 0x7F == 0x7E


def pin_quant_2d_blocks_share_scale(orc):
    rng = np.random.default_rng(84)
    x = _f16_blocks(rng, 300, 200)
    Q2, S2 = orc.quant_fp8(x, 128)
    assert S2.shape == (3, 2)
    # a 128 x 128 block quantized alone gives the same codes and scale
    for rb, kb, rs, ks in _blocks(300, 200, 128):
        Qb, Sb = orc.quant_fp8(np.ascontiguousarray(x[rs, ks]), 128)
        assert Sb.shape == (1, 1) and Sb[0, 0] == S2[rb, kb]
        assert np.array_equal(Qb, Q2[rs, ks])


# --------------------------------------------------------------------------------------
# block-scaled GEMM pins
# --------------------------------------------------------------------------------------
def _exact_fp8_gemm(A, SA, B, SB):
    Ad, Bd = _torch_decode(A), _torch_decode(B)
    M, K = A.shape
    N = B.shape[0]
    out = []
    for i in range(M):
        row = []
        for j in range(N):
            tot = Fraction(0)
            for kb in range(-(-K // BLOCK)):
                p = sum((Fraction(float(Ad[i, k])) * Fraction(float(Bd[j, k]))
                         for k in range(kb * BLOCK, min(K, kb * BLOCK + BLOCK))), Fraction(0))
                tot += Fraction(float(SA[i, kb])) * Fraction(float(SB[j // BLOCK, kb])) * p
            row.append(tot)
        out.append(row)
    return out


def pin_fp8_gemm_bruteforce_exact(orc):
    rng = np.random.default_rng(85)
    for M, N, K in [(3, 4, 1), (2, 3, 128), (4, 2, 129), (3, 3, 300), (1, 130, 40)]:
        A, B = _finite_codes(rng, (M, K)), _finite_codes(rng, (N, K))
        KB = -(-K // BLOCK)
        SA, SB = _scales(rng, (M, KB)), _scales(rng, (-(-N // BLOCK), KB))
        C = orc.gemm_fp8(A, SA, B, SB, relu=False)
        ex = _exact_fp8_gemm(A, SA, B, SB)
        Ad, Bd = np.abs(_torch_decode(A)), np.abs(_torch_decode(B))
        for i in range(M):
            for j in range(N):
                # one rounded product per block and KB - 1 rounded additions
                mag = sum(abs(float(SA[i, kb]) * float(SB[j // BLOCK, kb]))
                          * float(Ad[i, kb * BLOCK:(kb + 1) * BLOCK] @ Bd[j, kb * BLOCK:(kb + 1) * BLOCK])
                          for kb in range(KB))
                err = abs(Fraction(float(C[i, j])) - ex[i][j])
                assert err <= Fraction(2 * KB) * Fraction(1, 2 ** 53) * Fraction(mag) * (1 + Fraction(1, 2 ** 40)), \
                    (M, N, K, i, j, float(err), mag)
                if KB == 1:  # a single block: exact sum, one rounding
                    assert float(ex[i][j]) == C[i, j], (M, N, K, i, j)


def pin_fp8_gemm_unit_scales_is_f16_gemm(orc):
    rng = np.random.default_rng(86)
    M, N, K = 37, 29, 517
    A, B = _finite_codes(rng, (M, K), 0.02), _finite_codes(rng, (N, K), 0.02)
    KB = -(-K // BLOCK)
    C = orc.gemm_fp8(A, np.ones((M, KB), np.float32), B, np.ones((1, KB), np.float32), relu=False)
    Ah = _torch_decode(A).astype(np.float16)          # E4M3 values are exact in binary16
    Bh = np.ascontiguousarray(_torch_decode(B).T.astype(np.float16))
    assert np.array_equal(Ah.astype(np.float64), _torch_decode(A))
    R = orc.gemm(Ah.view(np.uint16), Bh.view(np.uint16), relu=False)
    mag = np.abs(_torch_decode(A)) @ np.abs(_torch_decode(B)).T
    assert np.all(np.abs(C - R) <= 2.0 ** -50 * mag)


def pin_fp8_gemm_closed_form(orc):
    M, N, K = 6, 300, 333
    A = np.full((M, K), 0x38, np.uint8)            # 1.0
    B = np.full((N, K), 0x38, np.uint8)
    KB = 3
    SA = np.array([[2.0 ** (i % 3) * (kb + 1) for kb in range(KB)] for i in range(M)], np.float32)
    SB = np.array([[0.5 * (jb + 1) + kb for kb in range(KB)] for jb in range(3)], np.float32)
    C = orc.gemm_fp8(A, SA, B, SB, relu=False)
    lens = [128, 128, 77]
    for i in range(M):
        for j in range(N):
            want = sum(2.0 ** (i % 3) * (kb + 1) * (0.5 * (j // 128 + 1) + kb) * lens[kb] for kb in range(KB))
            assert C[i, j] == want, (i, j, C[i, j], want)
    # negative codes (0xB8 = -1.0) flip the sign exactly; ReLU clears it
    Cn = orc.gemm_fp8(np.full((M, K), 0xB8, np.uint8), SA, B, SB, relu=False)
    assert np.array_equal(Cn, -C)
    assert np.array_equal(orc.gemm_fp8(np.full((M, K), 0xB8, np.uint8), SA, B, SB, relu=True), np.zeros_like(C))


def pin_fp8_gemm_scale_structure(orc):
    rng = np.random.default_rng(87)
    M, N, K = 9, 140, 400
    KB = 4
    A, B = _finite_codes(rng, (M, K)), _finite_codes(rng, (N, K))
    SA, SB = _scales(rng, (M, KB)), _scales(rng, (2, KB))
    C = orc.gemm_fp8(A, SA, B, SB, relu=False)
    # doubling a row's scales doubles that row exactly
    SA2 = SA.copy()
    SA2[4] *= 2
    C2 = orc.gemm_fp8(A, SA2, B, SB, relu=False)
    assert np.array_equal(C2[4], 2 * C[4]) and np.array_equal(np.delete(C2, 4, 0), np.delete(C, 4, 0))
    # the second 128-column group of outputs uses the second row of SB only
    SB2 = SB.copy()
    SB2[1] *= 4
    C3 = orc.gemm_fp8(A, SA, B, SB2, relu=False)
    assert np.array_equal(C3[:, :128], C[:, :128]) and np.array_equal(C3[:, 128:], 4 * C[:, 128:])
    # a zero scale for k-block 2 equals zeroing that block's codes
    SAz = SA.copy()
    SAz[:, 2] = 0
    Az = A.copy()
    Az[:, 256:384] = 0
    assert np.array_equal(orc.gemm_fp8(A, SAz, B, SB, relu=False), orc.gemm_fp8(Az, SA, B, SB, relu=False))
    # the product over the first block only equals the K = 128 product
    SAo = SA.copy()
    SAo[:, 1:] = 0
    C1 = orc.gemm_fp8(np.ascontiguousarray(A[:, :128]), SA[:, :1], np.ascontiguousarray(B[:, :128]), SB[:, :1],
                      relu=False)
    assert np.array_equal(orc.gemm_fp8(A, SAo, B, SB, relu=False), C1)


def pin_fp8_gemm_relu_threads_entries(orc):
    rng = np.random.default_rng(88)
    M, N, K = 23, 131, 260
    KB = 3
    A, B = _finite_codes(rng, (M, K)), _finite_codes(rng, (N, K))
    SA, SB = _scales(rng, (M, KB)), _scales(rng, (2, KB))
    C = orc.gemm_fp8(A, SA, B, SB, relu=False)
    Cr = orc.gemm_fp8(A, SA, B, SB, relu=True)
    assert np.array_equal(Cr, np.where(C > 0, C, 0.0)) and not np.signbit(Cr).any()
    assert np.array_equal(orc.gemm_fp8(A, SA, B, SB, relu=False, nthreads=1), C)
    rows, cols = rng.integers(0, M, 50), rng.integers(0, N, 50)
    assert np.array_equal(orc.gemm_fp8_entries(A, SA, B, SB, rows, cols, relu=True), Cr[rows, cols])


def pin_fp8_bound(orc):
    rng = np.random.default_rng(89)
    M, N, K = 5, 140, 300
    KB = 3
    A, B = _finite_codes(rng, (M, K)), _finite_codes(rng, (N, K))
    SA, SB = _scales(rng, (M, KB)), _scales(rng, (2, KB))
    E = orc.fp8_bound(A, SA, B, SB)
    Ad, Bd = np.abs(_torch_decode(A)), np.abs(_torch_decode(B))
    for i in range(M):
        for j in range(N):
            want = 0.0
            terms = 0.0
            for kb in range(KB):
                ks = slice(kb * BLOCK, min(K, kb * BLOCK + BLOCK))
                s = abs(float(SA[i, kb]) * float(SB[j // BLOCK, kb]))
                want += s * Ad[i, ks].max() * Bd[j, ks].max()
                terms += s * float((Ad[i, ks] * Bd[j, ks]).max())
            assert abs(E[i, j] - want) <= 1e-12 * want and E[i, j] >= terms * (1 - 1e-12)


def pin_fp8_bound_entries(orc):
    import oracle
    rng = np.random.default_rng(90)
    M, N, K = 7, 300, 520
    KB = 5
    A, B = _finite_codes(rng, (M, K)), _finite_codes(rng, (N, K))
    SA, SB = _scales(rng, (M, KB)), _scales(rng, (3, KB))
    E = orc.fp8_bound(A, SA, B, SB)
    rows, cols = rng.integers(0, M, 400), rng.integers(0, N, 400)
    got = oracle.fp8_bound_entries(A, SA, B, SB, rows, cols)
    assert np.all(np.abs(got - E[rows, cols]) <= 1e-12 * E[rows, cols])


FP8_PINS = [
    pin_e4m3_golden,
    pin_e4m3_decode_all_codes,
    pin_e4m3_encode_roundtrip,
    pin_e4m3_encode_ties_even,
    pin_e4m3_encode_vs_torch,
    pin_e4m3_saturation,
    pin_quant_scales_numpy,
    pin_quant_dequant_error,
    pin_quant_2d_blocks_share_scale,
    pin_fp8_gemm_bruteforce_exact,
    pin_fp8_gemm_unit_scales_is_f16_gemm,
    pin_fp8_gemm_closed_form,
    pin_fp8_gemm_scale_structure,
    pin_fp8_gemm_relu_threads_entries,
    pin_fp8_bound,
    pin_fp8_bound_entries,
]
