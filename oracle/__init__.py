"""CPU oracle for C = ReLU(A @ B) on binary16 inputs -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The GPU library never routes through it:
the oracle and the HIP path share no code, header, table or helper; the only
thing both sides see is the seeded input generator in ``tgemm_workloads``.

The arithmetic lives in ``tgemm_ref.c`` (plain C11 + OpenMP, built by gcc into
``liboracle_tgemm.so`` next to this file). It follows the plain definition of the
contraction in "Writing High-Performance Kernels in TileLang, from GEMM to MLA"
(atlascloud.ai), section "Let's write a GEMM" (C = ReLU(A @ B), float16 operands,
float accumulator, max(., 0) epilogue) and "TileLang-MUSA operator development"
(7yue.com), section 3 (the same GEMM without ReLU, checked against an fp32 product):
inputs are decoded exactly to float64, summed over k ascending in float64, and ReLU
is ``x > 0 ? x : +0``.

Pins (tests/test_oracle_*.py, all CPU): exact rational brute force, the closed forms
ones @ ones = K and A @ I = A, the ReLU sign invariants, transpose and thread-count
invariance, and numpy's binary16 codec over all 65536 bit patterns.

The fp8 block-scaled GEMM and its block quantizer live in ``tgemm_fp8_ref.c`` (same
library); their reading of the pages is stated at the top of that file, and their pins
are in tests/test_oracle_fp8_pins.py (torch's CPU float8_e4m3fn codec over all 256 codes,
ties-to-even at every midpoint, exact rational brute force, reduction to the binary16
oracle when every scale is 1, closed forms and scale linearity).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "tgemm_ref.c")
FP8_SOURCE = os.path.join(_HERE, "tgemm_fp8_ref.c")
LIBRARY = os.path.join(_HERE, "liboracle_tgemm.so")


def build(src: str = SOURCE, out: str = LIBRARY, verbose: bool = False, fp8_src: str = FP8_SOURCE) -> str:
    """Compile the oracle's C sources with gcc (portable -O2, OpenMP). Always recompiles."""
    tmp = f"{out}.{os.getpid()}.tmp"  # per process: parallel test workers may build at once
    cmd = ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall",
           "-o", tmp, src, fp8_src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _as_u16(x: np.ndarray) -> np.ndarray:
    """View a float16 / uint16 array as its uint16 bit patterns (no value conversion)."""
    x = np.asarray(x)
    if x.dtype == np.float16:
        x = x.view(np.uint16)
    if x.dtype != np.uint16:
        raise TypeError(f"expected float16 or uint16 bits, got {x.dtype}")
    return x


def _rowmajor_2d(x: np.ndarray):
    """Return (array, leading dimension in elements) for a 2-D row-major view."""
    if x.ndim != 2:
        raise ValueError("expected a 2-D array")
    if x.shape[0] > 0 and x.shape[1] > 0 and x.strides[1] != x.itemsize:
        x = np.ascontiguousarray(x)
    if x.shape[0] > 1 and x.strides[0] % x.itemsize == 0 and x.strides[0] >= x.shape[1] * x.itemsize:
        ld = x.strides[0] // x.itemsize
    else:
        x = np.ascontiguousarray(x)
        ld = max(1, x.shape[1])
    return x, ld


class Oracle:
    """One loaded build of the oracle library (the default one, or a test build)."""

    def __init__(self, path: str = LIBRARY):
        lib = ctypes.CDLL(path)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.oracle_f16_decode.restype = ctypes.c_double
        lib.oracle_f16_decode.argtypes = [ctypes.c_uint16]
        lib.oracle_f16_encode_rne.restype = ctypes.c_uint16
        lib.oracle_f16_encode_rne.argtypes = [ctypes.c_double]
        lib.oracle_f16_decode_array.argtypes = [p, p, i64]
        lib.oracle_f16_encode_array.argtypes = [p, p, i64]
        lib.oracle_gemm_f16.restype = ctypes.c_int
        lib.oracle_gemm_f16.argtypes = [i64, i64, i64, p, i64, p, i64, p, i64,
                                        ctypes.c_int, ctypes.c_int]
        lib.oracle_gemm_f16_entries.restype = None
        lib.oracle_gemm_f16_entries.argtypes = [i64, p, i64, p, i64, i64, p, p, p,
                                                ctypes.c_int, ctypes.c_int]
        lib.oracle_max_threads.restype = ctypes.c_int
        lib.oracle_e4m3_decode.restype = ctypes.c_double
        lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_encode_sat.restype = ctypes.c_uint8
        lib.oracle_e4m3_encode_sat.argtypes = [ctypes.c_double]
        lib.oracle_e4m3_decode_array.argtypes = [p, p, i64]
        lib.oracle_e4m3_encode_array.argtypes = [p, p, i64]
        lib.oracle_quant_fp8.restype = None
        lib.oracle_quant_fp8.argtypes = [i64, i64, p, i64, i64, p, i64, p]
        lib.oracle_gemm_fp8_block.restype = ctypes.c_int
        lib.oracle_gemm_fp8_block.argtypes = [i64, i64, i64, p, i64, p, p, i64, p, p, i64,
                                              ctypes.c_int, ctypes.c_int]
        lib.oracle_gemm_fp8_block_entries.restype = None
        lib.oracle_gemm_fp8_block_entries.argtypes = [i64, p, i64, p, p, i64, p, i64, p, p, p,
                                                      ctypes.c_int, ctypes.c_int]
        lib.oracle_fp8_block_bound.restype = None
        lib.oracle_fp8_block_bound.argtypes = [i64, i64, i64, p, i64, p, p, i64, p, p]
        self.lib = lib
        self.path = path

    def f16_decode(self, bits: np.ndarray) -> np.ndarray:
        """Exact binary16 -> float64 decode of every element (the oracle's own codec)."""
        b = np.ascontiguousarray(_as_u16(bits))
        out = np.empty(b.shape, dtype=np.float64)
        self.lib.oracle_f16_decode_array(b.ctypes.data, out.ctypes.data, b.size)
        return out

    def f16_encode(self, x: np.ndarray) -> np.ndarray:
        """float64 -> binary16 bits, round to nearest even (the oracle's own codec)."""
        x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
        out = np.empty(x.shape, dtype=np.uint16)
        self.lib.oracle_f16_encode_array(x.ctypes.data, out.ctypes.data, x.size)
        return out

    def gemm(self, A: np.ndarray, B: np.ndarray, relu: bool, nthreads: int = 0) -> np.ndarray:
        """Full product ReLU?(A @ B) in float64 from binary16 A (M x K) and B (K x N)."""
        A, lda = _rowmajor_2d(_as_u16(A))
        B, ldb = _rowmajor_2d(_as_u16(B))
        M, K = A.shape
        K2, N = B.shape
        if K != K2:
            raise ValueError(f"inner dimensions differ: {A.shape} @ {B.shape}")
        C = np.empty((M, N), dtype=np.float64)
        if M == 0 or N == 0:
            return C
        rc = self.lib.oracle_gemm_f16(M, N, K, A.ctypes.data, lda, B.ctypes.data, ldb,
                                      C.ctypes.data, N, int(bool(relu)), int(nthreads))
        if rc != 0:
            raise MemoryError("oracle could not allocate its decode buffer")
        return C

    def gemm_entries(self, A: np.ndarray, B: np.ndarray, rows, cols, relu: bool,
                     nthreads: int = 0) -> np.ndarray:
        """Entries (rows[t], cols[t]) of ReLU?(A @ B), one by one, bitwise equal to gemm()."""
        A, lda = _rowmajor_2d(_as_u16(A))
        B, ldb = _rowmajor_2d(_as_u16(B))
        M, K = A.shape
        K2, N = B.shape
        if K != K2:
            raise ValueError(f"inner dimensions differ: {A.shape} @ {B.shape}")
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        cols = np.ascontiguousarray(np.asarray(cols, dtype=np.int64))
        if rows.shape != cols.shape:
            raise ValueError("rows and cols differ in shape")
        if rows.size and (rows.min() < 0 or rows.max() >= M or cols.min() < 0 or cols.max() >= N):
            raise IndexError("entry index out of range")
        out = np.empty(rows.shape, dtype=np.float64)
        self.lib.oracle_gemm_f16_entries(K, A.ctypes.data, lda, B.ctypes.data, ldb, rows.size,
                                         rows.ctypes.data, cols.ctypes.data, out.ctypes.data,
                                         int(bool(relu)), int(nthreads))
        return out

    def max_threads(self) -> int:
        return int(self.lib.oracle_max_threads())

    # ---------------------------------------------------------------- fp8 (E4M3) path
    def e4m3_decode(self, codes: np.ndarray) -> np.ndarray:
        """Exact E4M3 code -> float64 of every element (the oracle's own codec)."""
        c = np.ascontiguousarray(np.asarray(codes, dtype=np.uint8))
        out = np.empty(c.shape, dtype=np.float64)
        self.lib.oracle_e4m3_decode_array(c.ctypes.data, out.ctypes.data, c.size)
        return out

    def e4m3_encode(self, x: np.ndarray) -> np.ndarray:
        """float64 -> E4M3 code, nearest even, saturating to +-448 (the oracle's own codec)."""
        x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
        out = np.empty(x.shape, dtype=np.uint8)
        self.lib.oracle_e4m3_encode_array(x.ctypes.data, out.ctypes.data, x.size)
        return out

    def quant_fp8(self, X: np.ndarray, block_rows: int):
        """Block quantizer: binary16 X (R x K) -> (codes R x K uint8, scales RB x KB float32)."""
        X, ldx = _rowmajor_2d(_as_u16(X))
        R, K = X.shape
        if block_rows < 1:
            raise ValueError("block_rows must be positive")
        KB = -(-K // FP8_BLOCK)
        RB = -(-R // block_rows)
        Q = np.zeros((R, K), dtype=np.uint8)
        S = np.zeros((RB, KB), dtype=np.float32)
        if R and K:
            self.lib.oracle_quant_fp8(R, K, X.ctypes.data, ldx, block_rows, Q.ctypes.data, max(1, K),
                                      S.ctypes.data)
        return Q, S

    @staticmethod
    def _fp8_operands(A, SA, B, SB):
        A, lda = _rowmajor_2d(np.asarray(A, dtype=np.uint8))
        B, ldb = _rowmajor_2d(np.asarray(B, dtype=np.uint8))
        M, K = A.shape
        N, K2 = B.shape
        if K != K2:
            raise ValueError(f"inner dimensions differ: A {A.shape}, B (N x K) {B.shape}")
        KB = -(-K // FP8_BLOCK)
        SA = np.ascontiguousarray(np.asarray(SA, dtype=np.float32))
        SB = np.ascontiguousarray(np.asarray(SB, dtype=np.float32))
        if SA.shape != (M, KB) or SB.shape != (-(-N // FP8_BLOCK), KB):
            raise ValueError(f"scale shapes {SA.shape}, {SB.shape} do not match M={M} N={N} K={K}")
        return A, lda, SA, B, ldb, SB, M, N, K

    def gemm_fp8(self, A, SA, B, SB, relu: bool, nthreads: int = 0) -> np.ndarray:
        """Block-scaled product (float64, unrounded): A (M x K) and B (N x K) E4M3 codes,
        SA (M x KB) and SB (ceil(N/128) x KB) float32 scales."""
        A, lda, SA, B, ldb, SB, M, N, K = self._fp8_operands(A, SA, B, SB)
        C = np.empty((M, N), dtype=np.float64)
        if M and N:
            self.lib.oracle_gemm_fp8_block(M, N, K, A.ctypes.data, lda, SA.ctypes.data, B.ctypes.data, ldb,
                                           SB.ctypes.data, C.ctypes.data, N, int(bool(relu)), int(nthreads))
        return C

    def gemm_fp8_entries(self, A, SA, B, SB, rows, cols, relu: bool, nthreads: int = 0) -> np.ndarray:
        A, lda, SA, B, ldb, SB, M, N, K = self._fp8_operands(A, SA, B, SB)
        rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        cols = np.ascontiguousarray(np.asarray(cols, dtype=np.int64))
        if rows.shape != cols.shape:
            raise ValueError("rows and cols differ in shape")
        if rows.size and (rows.min() < 0 or rows.max() >= M or cols.min() < 0 or cols.max() >= N):
            raise IndexError("entry index out of range")
        out = np.empty(rows.shape, dtype=np.float64)
        self.lib.oracle_gemm_fp8_block_entries(K, A.ctypes.data, lda, SA.ctypes.data, B.ctypes.data, ldb,
                                               SB.ctypes.data, rows.size, rows.ctypes.data, cols.ctypes.data,
                                               out.ctypes.data, int(bool(relu)), int(nthreads))
        return out

    def fp8_bound(self, A, SA, B, SB) -> np.ndarray:
        """sum_kb |SA SB| * max|a| * max|w| per output element (float64, M x N)."""
        A, lda, SA, B, ldb, SB, M, N, K = self._fp8_operands(A, SA, B, SB)
        E = np.zeros((M, N), dtype=np.float64)
        if M and N:
            self.lib.oracle_fp8_block_bound(M, N, K, A.ctypes.data, lda, SA.ctypes.data, B.ctypes.data, ldb,
                                            SB.ctypes.data, E.ctypes.data)
        return E


_default = None


def default() -> Oracle:
    """The oracle built from tgemm_ref.c (compiled on first use if missing or stale)."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY) or os.path.getmtime(LIBRARY) < max(
                os.path.getmtime(SOURCE), os.path.getmtime(FP8_SOURCE)):
            build()
        _default = Oracle(LIBRARY)
    return _default


def f16_decode(bits):
    return default().f16_decode(bits)


def f16_encode(x):
    return default().f16_encode(x)


def gemm(A, B, relu, nthreads=0):
    return default().gemm(A, B, relu, nthreads)


def gemm_entries(A, B, rows, cols, relu, nthreads=0):
    return default().gemm_entries(A, B, rows, cols, relu, nthreads)


def max_threads() -> int:
    return default().max_threads()


FP8_BLOCK = 128


def e4m3_decode(codes):
    return default().e4m3_decode(codes)


def e4m3_encode(x):
    return default().e4m3_encode(x)


def quant_fp8(X, block_rows):
    return default().quant_fp8(X, block_rows)


def gemm_fp8(A, SA, B, SB, relu, nthreads=0):
    return default().gemm_fp8(A, SA, B, SB, relu, nthreads)


def gemm_fp8_entries(A, SA, B, SB, rows, cols, relu, nthreads=0):
    return default().gemm_fp8_entries(A, SA, B, SB, rows, cols, relu, nthreads)


def fp8_bound(A, SA, B, SB):
    return default().fp8_bound(A, SA, B, SB)


def fp8_bound_entries(A, SA, B, SB, rows, cols) -> np.ndarray:
    """fp8_bound at entries (rows[t], cols[t]) only, for sizes where the full matrix is too
    slow. Per (row, block) maxima are taken on the codes' magnitude bits (their order is the
    order of the values for finite codes) and decoded with the oracle's codec."""
    A = np.asarray(A, dtype=np.uint8)
    B = np.asarray(B, dtype=np.uint8)
    M, K = A.shape
    N = B.shape[0]
    KB = -(-K // FP8_BLOCK)
    mag = np.abs(e4m3_decode(np.arange(128, dtype=np.uint8)))

    def block_max(X):
        R = X.shape[0]
        pad = np.zeros((R, KB * FP8_BLOCK), dtype=np.uint8)
        pad[:, :K] = X & 0x7F
        return mag[pad.reshape(R, KB, FP8_BLOCK).max(axis=2)]

    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    am = block_max(A) * np.abs(np.asarray(SA, dtype=np.float64))
    bm = block_max(B) * np.abs(np.asarray(SB, dtype=np.float64))[np.arange(N) // FP8_BLOCK]
    return np.einsum("tk,tk->t", am[rows], bm[cols])


# --------------------------------------------------------------------------------------
# Tolerance: |c - ref| <= 4e-3 * |ref| + 1e-3 * sqrt(K), elementwise, with c the decoded
# binary16 GPU output and ref the oracle's unrounded float64 value. The relative term
# covers the final rounding to binary16 (at most 2^-11 relative); the absolute term covers
# float32 accumulation in any order. A second, scale-aware form replaces sqrt(K) by
# sigma_A * sigma_B * sqrt(K) for inputs drawn with a standard deviation other than 1.
# --------------------------------------------------------------------------------------
REL_TOL = 4e-3
ABS_TOL_PER_SQRT_K = 1e-3


def tolerance(ref: np.ndarray, K: int, scale: float = 1.0) -> np.ndarray:
    return REL_TOL * np.abs(ref) + ABS_TOL_PER_SQRT_K * scale * math.sqrt(max(K, 1))


def compare(c_bits: np.ndarray, ref: np.ndarray, K: int, scale: float = 1.0) -> dict:
    """Compare binary16 output bits against the float64 reference; returns a report."""
    c = f16_decode(c_bits)
    if c.shape != ref.shape:
        raise ValueError(f"shape mismatch {c.shape} vs {ref.shape}")
    err = np.abs(c - ref)
    tol = tolerance(ref, K, scale)
    bad = ~(err <= tol)  # NaN counts as a failure
    ratio = np.where(tol > 0, err / tol, np.inf)
    return {
        "n": int(c.size),
        "fails": int(bad.sum()),
        "max_abs_err": float(err.max()) if c.size else 0.0,
        "max_ratio": float(np.nanmax(ratio)) if c.size else 0.0,
        "first_fail": (tuple(int(v) for v in np.argwhere(bad)[0]) if bad.any() else None),
    }


# --------------------------------------------------------------------------------------
# Tolerance of the fp8 path: |c - ref| <= 4e-3 * |ref| + 2^-8 * E, elementwise, with E =
# sum_kb |SA SB| * max|a| * max|w| (fp8_bound). The fp8 matrix instructions of gfx950 sum
# the 128 products of a block with less than float32 precision (measured: deviations up
# to 2^-10.1 of the block's largest product, none when all products share a binade); the
# method applies the scales and accumulates across blocks in float32 after each block,
# which is what the block-sized scaling is for. 2^-8 keeps a 4x margin over the measured
# deviation; float32 rounding of the scaled block sums (<= 2^-17 E) and the final rounding
# to binary16 (covered by the relative term) sit far below it.
# --------------------------------------------------------------------------------------
FP8_BLOCK_ERR = 2.0 ** -8


def tolerance_fp8(ref: np.ndarray, bound: np.ndarray) -> np.ndarray:
    return REL_TOL * np.abs(ref) + FP8_BLOCK_ERR * bound


def compare_fp8(c_bits: np.ndarray, ref: np.ndarray, bound: np.ndarray) -> dict:
    """Compare binary16 output bits of the fp8 path against the float64 reference."""
    c = f16_decode(c_bits)
    if c.shape != ref.shape or bound.shape != ref.shape:
        raise ValueError(f"shape mismatch {c.shape} / {ref.shape} / {bound.shape}")
    err = np.abs(c - ref)
    tol = tolerance_fp8(ref, bound)
    bad = ~(err <= tol)
    ratio = np.where(tol > 0, err / np.where(tol > 0, tol, 1.0), np.where(err > 0, np.inf, 0.0))
    return {
        "n": int(c.size),
        "fails": int(bad.sum()),
        "max_abs_err": float(err.max()) if c.size else 0.0,
        "max_ratio": float(ratio.max()) if c.size else 0.0,
        "first_fail": (tuple(int(v) for v in np.argwhere(bad)[0]) if bad.any() else None),
    }
