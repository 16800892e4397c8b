"""Seeded synthetic inputs for the fp16 GEMM(+ReLU) workloads.

This module holds no arithmetic of the method: it only draws random binary16
matrices from a seed, so the GPU path and the CPU oracle read the very same bytes.

Recipe (fixed): numpy ``default_rng(seed)`` (PCG64); A (M x K) is drawn before B
(K x N) from the one generator; values are drawn in float32 and rounded to binary16
with numpy's round-to-nearest-even cast. Distributions:
  * ``normal``  : standard normal times ``std``;
  * ``uniform`` : uniform on [-1, 1) (float32 ``random()`` * 2 - 1).

The workloads mirror the pages' synthetic ``randn`` float16 inputs: the 1024^3
example of "Writing High-Performance Kernels in TileLang, from GEMM to MLA"
(atlascloud.ai), section "Let's write a GEMM", and the 4096^3 fp16 benchmark of the
nxmr.cn TileLang-on-A100 write-up, section 2.2.

fp8 (E4M3) block-scaled inputs (``make_fp8_inputs``) are drawn as codes, not quantized:
sign uniform, exponent field from a normal of mean 11 and deviation 2 rounded and clipped
to 0..15, fraction uniform, the NaN pattern S.1111.111 replaced by S.1111.110 (448).
Scales are float32 2^u with u uniform on [-10, -5). Order: A codes, SA, B codes, SB. The
linear workload draws x (binary16 N(0,1)) first, then the weight codes and their scales.
No page gives fp8 inputs; these have the spread block-quantized data has (most codes
within a few binades below the block maximum 448).
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    relu: bool
    dist: str       # "normal" or "uniform"
    std: float      # standard deviation for "normal" (ignored for "uniform")
    seed: int
    trans_a: bool = False  # A handed to the library stored transposed (K x M)
    trans_b: bool = False  # B handed to the library stored transposed (N x K)

    @property
    def flop(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def scale(self) -> float:
        """sigma_A * sigma_B of the input distribution (1 for N(0,1))."""
        s = self.std if self.dist == "normal" else 1.0 / math.sqrt(3.0)
        return s * s

    def inputs(self):
        """The logical operands op(A) (M x K) and op(B) (K x N)."""
        return make_inputs(self.M, self.N, self.K, self.dist, self.std, self.seed)

    def stored(self, A, B):
        """The matrices as handed to the library: transposed copies where trans_a/trans_b."""
        return (np.ascontiguousarray(A.T) if self.trans_a else A,
                np.ascontiguousarray(B.T) if self.trans_b else B)


# The five measured configurations (seed = position, A drawn before B).
WORKLOADS = {
    "relu_1024": Workload("relu_1024", 1024, 1024, 1024, True, "normal", 1.0, 1),
    "plain_4096": Workload("plain_4096", 4096, 4096, 4096, False, "normal", 1.0, 2),
    "relu_edge_4095x3000x1000": Workload("relu_edge_4095x3000x1000", 4095, 3000, 1000, True,
                                         "uniform", 1.0, 3),
    "relu_8192": Workload("relu_8192", 8192, 8192, 8192, True, "normal", 1.0 / math.sqrt(8192.0), 4),
    "relu_tall_16384x512x4096": Workload("relu_tall_16384x512x4096", 16384, 512, 4096, True,
                                         "normal", 1.0, 5),
}

# The headline: 4096^3 with the ReLU epilogue on, same inputs as plain_4096.
HEADLINE = Workload("relu_4096", 4096, 4096, 4096, True, "normal", 1.0, 2)

# Transposed-operand GEMMs at 4096^3 on the same logical inputs: the two backward GEMMs
# of the autograd wrapper (dA = dC @ B^T takes its second operand stored transposed,
# dB = A^T @ dC its first) and both transposed with ReLU.
LAYOUT_WORKLOADS = {
    "plain_4096_nt": Workload("plain_4096_nt", 4096, 4096, 4096, False, "normal", 1.0, 2, trans_b=True),
    "plain_4096_tn": Workload("plain_4096_tn", 4096, 4096, 4096, False, "normal", 1.0, 2, trans_a=True),
    "relu_4096_tt": Workload("relu_4096_tt", 4096, 4096, 4096, True, "normal", 1.0, 2, trans_a=True,
                             trans_b=True),
}


# Small output grids: a weight-gradient GEMM of the autograd wrapper's backward
# (dB = A^T @ dC for a 1024 x 1024 weight over 32768 rows of activations, A stored
# transposed) and one GPU's row shard of the 4096^3 headline split over 8 GPUs
# (M = 4096 / 8); the shapes split-K is for.
SPLIT_WORKLOADS = {
    "plain_tn_1024x1024x32768": Workload("plain_tn_1024x1024x32768", 1024, 1024, 32768, False, "normal", 1.0, 6,
                                         trans_a=True),
    "relu_shard_512x4096x4096": Workload("relu_shard_512x4096x4096", 512, 4096, 4096, True, "normal", 1.0, 7),
}


@dataclass(frozen=True)
class GroupedWorkload:
    """Independent GEMMs of one layout: expert e multiplies its M[e] rows by its own K x N
    weight (a mixture-of-experts layer with uneven routing)."""
    name: str
    Ms: tuple
    N: int
    K: int
    relu: bool
    seed: int

    @property
    def flop(self) -> int:
        return 2 * sum(self.Ms) * self.N * self.K

    def inputs(self):
        """[(A_e, B_e)] from seeds seed, seed + 1, ... (same recipe as make_inputs)."""
        return [make_inputs(m, self.N, self.K, "normal", 1.0, self.seed + e) for e, m in enumerate(self.Ms)]


# 8 experts, 16384 routed rows in all, hidden 4096 -> expert width 2048 (the up projection).
GROUPED_WORKLOADS = {
    "moe_8x_16384x2048x4096": GroupedWorkload("moe_8x_16384x2048x4096",
                                              (3072, 2560, 2048, 2048, 1792, 1536, 1280, 2048), 2048, 4096,
                                              True, 20),
}


def all_workloads():
    """Headline, the five measured configurations, the transposed-operand ones, then the
    small-grid (split-K) ones."""
    return ([HEADLINE] + list(WORKLOADS.values()) + list(LAYOUT_WORKLOADS.values())
            + list(SPLIT_WORKLOADS.values()))


def by_name(name: str) -> Workload:
    for w in all_workloads():
        if w.name == name:
            return w
    raise KeyError(name)


def _draw(rng: np.random.Generator, shape, dist: str, std: float) -> np.ndarray:
    if dist == "normal":
        x = rng.standard_normal(shape, dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
    elif dist == "uniform":
        x = rng.random(shape, dtype=np.float32)
        x *= np.float32(2.0)
        x -= np.float32(1.0)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return x.astype(np.float16)


def make_inputs(M: int, N: int, K: int, dist: str = "normal", std: float = 1.0, seed: int = 0):
    """Return (A, B): float16 arrays of shape (M, K) and (K, N), C-contiguous."""
    rng = np.random.default_rng(seed)
    A = _draw(rng, (M, K), dist, std)
    B = _draw(rng, (K, N), dist, std)
    return A, B


FP8_BLOCK = 128


def _fp8_codes(rng: np.random.Generator, shape) -> np.ndarray:
    sign = rng.integers(0, 2, size=shape).astype(np.uint8) << 7
    e = np.clip(np.rint(rng.normal(11.0, 2.0, size=shape)), 0, 15).astype(np.uint8)
    f = rng.integers(0, 8, size=shape).astype(np.uint8)
    c = sign | (e << 3) | f
    nan = (c & 0x7F) == 0x7F
    c[nan] = (c[nan] & 0x80) | 0x7E
    return c


def _fp8_scales(rng: np.random.Generator, shape) -> np.ndarray:
    return np.exp2(rng.uniform(-10.0, -5.0, size=shape)).astype(np.float32)


def make_fp8_inputs(M: int, N: int, K: int, seed: int = 0):
    """(A codes M x K, SA M x KB, B codes N x K, SB ceil(N/128) x KB)."""
    rng = np.random.default_rng(seed)
    KB = -(-K // FP8_BLOCK)
    A = _fp8_codes(rng, (M, K))
    SA = _fp8_scales(rng, (M, KB))
    B = _fp8_codes(rng, (N, K))
    SB = _fp8_scales(rng, (-(-N // FP8_BLOCK), KB))
    return A, SA, B, SB


def make_fp8_linear_inputs(M: int, N: int, K: int, seed: int = 0):
    """(x binary16 M x K N(0,1), weight codes N x K, weight scales ceil(N/128) x KB)."""
    rng = np.random.default_rng(seed)
    x = _draw(rng, (M, K), "normal", 1.0)
    W = _fp8_codes(rng, (N, K))
    SW = _fp8_scales(rng, (-(-N // FP8_BLOCK), -(-K // FP8_BLOCK)))
    return x, W, SW


@dataclass(frozen=True)
class Fp8Workload:
    """An fp8 block-scaled GEMM (``linear`` False: pre-quantized A, SA, B, SB) or the
    fp8_block_scaled_linear step (``linear`` True: quantize x per 1 x 128, then the GEMM)."""
    name: str
    M: int
    N: int
    K: int
    relu: bool
    seed: int
    linear: bool = False

    @property
    def flop(self) -> int:
        return 2 * self.M * self.N * self.K

    @property
    def compulsory_bytes(self) -> int:
        """E4M3 operands (1 byte), float32 scales and the binary16 output, once each."""
        KB = -(-self.K // FP8_BLOCK)
        return (self.M * self.K + self.N * self.K + 2 * self.M * self.N
                + 4 * (self.M * KB + -(-self.N // FP8_BLOCK) * KB))

    def inputs(self):
        if self.linear:
            return make_fp8_linear_inputs(self.M, self.N, self.K, self.seed)
        return make_fp8_inputs(self.M, self.N, self.K, self.seed)


FP8_WORKLOADS = {
    "fp8_block_4096": Fp8Workload("fp8_block_4096", 4096, 4096, 4096, False, 30),
    "fp8_block_relu_8192": Fp8Workload("fp8_block_relu_8192", 8192, 8192, 8192, True, 31),
    "fp8_linear_4096": Fp8Workload("fp8_linear_4096", 4096, 4096, 4096, False, 32, linear=True),
}


def digest(x: np.ndarray) -> str:
    """SHA-256 of the raw bytes (recorded with results so runs can be matched)."""
    return hashlib.sha256(np.ascontiguousarray(x).tobytes()).hexdigest()
