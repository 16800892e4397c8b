"""Helpers for the GPU tests: move seeded numpy fp16 inputs to the device, run the library
through its C ABI (via the binding), read the fp16 output bits back."""
from __future__ import annotations

import math

import numpy as np

import oracle
import tiled_dense_gemm_04_amd as tg


def torch_cuda():
    import torch
    return torch


def to_dev(x: np.ndarray):
    torch = torch_cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda")


def library_for(cfg, fp8: bool = False):
    """The build that compiles table row ``cfg``: the product library (None, the binding's
    default) unless the row is a sweep-only variant, then the tooling build."""
    if cfg is None or cfg < 0:
        return None
    desc = tg.tgemm_fp8_config_desc(cfg) if fp8 else tg.tgemm_config_desc(cfg)
    return None if desc["built"] else tg.stamps_lib()


def run(A: np.ndarray, B: np.ndarray, relu: bool, cfg=None, stream=None, trans_a=False,
        trans_b=False) -> np.ndarray:
    """fp16 numpy in (the logical op(A) M x K and op(B) K x N) -> fp16 output bits (uint16
    numpy) out. With trans_a / trans_b the operand goes to the library stored transposed
    (a row-major copy of its transpose) through gemm_f16_ex. A sweep-only config runs on
    the tooling build."""
    torch = torch_cuda()
    a = to_dev(A.T if trans_a else A)
    b = to_dev(B.T if trans_b else B)
    c = torch.full((A.shape[0], B.shape[1]), float("nan"), dtype=torch.float16, device="cuda")
    tg.gemm_f16_ex(a, b, c, trans_a=trans_a, trans_b=trans_b, relu=relu, cfg=cfg, stream=stream,
                   library=library_for(cfg))
    torch.cuda.synchronize()
    return c.cpu().numpy().view(np.uint16)


def assert_close(c_bits: np.ndarray, ref: np.ndarray, K: int, scale: float = 1.0, what: str = ""):
    rep = oracle.compare(c_bits, ref, K, scale)
    assert rep["fails"] == 0, f"{what}: {rep}"
    return rep


def log(msg: str):
    print(msg, flush=True)


def sample_entries(M: int, N: int, rng: np.random.Generator, n_rows=8, n_cols=8, n_rand=8192):
    """Entry coordinates for sampled checks at full size: a few whole rows and whole
    columns (first, last and random ones, which cross every tile edge) plus random entries."""
    rows = np.unique(np.concatenate([[0, M - 1], rng.integers(0, M, n_rows)]))
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, n_cols)]))
    rr = [np.repeat(rows, N), np.repeat(np.arange(M), len(cols)), rng.integers(0, M, n_rand)]
    cc = [np.tile(np.arange(N), len(rows)), np.tile(cols, M), rng.integers(0, N, n_rand)]
    return np.concatenate(rr), np.concatenate(cc)


def relu_bits(plain_bits: np.ndarray) -> np.ndarray:
    """max(x, +0) applied to fp16 bit patterns (what ReLU before rounding must give)."""
    v = plain_bits.view(np.float16)
    return np.where(v > 0, plain_bits, np.uint16(0)).astype(np.uint16)


def sqrt_k(K):
    return math.sqrt(max(K, 1))
