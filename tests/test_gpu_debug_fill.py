"""The debugging build libtgemm_debugfill.so (TGEMM_DEBUG_FILL) on the GPU: every LDS copy
destination is overwritten with NaN bytes and that write awaited before the copy is
issued, so a fragment read that runs ahead of its copy's wait or barrier, or behind the
next copy into its slot, reads NaN and the output shows it. Every config the build
compiles (fp16 in all the layouts it takes, fp8), split-K and grouped launches run on
shapes with ragged tails against the oracle; the outputs must also equal the product
library's bit for bit (the poison only ever sits in bytes that a copy overwrites)."""
import numpy as np
import pytest

import oracle
import tgemm_workloads as W
from gpu_util import assert_close, log, to_dev, torch_cuda

import tiled_dense_gemm_04_amd as tg

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = torch_cuda()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tg.lib()
    tg.debugfill_lib()
    oracle.default()
    return torch


SHAPES = [(520, 392, 1000), (256, 256, 64), (1000, 1032, 520), (136, 264, 2048)]


def _run(lib, A, B, relu, cfg, ta, tb):
    torch = torch_cuda()
    a = to_dev(A.T if ta else A)
    b = to_dev(B.T if tb else B)
    c = torch.full((A.shape[0], B.shape[1]), float("nan"), dtype=torch.float16, device="cuda")
    tg.gemm_f16_ex(a, b, c, trans_a=ta, trans_b=tb, relu=relu, cfg=cfg, library=lib)
    torch.cuda.synchronize()
    return c.cpu().numpy().view(np.uint16)


def test_every_built_config_and_layout():
    D, P = tg.debugfill_lib(), tg.lib()
    for idx, cdesc in enumerate(tg.configs()):
        if not cdesc["built"]:
            continue
        for s, (M, N, K) in enumerate(SHAPES):
            A, B = W.make_inputs(M, N, K, "normal", 1.0, seed=3100 + s)
            ref = oracle.gemm(A, B, True)
            for lay in range(4):
                if not (cdesc["layouts"] >> lay) & 1:
                    continue
                ta, tb = bool(lay & 2), bool(lay & 1)
                log(f"debug fill cfg {idx} {cdesc['name']} {M}x{N}x{K} layout {lay}")
                got = _run(D, A, B, True, idx, ta, tb)
                assert_close(got, ref, K, what=f"debug fill cfg{idx} {M}x{N}x{K} layout {lay}")
                assert np.array_equal(got, _run(P, A, B, True, idx, ta, tb)), "differs from the product library"


def test_split_k_and_grouped():
    torch = torch_cuda()
    D = tg.debugfill_lib()
    for s, (M, N, K) in enumerate([(256, 256, 4096), (520, 392, 3000)]):
        A, B = W.make_inputs(M, N, K, "normal", 1.0, seed=3200 + s)
        ref = oracle.gemm(A, B, True)
        a, b = to_dev(A), to_dev(B)
        for cfg in (9, 15):
            for splits in (2, 5):
                c = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
                log(f"debug fill split cfg {cfg} x{splits} {M}x{N}x{K}")
                tg.gemm_f16_ws(a, b, c, relu=True, cfg=cfg, splits=splits, library=D)
                torch.cuda.synchronize()
                assert_close(c.cpu().numpy().view(np.uint16), ref, K, what=f"split cfg{cfg} x{splits}")
    shapes = [(300, 264, 136), (512, 384, 192), (64, 8, 8)]
    ins = [W.make_inputs(M, N, K, "uniform", 1.0, seed=3300 + i) for i, (M, N, K) in enumerate(shapes)]
    log("debug fill grouped")
    outs = tg.gemm_f16_grouped([(to_dev(A), to_dev(B)) for A, B in ins], relu=False, library=D)
    torch.cuda.synchronize()
    for (A, B), c, (M, N, K) in zip(ins, outs, shapes):
        assert_close(c.cpu().numpy().view(np.uint16), oracle.gemm(A, B, False), K, scale=1 / 3, what="grouped")


def test_fp8_every_built_config():
    torch = torch_cuda()
    D = tg.debugfill_lib()
    for cfg, cdesc in enumerate(tg.fp8_configs()):
        if not cdesc["built"]:
            continue
        for s, (M, N, K) in enumerate([(300, 264, 1008), (520, 392, 272), (257, 136, 2048)]):
            A, SA, B, SB = W.make_fp8_inputs(M, N, K, seed=3400 + s)
            a, sa, b, sb = (to_dev(x) for x in (A, SA, B, SB))
            c = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
            log(f"debug fill fp8 cfg {cfg} {M}x{N}x{K}")
            tg.gemm_fp8_block(a, sa, b, sb, c, relu=False, cfg=cfg, library=D)
            torch.cuda.synchronize()
            rep = oracle.compare_fp8(c.cpu().numpy().view(np.uint16), oracle.gemm_fp8(A, SA, B, SB, False),
                                     oracle.fp8_bound(A, SA, B, SB))
            assert rep["fails"] == 0, (cfg, M, N, K, rep)
