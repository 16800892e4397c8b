"""GPU parity of split-K (gemm_f16_ws / gemm_f16_ws_cfg): every split-capable config, split
counts 2 .. 8, all four operand layouts, against the CPU oracle element by element; the
ordered fixup must make repeated calls bit-identical; one workspace serves calls of
different shapes in turn (each call leaves its counters at zero); the planned splits of
the small measured workloads against the whole oracle matrix."""
import numpy as np
import pytest

import oracle
import tgemm_workloads as W
from gpu_util import assert_close, library_for, log, to_dev, torch_cuda

import tiled_dense_gemm_04_amd as tg

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = torch_cuda()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tg.lib()
    oracle.default()
    return torch


def _split_cfgs():
    return [i for i, c in enumerate(tg.configs()) if c["layouts"] == 0xF and not c["generic"]]


def _run_ws(A, B, relu, cfg, splits, ta=False, tb=False, workspace=None):
    torch = torch_cuda()
    a = to_dev(A.T if ta else A)
    b = to_dev(B.T if tb else B)
    c = torch.full((A.shape[0], B.shape[1]), float("nan"), dtype=torch.float16, device="cuda")
    tg.gemm_f16_ws(a, b, c, ta, tb, relu=relu, cfg=cfg, splits=splits, workspace=workspace,
                   library=library_for(cfg))
    torch.cuda.synchronize()
    return c.cpu().numpy().view(np.uint16)


SHAPES = [(520, 392, 1000), (256, 256, 512), (136, 264, 2048), (1000, 1032, 520), (8, 8, 264)]


@pytest.mark.parametrize("cfg_pos", range(5))
def test_split_each_config_and_layout(cfg_pos):
    cfgs = _split_cfgs()
    if cfg_pos >= len(cfgs):
        pytest.skip("no such config")
    idx = cfgs[cfg_pos]
    bk = tg.tgemm_config_desc(idx)["block_k"]
    for s, (M, N, K) in enumerate(SHAPES):
        A, B = W.make_inputs(M, N, K, "normal", 1.0, seed=1100 + s)
        ref = oracle.gemm(A, B, True)
        for splits in (2, 3, 5, 8):
            if splits > -(-K // bk):
                continue
            ta, tb = (s + splits) % 2, (s + splits // 2) % 2
            log(f"split cfg {idx} splits {splits} {M}x{N}x{K} layout {ta}{tb}")
            c = _run_ws(A, B, True, idx, splits, bool(ta), bool(tb))
            assert_close(c, ref, K, what=f"cfg{idx} x{splits} {M}x{N}x{K} layout {ta}{tb}")


def test_split_deterministic_and_workspace_reuse(gpu):
    torch = gpu
    idx = _split_cfgs()[0]
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    cases = [(1000, 1032, 1024, 4), (256, 256, 512, 2), (1000, 1032, 1024, 4), (520, 392, 1000, 8)]
    first = {}
    for n, (M, N, K, splits) in enumerate(cases):
        A, B = W.make_inputs(M, N, K, "uniform", 1.0, seed=1200 + M)
        log(f"workspace reuse call {n}: {M}x{N}x{K} splits {splits}")
        c = _run_ws(A, B, n % 2 == 0, idx, splits, workspace=ws)
        assert_close(c, oracle.gemm(A, B, n % 2 == 0), K, scale=1 / 3, what=f"reuse call {n}")
        key = (M, N, K, splits)
        if key in first:
            assert np.array_equal(first[key], c), "split-K result changed between identical calls"
        first[key] = c
    # every call left the counter region zero
    torch.cuda.synchronize()
    assert int(ws[:4096].count_nonzero()) == 0


@pytest.mark.parametrize("name", list(W.SPLIT_WORKLOADS))
def test_planned_split_workloads_every_element(name):
    w = W.SPLIT_WORKLOADS[name]
    A, B = w.inputs()
    SA, SB = w.stored(A, B)
    plan = tg.tgemm_split_plan(w.trans_a, w.trans_b, w.M, w.N, w.K)
    log(f"workload {name} split plan {plan}")
    torch = torch_cuda()
    c = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
    tg.gemm_f16_ws(to_dev(SA), to_dev(SB), c, w.trans_a, w.trans_b, relu=w.relu)
    torch.cuda.synchronize()
    got = c.cpu().numpy().view(np.uint16)
    assert_close(got, oracle.gemm(A, B, w.relu), w.K, w.scale, name)
    if plan[1] == 1:
        # the table found the unsplit choice fastest here: split it anyway, at full size
        idx = [i for i, cd in enumerate(tg.configs()) if cd["name"].startswith("m128x128x32")][0]
        log(f"workload {name} forced split cfg {idx} x2")
        tg.gemm_f16_ws(to_dev(SA), to_dev(SB), c, w.trans_a, w.trans_b, relu=w.relu, cfg=idx, splits=2)
        torch.cuda.synchronize()
        assert_close(c.cpu().numpy().view(np.uint16), oracle.gemm(A, B, w.relu), w.K, w.scale, name + " x2")
    # the unsplit kernel agrees within the same tolerance (only the summation order differs)
    assert_close(got, oracle.gemm(A, B, w.relu), w.K, w.scale, name)
    c2 = torch.empty_like(c)
    tg.gemm_f16_ex(to_dev(SA), to_dev(SB), c2, w.trans_a, w.trans_b, relu=w.relu)
    torch.cuda.synchronize()
    assert_close(c2.cpu().numpy().view(np.uint16), oracle.gemm(A, B, w.relu), w.K, w.scale, name + " unsplit")


def test_no_split_needs_no_workspace(gpu):
    torch = gpu
    M = N = K = 1024
    assert tg.tgemm_workspace_bytes(0, 0, M, N, K) == 0
    A, B = W.make_inputs(M, N, K, "normal", 1.0, seed=77)
    a, b = to_dev(A), to_dev(B)
    c = torch.empty((M, N), dtype=torch.float16, device="cuda")
    log("gemm_f16_ws without a workspace on a grid that does not split")
    rc = tg.lib().gemm_f16_ws(0, 0, M, N, K, a.data_ptr(), K, b.data_ptr(), N, c.data_ptr(), N, 1, None, 0,
                              torch.cuda.current_stream().cuda_stream)
    assert rc == tg.TGEMM_OK
    c0 = tg.gemm_f16(a, b, relu=True)
    torch.cuda.synchronize()
    assert torch.equal(c, c0)
