"""GPU parity of the transposed-operand GEMMs (gemm_f16_ex): op(A) @ op(B) with A given
as M x K or K x M and B as K x N or N x K, against the CPU oracle on the logical
operands, element by element; on the fast path the four layouts of the same logical
operands must also agree bit for bit (every layout feeds the MFMAs the same fragments).
Also the autograd wrapper's backward, dA = dC @ B^T and dB = A^T @ dC."""
import numpy as np
import pytest

import oracle
import tgemm_workloads as W
from gpu_util import assert_close, log, run, to_dev, torch_cuda

import tiled_dense_gemm_04_amd as tg

pytestmark = pytest.mark.gpu

LAYOUTS = [(0, 0), (0, 1), (1, 0), (1, 1)]


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = torch_cuda()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tg.lib()
    oracle.default()
    return torch


def _all_layout_cfgs():
    return [i for i, c in enumerate(tg.configs()) if c["layouts"] == 0xF]


# M, N, K multiples of 8 (the fast path's contiguous dimensions), ragged against the tiles
FAST_SHAPES = [(256, 256, 64), (520, 392, 264), (136, 264, 1000), (8, 8, 8), (1024, 256, 24),
               (264, 128, 40), (392, 520, 136)]
ODD_SHAPES = [(17, 23, 29), (65, 63, 33), (1, 1, 1), (130, 7, 250)]


@pytest.mark.parametrize("cfg_pos", range(6))
def test_layouts_each_config(cfg_pos):
    cfgs = _all_layout_cfgs()
    if cfg_pos >= len(cfgs):
        pytest.skip("no such config")
    idx = cfgs[cfg_pos]
    desc = tg.tgemm_config_desc(idx)
    shapes = FAST_SHAPES + (ODD_SHAPES if desc["generic"] else [])
    for s, (M, N, K) in enumerate(shapes):
        A, B = W.make_inputs(M, N, K, "normal", 1.0, seed=300 + s)
        ref = oracle.gemm(A, B, True)
        outs = {}
        for ta, tb in LAYOUTS:
            log(f"cfg {idx} {desc['name']} {M}x{N}x{K} trans_a={ta} trans_b={tb}")
            outs[(ta, tb)] = run(A, B, True, cfg=idx, trans_a=bool(ta), trans_b=bool(tb))
            assert_close(outs[(ta, tb)], ref, K, what=f"cfg{idx} {M}x{N}x{K} layout {ta}{tb}")
        if not desc["generic"]:
            for lay in LAYOUTS[1:]:
                assert np.array_equal(outs[lay], outs[(0, 0)]), f"layout {lay} differs bitwise from NN"


def test_layout_edge_sweep_default_selection():
    rng = np.random.default_rng(31)
    edge8 = [8, 16, 24, 56, 64, 72, 120, 128, 136, 248, 256, 264]
    edge = [1, 15, 17, 31, 63, 65, 127, 129, 255, 257]
    for t in range(48):
        ta, tb = LAYOUTS[t % 4]
        pool = edge8 if t % 3 else edge
        M, N, K = (int(v) for v in rng.choice(pool, 3))
        A, B = W.make_inputs(M, N, K, "uniform", 1.0, seed=700 + t)
        relu = bool(t % 2)
        cfg = tg.tgemm_select_config_ex(ta, tb, M, N, K, 16, M if ta else K, 16, K if tb else N, 16, N)
        log(f"layout edge M={M} N={N} K={K} trans_a={ta} trans_b={tb} relu={relu} cfg={cfg}")
        c = run(A, B, relu, trans_a=bool(ta), trans_b=bool(tb))
        assert_close(c, oracle.gemm(A, B, relu), K, scale=1 / 3, what=f"{M}x{N}x{K} layout {ta}{tb}")


@pytest.mark.parametrize("ta,tb", [(0, 1), (1, 0), (1, 1)])
def test_layouts_full_size_4096(ta, tb):
    """4096^3 with each transposed layout: every element against the oracle, and bit for
    bit the NN result (the headline's inputs)."""
    w = W.HEADLINE
    A, B = w.inputs()
    log(f"4096^3 layout {ta}{tb} (cfg {tg.tgemm_select_config_ex(ta, tb, w.M, w.N, w.K, 16, w.M if ta else w.K, 16, w.K if tb else w.N, 16, w.N)})")
    c = run(A, B, True, trans_a=bool(ta), trans_b=bool(tb))
    c0 = run(A, B, True)
    assert np.array_equal(c, c0)
    assert_close(c, oracle.gemm(A, B, True), w.K, what=f"4096 layout {ta}{tb}")


def test_autograd_backward(gpu):
    """The pages' wrapper: forward C = A @ B, backward dA = dC @ B^T, dB = A^T @ dC, all
    three through the library; each against the oracle on the same fp16 values."""
    torch = gpu
    M, N, K = 520, 392, 264
    A, B = W.make_inputs(M, N, K, "normal", 1.0, seed=41)
    dC, _ = W.make_inputs(M, 8, N, "normal", 1.0, seed=42)  # an M x N upstream gradient
    a = to_dev(A).requires_grad_(True)
    b = to_dev(B).requires_grad_(True)
    log("autograd forward/backward 520x392x264")
    c = tg.GemmFunction.apply(a, b)
    c.backward(to_dev(dC))
    torch.cuda.synchronize()
    assert_close(c.detach().cpu().numpy().view(np.uint16), oracle.gemm(A, B, False), K, what="forward")
    dA_ref = oracle.gemm(dC, np.ascontiguousarray(B.T), False)
    dB_ref = oracle.gemm(np.ascontiguousarray(A.T), dC, False)
    assert_close(a.grad.cpu().numpy().view(np.uint16), dA_ref, N, what="dA = dC @ B^T")
    assert_close(b.grad.cpu().numpy().view(np.uint16), dB_ref, M, what="dB = A^T @ dC")


def test_autograd_broadcast_gradient(gpu):
    """An upstream gradient that is a broadcast view (stride 0 along rows, as C.sum(0)
    gives) is made dense before the backward GEMMs; dA and dB against the oracle."""
    torch = gpu
    M, N, K = 264, 136, 96
    A, B = W.make_inputs(M, N, K, "normal", 1.0, seed=44)
    v, _ = W.make_inputs(1, 8, N, "normal", 1.0, seed=45)   # a 1 x N weight row
    a = to_dev(A).requires_grad_(True)
    b = to_dev(B).requires_grad_(True)
    log("autograd with a broadcast upstream gradient")
    c = tg.GemmFunction.apply(a, b)
    (c.sum(0).float() * to_dev(v[0]).float()).sum().backward()   # dC = v broadcast over rows
    torch.cuda.synchronize()
    dC = np.repeat(v, M, axis=0)
    dA_ref = oracle.gemm(dC, np.ascontiguousarray(B.T), False)
    dB_ref = oracle.gemm(np.ascontiguousarray(A.T), dC, False)
    assert_close(a.grad.cpu().numpy().view(np.uint16), dA_ref, N, what="dA, broadcast dC")
    assert_close(b.grad.cpu().numpy().view(np.uint16), dB_ref, M, what="dB, broadcast dC")


def test_matmul_views_match_explicit_layouts(gpu):
    torch = gpu
    M, N, K = 264, 136, 128
    A, B = W.make_inputs(M, N, K, "normal", 1.0, seed=43)
    at = to_dev(np.ascontiguousarray(A.T))  # K x M storage
    bt = to_dev(np.ascontiguousarray(B.T))  # N x K storage
    log("matmul on transposed views")
    c_views = tg.matmul(at.t(), bt.t(), relu=True)
    c_ex = tg.gemm_f16_ex(at, bt, trans_a=True, trans_b=True, relu=True)
    torch.cuda.synchronize()
    assert torch.equal(c_views, c_ex)
    assert_close(c_ex.cpu().numpy().view(np.uint16), oracle.gemm(A, B, True), K, what="matmul views")
    with pytest.raises(ValueError):
        tg.matmul(to_dev(A)[:, ::2], to_dev(B)[: K // 2])
