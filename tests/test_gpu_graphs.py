"""Every entry point enqueues kernels only (no allocation, no memset, no host sync), so
the calls can be captured in a HIP graph and replayed: a graph holding an NN GEMM, a
transposed-operand GEMM, a split-K GEMM (its workspace allocated before capture), a
grouped GEMM, the fp8 block quantizer feeding the fp8 block-scaled GEMM (quantizer output
buffers allocated before capture) and the generic fp8 kernel is replayed several times,
with eager work and synchronisations in between, and every replay must reproduce the
eager results bit for bit."""
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
    return torch


def test_graph_replays_match_eager(gpu):
    torch = gpu
    A1, B1 = W.make_inputs(1000, 1032, 520, "normal", 1.0, seed=3001)
    A2, B2 = W.make_inputs(520, 392, 264, "normal", 1.0, seed=3002)
    A3, B3 = W.make_inputs(512, 512, 16384, "normal", 1.0, seed=3003)
    G = [W.make_inputs(m, 256, 512, "normal", 1.0, seed=3010 + i) for i, m in enumerate((264, 136, 512))]
    a1, b1 = to_dev(A1), to_dev(B1)
    a2t, b2t = to_dev(np.ascontiguousarray(A2.T)), to_dev(np.ascontiguousarray(B2.T))
    a3, b3 = to_dev(A3), to_dev(B3)
    gp = [(to_dev(A), to_dev(B)) for A, B in G]
    plan = tg.tgemm_split_plan(False, False, 512, 512, 16384)
    assert plan[1] > 1
    ws = torch.zeros(plan[2], dtype=torch.uint8, device="cuda")
    c1 = torch.empty((1000, 1032), dtype=torch.float16, device="cuda")
    c2 = torch.empty((520, 392), dtype=torch.float16, device="cuda")
    c3 = torch.empty((512, 512), dtype=torch.float16, device="cuda")
    cg = [torch.empty((a.shape[0], 256), dtype=torch.float16, device="cuda") for a, _ in gp]
    # fp8: x quantized per 1 x 128 block, then multiplied with an E4M3 weight; and the
    # generic fp8 kernel (K not a multiple of 16)
    X8, W8, SW8 = W.make_fp8_linear_inputs(300, 392, 1040, seed=3020)
    x8, w8, sw8 = to_dev(X8), to_dev(W8), to_dev(SW8)
    xq = torch.empty((300, 1040), dtype=torch.uint8, device="cuda")
    sx = torch.empty((300, 9), dtype=torch.float32, device="cuda")
    c8 = torch.empty((300, 392), dtype=torch.float16, device="cuda")
    A9, SA9, B9, SB9 = W.make_fp8_inputs(130, 264, 200, seed=3021)
    a9, sa9, b9, sb9 = to_dev(A9), to_dev(SA9), to_dev(B9), to_dev(SB9)
    c9 = torch.empty((130, 264), dtype=torch.float16, device="cuda")
    outs = [c1, c2, c3] + cg + [xq, sx, c8, c9]

    def work(stream):
        tg.gemm_f16(a1, b1, c1, relu=True, stream=stream)
        tg.gemm_f16_ex(a2t, b2t, c2, True, True, relu=False, stream=stream)
        tg.gemm_f16_ws(a3, b3, c3, relu=True, stream=stream, workspace=ws)
        tg.gemm_f16_grouped([(a, b, c) for (a, b), c in zip(gp, cg)], relu=True, stream=stream)
        tg.quant_fp8_block(x8, 1, xq, sx, stream=stream)
        tg.gemm_fp8_block(xq, sx, w8, sw8, c8, relu=True, stream=stream)
        tg.gemm_fp8_block(a9, sa9, b9, sb9, c9, relu=False, stream=stream)

    log("eager pass")
    work(None)
    torch.cuda.synchronize()
    eager = [c.clone() for c in outs]
    assert_close(c1.cpu().numpy().view(np.uint16), oracle.gemm(A1, B1, True), 520, what="nn")
    assert_close(c2.cpu().numpy().view(np.uint16), oracle.gemm(A2, B2, False), 264, what="tt")
    assert_close(c3.cpu().numpy().view(np.uint16), oracle.gemm(A3, B3, True), 16384, what="split-k")
    Q8, S8 = oracle.quant_fp8(X8, 1)
    assert np.array_equal(xq.cpu().numpy(), Q8) and np.array_equal(sx.cpu().numpy(), S8)
    for c, args, relu in ((c8, (Q8, S8, W8, SW8), True), (c9, (A9, SA9, B9, SB9), False)):
        rep_ = oracle.compare_fp8(c.cpu().numpy().view(np.uint16), oracle.gemm_fp8(*args, relu), oracle.fp8_bound(*args))
        assert rep_["fails"] == 0, rep_

    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    log("capture")
    with torch.cuda.graph(graph, stream=side):
        work(side)
    torch.cuda.synchronize()
    for r in range(4):
        for c in outs:
            c.fill_(float("nan") if c.dtype != torch.uint8 else 0)
        scratch = torch.randn(1 << 20, device="cuda")  # eager work between replays
        scratch.mul_(2.0)
        torch.cuda.synchronize()
        log(f"replay {r}")
        graph.replay()
        torch.cuda.synchronize()
        for i, (c, e) in enumerate(zip(outs, eager)):
            assert torch.equal(c, e), f"replay {r}: output {i} differs from the eager result"
    assert int(ws[:4096].count_nonzero()) == 0
