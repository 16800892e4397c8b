"""Every entry point enqueues kernels only (no allocation, no memset, no host sync), so
the calls can be captured in a HIP graph and replayed: a graph holding an NN GEMM, a
transposed-operand GEMM, a split-K GEMM (its workspace allocated before capture) and a
grouped GEMM is replayed several times, with eager work and synchronisations in between,
and every replay must reproduce the eager results bit for bit."""
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

    def work(stream):
        tg.gemm_f16(a1, b1, c1, relu=True, stream=stream)
        tg.gemm_f16_ex(a2t, b2t, c2, True, True, relu=False, stream=stream)
        tg.gemm_f16_ws(a3, b3, c3, relu=True, stream=stream, workspace=ws)
        tg.gemm_f16_grouped([(a, b, c) for (a, b), c in zip(gp, cg)], relu=True, stream=stream)

    log("eager pass")
    work(None)
    torch.cuda.synchronize()
    eager = [c.clone() for c in [c1, c2, c3] + cg]
    assert_close(c1.cpu().numpy().view(np.uint16), oracle.gemm(A1, B1, True), 520, what="nn")
    assert_close(c2.cpu().numpy().view(np.uint16), oracle.gemm(A2, B2, False), 264, what="tt")
    assert_close(c3.cpu().numpy().view(np.uint16), oracle.gemm(A3, B3, True), 16384, what="split-k")

    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    log("capture")
    with torch.cuda.graph(graph, stream=side):
        work(side)
    torch.cuda.synchronize()
    for r in range(4):
        for c in [c1, c2, c3] + cg:
            c.fill_(float("nan"))
        scratch = torch.randn(1 << 20, device="cuda")  # eager work between replays
        scratch.mul_(2.0)
        torch.cuda.synchronize()
        log(f"replay {r}")
        graph.replay()
        torch.cuda.synchronize()
        for i, (c, e) in enumerate(zip([c1, c2, c3] + cg, eager)):
            assert torch.equal(c, e), f"replay {r}: output {i} differs from the eager result"
    assert int(ws[:4096].count_nonzero()) == 0
