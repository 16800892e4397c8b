"""GPU parity of the grouped GEMM (gemm_f16_grouped): independent GEMMs of any sizes in one
launch (up to 32 per launch), every one against the CPU oracle element by element and bit
for bit against the same config run alone; empty GEMMs, K == 0 and GEMMs only the generic
kernel takes, mixed into one call; the mixture-of-experts workload in full."""
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
    oracle.default()
    return torch


def _stored(A, B, ta, tb):
    return to_dev(A.T if ta else A), to_dev(B.T if tb else B)


@pytest.mark.parametrize("ta,tb", [(0, 0), (0, 1), (1, 0), (1, 1)])
def test_grouped_random_shapes(gpu, ta, tb):
    torch = gpu
    rng = np.random.default_rng(90 + 2 * ta + tb)
    count = 37  # two launches of up to 32
    shapes = [(int(rng.choice([8, 64, 136, 264, 520])), int(rng.choice([8, 128, 136, 256])),
               int(rng.choice([8, 40, 256, 264]))) for _ in range(count)]
    shapes[3] = (0, 64, 64)        # empty
    shapes[5] = (64, 64, 0)        # K == 0: zero fill
    shapes[7] = (65, 72, 33)       # K not a multiple of 8: generic kernel (M too, for A^T)
    ins = [W.make_inputs(M, N, K, "normal", 1.0, seed=2000 + i) for i, (M, N, K) in enumerate(shapes)]
    probs = []
    for (A, B) in ins:
        a, b = _stored(A, B, ta, tb)
        c = torch.full((A.shape[0], B.shape[1]), float("nan"), dtype=torch.float16, device="cuda")
        probs.append((a, b, c))
    log(f"grouped {count} GEMMs layout {ta}{tb}")
    outs = tg.gemm_f16_grouped(probs, bool(ta), bool(tb), relu=True)
    torch.cuda.synchronize()
    for i, ((A, B), c) in enumerate(zip(ins, outs)):
        M, N, K = shapes[i]
        if M == 0:
            continue
        assert_close(c.cpu().numpy().view(np.uint16), oracle.gemm(A, B, True), K, what=f"group {i} {shapes[i]}")


@pytest.mark.parametrize("shapes", [
    [(1000, 1024, 512), (264, 392, 1000), (2048, 256, 128), (8, 8, 64), (520, 136, 264)],  # 119 tiles of 128^2
    [(2048, 2048, 128), (520, 1000, 256)],                                                 # 296: 256^2 tiles
], ids=["tiles128", "tiles256"])
def test_grouped_equals_single_launches_bitwise(gpu, shapes):
    """Each GEMM of a group gives exactly the bits of the same config run on its own. The
    group takes 128 x 128 tiles when all of them fit one round of 256 workgroups, else
    256 x 256."""
    torch = gpu
    ins = [W.make_inputs(M, N, K, "uniform", 1.0, seed=2100 + i) for i, (M, N, K) in enumerate(shapes)]
    probs = [(to_dev(A), to_dev(B)) for A, B in ins]
    t128 = sum(-(-M // 128) * -(-N // 128) for M, N, K in shapes)
    cfg_name = "m128x128x32_s4_w2x4_p4_x1" if t128 <= 256 else "m256x256x32_s4_w2x4_p4_x1"
    idx = [c["name"] for c in tg.configs()].index(cfg_name)
    log(f"grouped vs single launches, config {cfg_name}")
    outs = tg.gemm_f16_grouped(probs, relu=False)
    singles = [tg.gemm_f16(a, b, relu=False, cfg=idx) for a, b in probs]
    torch.cuda.synchronize()
    for i, (c, c1) in enumerate(zip(outs, singles)):
        assert torch.equal(c, c1), f"group member {i} differs from its single launch"
        A, B = ins[i]
        assert_close(c.cpu().numpy().view(np.uint16), oracle.gemm(A, B, False), shapes[i][2], scale=1 / 3,
                     what=f"member {i}")


def test_grouped_moe_workload_every_element(gpu):
    torch = gpu
    w = W.GROUPED_WORKLOADS["moe_8x_16384x2048x4096"]
    ins = w.inputs()
    probs = [(to_dev(A), to_dev(B)) for A, B in ins]
    log(f"grouped workload {w.name}")
    outs = tg.gemm_f16_grouped(probs, relu=w.relu)
    torch.cuda.synchronize()
    for e, ((A, B), c) in enumerate(zip(ins, outs)):
        assert_close(c.cpu().numpy().view(np.uint16), oracle.gemm(A, B, w.relu), w.K, what=f"expert {e}")
