"""GPU checks of the measurement tooling: the MFMA probe and the instrumented build
(libtgemm_stamps.so), which must compute exactly what libtgemm.so computes."""
import numpy as np
import pytest

import oracle
import tgemm_workloads as W
from gpu_util import assert_close, log, torch_cuda

import tiled_dense_gemm_04_amd as tg

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = torch_cuda()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tg.lib()
    tg.stamps_lib()
    return torch


def test_mfma_probe_runs_and_is_deterministic(gpu):
    torch = gpu
    blocks, iters = 16, 64
    outs = []
    for library in (tg.stamps_lib(),) * 3:
        out = torch.full((blocks * tg.PROBE_THREADS,), float("nan"), dtype=torch.float32, device="cuda")
        log(f"probe blocks={blocks} iters={iters}")
        flop = tg.tgemm_mfma_probe(blocks, iters, out, library=library)
        torch.cuda.synchronize()
        assert flop == blocks * 8 * iters * 16 * 16384
        o = out.cpu().numpy()
        assert np.all(np.isfinite(o))
        assert np.count_nonzero(o) > o.size // 2
        outs.append(o)
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


@pytest.mark.parametrize("mode", ["operands", "operands_32x32", "lds_reads"])
def test_mfma_probe_modes_exact_on_ones(gpu, mode):
    """With every operand 1.0 each accumulator element gains k (32 or 16) per round, exactly
    in float32 at these counts, so every thread's sum is 2048 per round in each mode (16
    accumulators x 4 elements x 32, or 8 x 16 x 16); N(0,1) operands give finite,
    repeatable sums."""
    torch = gpu
    blocks, iters = 8, 40
    ones = torch.ones(tg.PROBE_THREADS * 64, dtype=torch.float16, device="cuda")
    out = torch.full((blocks * tg.PROBE_THREADS,), float("nan"), dtype=torch.float32, device="cuda")
    log(f"probe {mode} ones blocks={blocks} iters={iters}")
    flop = tg.tgemm_mfma_probe_ex(mode, blocks, iters, out, operands=ones)
    torch.cuda.synchronize()
    assert flop == blocks * 8 * iters * 16 * 16384
    assert torch.all(out == 2048.0 * iters), out.unique()[:8]
    A, _ = W.make_inputs(tg.PROBE_THREADS, 1, 64, "normal", 1.0, seed=40)
    ops = torch.from_numpy(A).cuda().contiguous()
    got = []
    for _ in range(2):
        out.fill_(float("nan"))
        tg.tgemm_mfma_probe_ex(mode, blocks, iters, out, operands=ops)
        torch.cuda.synchronize()
        o = out.cpu().numpy()
        assert np.all(np.isfinite(o)) and np.count_nonzero(o) > o.size // 2
        got.append(o)
    assert np.array_equal(got[0], got[1])


@pytest.mark.parametrize("cfg_name", ["m256x256x32_s4_w2x4_p4_x1", "p128x128x64_s2_w2x2_p4_x1",
                                      "m256x192x32_s4_w2x4_p4_x1"])
def test_stamps_build_same_result_and_sane_stamps(gpu, cfg_name):
    torch = gpu
    idx = [c["name"] for c in tg.configs()].index(cfg_name)
    desc = tg.tgemm_config_desc(idx)
    M, N, K = 1000, 1032, 520
    A, B = W.make_inputs(M, N, K, "normal", 1.0, seed=71)
    a = torch.from_numpy(A).cuda()
    b = torch.from_numpy(B).cuda()
    c0 = torch.empty((M, N), dtype=torch.float16, device="cuda")
    c1 = torch.empty_like(c0)
    log(f"stamps cfg {cfg_name} {M}x{N}x{K}")
    tg.tgemm_stamps_clear()
    tg.gemm_f16(a, b, c0, relu=True, cfg=idx)
    tg.gemm_f16(a, b, c1, relu=True, cfg=idx, library=tg.stamps_lib())
    torch.cuda.synchronize()
    c0b = c0.cpu().numpy().view(np.uint16)
    assert np.array_equal(c0b, c1.cpu().numpy().view(np.uint16))
    assert_close(c0b, oracle.gemm(A, B, True), K, what=cfg_name)
    nwg = tg.tgemm_num_workgroups(idx, M, N)
    st = tg.tgemm_stamps_read(nwg + 4).astype(np.int64)
    rows, extra = st[:nwg], st[nwg:]
    assert np.all(rows[:, 7] == 1), "every workgroup wrote its row"
    assert np.all(extra == 0), "no row beyond the launch"
    assert np.all(rows[:, 6] == 64 * desc["waves_m"] * desc["waves_n"])
    assert np.all(rows[:, 5] == -(-K // desc["block_k"]))
    assert np.all(rows[:, 0] <= rows[:, 1]) and np.all(rows[:, 1] <= rows[:, 2])
    assert np.all(rows[:, 2] <= rows[:, 3])
    ghz = rows[:, 4] / np.maximum(rows[:, 2] - rows[:, 0], 1) * 0.1
    assert np.all((ghz > 0.3) & (ghz < 3.5)), ghz
