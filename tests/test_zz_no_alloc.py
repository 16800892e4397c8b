"""gemm_f16_ws_static -- split-K with the library's static scratch array instead of a
caller workspace -- through the C ABI, against gemm_f16_ws (the entry point it varies) on
the same inputs, and against the oracle. Two split launches in a row, the second over a
smaller output with fewer splits, so the second call runs on scratch the first one left
behind (counters must be back at zero, stale partial tiles must not leak in); then the
first shape again in another layout."""
import ctypes

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


def _both(A, B, ta, tb, relu):
    """Run one logical GEMM through gemm_f16_ws (own workspace) and gemm_f16_ws_static
    (raw C call); returns both outputs' bits."""
    torch = torch_cuda()
    M, K = A.shape
    N = B.shape[1]
    a = to_dev(A.T if ta else A)
    b = to_dev(B.T if tb else B)
    c_ws = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    c_st = torch.full((M, N), float("nan"), dtype=torch.float16, device="cuda")
    tg.gemm_f16_ws(a, b, c_ws, trans_a=ta, trans_b=tb, relu=relu)
    stream = torch.cuda.current_stream().cuda_stream
    rc = tg.lib().gemm_f16_ws_static(int(ta), int(tb), M, N, K, a.data_ptr(), a.stride(0), b.data_ptr(),
                                     b.stride(0), c_st.data_ptr(), c_st.stride(0), int(relu), stream)
    assert rc == tg.TGEMM_OK, tg.tgemm_strerror(rc)
    torch.cuda.synchronize()
    return c_ws.cpu().numpy().view(np.uint16), c_st.cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("shapes", [
    # (M, N, K, trans_a, trans_b, relu): a larger split launch, then a smaller one
    [(512, 512, 16384, True, False, False), (256, 384, 8192, False, False, True),
     (512, 512, 16384, False, True, True)],
])
def test_static_scratch_matches_workspace(shapes):
    for i, (M, N, K, ta, tb, relu) in enumerate(shapes):
        cfg, splits, need = tg.tgemm_split_plan(ta, tb, M, N, K)
        assert splits > 1, "the shape must take the split-K path (it uses the scratch)"
        assert need <= tg.STATIC_SCRATCH_BYTES
        log(f"static scratch call {i}: {M}x{N}x{K} layout ({int(ta)}, {int(tb)}) relu={relu} "
            f"cfg {cfg} splits {splits} ({need} bytes)")
        A, B = W.make_inputs(M, N, K, "normal", 1.0, seed=900 + i)
        c_ws, c_st = _both(A, B, ta, tb, relu)
        assert np.array_equal(c_ws, c_st), "static-scratch result differs from the workspace entry point"
        assert_close(c_st, oracle.gemm(A, B, relu), K, what=f"static scratch call {i}")


def test_static_scratch_unsplit_and_degenerate():
    """Shapes the plan does not split (no scratch touched), K = 0 and empty outputs."""
    torch = torch_cuda()
    A, B = W.make_inputs(520, 392, 264, "normal", 1.0, seed=910)
    c_ws, c_st = _both(A, B, False, False, True)
    assert np.array_equal(c_ws, c_st)
    c = torch.full((7, 9), float("nan"), dtype=torch.float16, device="cuda")
    a = torch.empty((7, 0), dtype=torch.float16, device="cuda")
    b = torch.empty((0, 9), dtype=torch.float16, device="cuda")
    tg.gemm_f16_ws_static(a, b, c, relu=True)
    torch.cuda.synchronize()
    assert (c == 0).all()
    # invalid arguments are rejected before anything is enqueued
    assert tg.gemm_f16_ws_static_raw(0, 0, 8, 8, 8, 256, 7, 256, 8, 256, 8, 0, None) == tg.TGEMM_EINVAL_LD
