"""GPU parity of the fp8 (E4M3) block-scaled path through the C ABI.

gemm_fp8_block on every fp8 config and on the generic kernel against the CPU oracle,
element by element, within |c - ref| <= 4e-3 |ref| + 2^-8 E (E = sum_kb |sa sb| max|a|
max|b|, the size of each block's largest product: the fp8 matrix instructions sum a
block with less than float32 precision); ragged M, N and k-tails, degenerate sizes,
strided operands, ReLU and run-to-run determinism. quant_fp8_block bit for bit against
the oracle (codes and scales, 1 x 128 and 128 x 128 blocks, vector and element paths).
fp8_block_scaled_linear end to end. The measured workloads in full on sampled entries.
"""
import numpy as np
import pytest

import oracle
import tgemm_workloads as W
from choice_table import smallest_exact_shape
from gpu_util import library_for, log, relu_bits, sample_entries, to_dev, torch_cuda

import tiled_dense_gemm_04_amd as tg

pytestmark = pytest.mark.gpu

BLOCK = 128


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = torch_cuda()
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tg.lib()
    oracle.default()
    return torch


def _gemm(A, SA, B, SB, relu, cfg=None, a_pad=0, b_pad=0, c_pad=0):
    """Run gemm_fp8_block on device copies (optionally inside wider row buffers) and
    return the fp16 output bits."""
    torch = torch_cuda()
    M, K = A.shape
    N = B.shape[0]

    def padded(X, pad):
        if pad == 0:
            return to_dev(X)
        buf = np.zeros((X.shape[0], X.shape[1] + pad), dtype=X.dtype)
        buf[:, :X.shape[1]] = X
        return to_dev(buf)[:, :X.shape[1]]

    a, b = padded(A, a_pad), padded(B, b_pad)
    sa, sb = to_dev(SA), to_dev(SB)
    cbuf = torch.full((M, N + c_pad), float("nan"), dtype=torch.float16, device="cuda")
    c = cbuf[:, :N]
    tg.gemm_fp8_block(a, sa, b, sb, c, relu=relu, cfg=cfg, library=library_for(cfg, fp8=True))
    torch.cuda.synchronize()
    if c_pad:  # padding between rows untouched
        assert torch.isnan(cbuf[:, N:]).all()
    return c.cpu().numpy().view(np.uint16)


def _check(A, SA, B, SB, relu, cfg=None, what="", **pads):
    c = _gemm(A, SA, B, SB, relu, cfg, **pads)
    ref = oracle.gemm_fp8(A, SA, B, SB, relu)
    rep = oracle.compare_fp8(c, ref, oracle.fp8_bound(A, SA, B, SB))
    assert rep["fails"] == 0, f"{what}: {rep}"
    return c, rep


# K spans 1 to 16 blocks of 128, with partial groups of 4 blocks of row scales (6, 7 and 9
# blocks) and a single row with several groups (every other slice of row scales empty).
SHAPES = [(256, 256, 128), (300, 264, 1008), (520, 392, 272), (1, 8, 16), (257, 136, 64),
          (640, 1152, 1040), (33, 520, 2048), (1024, 256, 16), (129, 1000, 400),
          (1, 136, 1040), (96, 264, 704), (200, 136, 848)]
ODD = [(17, 23, 29), (65, 63, 129), (1, 1, 1), (130, 7, 250), (40, 200, 100)]


FP8_TABLE_CONFIGS = 5  # rows of the fp8 config table (tests/test_host_abi.py checks the count)


@pytest.mark.parametrize("cfg", list(range(FP8_TABLE_CONFIGS)) + [tg.FP8_GENERIC])
def test_each_config(cfg):
    shapes = SHAPES + (ODD if cfg == tg.FP8_GENERIC else [])
    worst = 0.0
    for s, (M, N, K) in enumerate(shapes):
        A, SA, B, SB = W.make_fp8_inputs(M, N, K, seed=400 + s)
        for relu in (False, True):
            log(f"fp8 cfg {cfg} {M}x{N}x{K} relu={relu}")
            _, rep = _check(A, SA, B, SB, relu, cfg, what=f"cfg{cfg} {M}x{N}x{K} relu={relu}")
            worst = max(worst, rep["max_ratio"])
    log(f"fp8 cfg {cfg}: worst error / tolerance {worst:.3f}")


def test_default_selection_and_edges():
    rng = np.random.default_rng(4242)
    for t in range(24):
        M = int(rng.choice([1, 15, 16, 17, 127, 128, 129, 255, 256, 257]))
        N = int(rng.choice([8, 16, 120, 128, 136, 248, 256, 264]))
        K = int(rng.choice([16, 32, 112, 128, 144, 240, 256, 272, 1008]))
        A, SA, B, SB = W.make_fp8_inputs(M, N, K, seed=600 + t)
        log(f"fp8 edge {M}x{N}x{K} cfg {tg.tgemm_fp8_select_config(M, N, K)}")
        _check(A, SA, B, SB, bool(t % 2), what=f"edge {M}x{N}x{K}")


def test_relu_and_determinism():
    A, SA, B, SB = W.make_fp8_inputs(520, 392, 1040, seed=701)
    plain = _gemm(A, SA, B, SB, False)
    again = _gemm(A, SA, B, SB, False)
    assert np.array_equal(plain, again), "two identical calls differ"
    r = _gemm(A, SA, B, SB, True)
    assert np.array_equal(r, relu_bits(plain)), "ReLU output is not max(plain, +0) bit for bit"


def test_strided_operands():
    M, N, K = 300, 264, 1008
    A, SA, B, SB = W.make_fp8_inputs(M, N, K, seed=702)
    ref_fast = _gemm(A, SA, B, SB, True)
    # row strides that keep the fast path (multiples of 16), and ones that need the generic kernel
    assert np.array_equal(_gemm(A, SA, B, SB, True, a_pad=32, b_pad=48, c_pad=8), ref_fast)
    log("fp8 strided generic (lda = K + 8)")
    assert tg.tgemm_fp8_select_config(M, N, K, lda=K + 8) == tg.FP8_GENERIC
    c, _ = _check(A, SA, B, SB, True, a_pad=8, what="lda = K + 8")


def test_strides_past_fast_limit():
    """Byte strides above 2^23 (past the fast kernels' 32-bit buffer ranges) are served by
    the generic kernel, against the oracle; the quantizer takes them with 64-bit indexing."""
    torch = torch_cuda()
    M, N, K = 20, 24, 272
    A, SA, B, SB = W.make_fp8_inputs(M, N, K, seed=703)
    big = (1 << 23) + 16
    assert tg.tgemm_fp8_select_config(M, N, K, lda=big, ldb=big) == tg.FP8_GENERIC
    log("fp8 lda = ldb = 2^23 + 16 bytes")
    _check(A, SA, B, SB, True, a_pad=big - K, b_pad=big - K, what="lda = ldb = 2^23 + 16")
    R, Kx = 6, 384
    x = _quant_inputs(R, Kx, 804)
    Qr, Sr = oracle.quant_fp8(x, 1)
    ld = (1 << 22) + 8
    xbuf = torch.zeros(((R - 1) * ld + Kx,), dtype=torch.float16, device="cuda")
    qbuf = torch.zeros(((R - 1) * ld + Kx,), dtype=torch.uint8, device="cuda")
    for i in range(R):
        xbuf[i * ld:i * ld + Kx] = to_dev(x[i])
    xd, qd = xbuf.as_strided((R, Kx), (ld, 1)), qbuf.as_strided((R, Kx), (ld, 1))
    log("quant ldx = ldq = 2^22 + 8")
    q, sc = tg.quant_fp8_block(xd, 1, q=qd)
    torch.cuda.synchronize()
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), Sr.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), Qr)


def test_zero_k_and_empty():
    torch = torch_cuda()
    a = torch.zeros((5, 0), dtype=torch.uint8, device="cuda")
    b = torch.zeros((7, 0), dtype=torch.uint8, device="cuda")
    sa = torch.zeros((5, 0), dtype=torch.float32, device="cuda")
    sb = torch.zeros((1, 0), dtype=torch.float32, device="cuda")
    c = torch.full((5, 7), float("nan"), dtype=torch.float16, device="cuda")
    tg.gemm_fp8_block(a, sa, b, sb, c, relu=True)
    torch.cuda.synchronize()
    assert (c == 0).all()
    e = torch.zeros((0, 7), dtype=torch.float16, device="cuda")
    tg.gemm_fp8_block(torch.zeros((0, 16), dtype=torch.uint8, device="cuda"),
                      torch.zeros((0, 1), dtype=torch.float32, device="cuda"),
                      torch.zeros((7, 16), dtype=torch.uint8, device="cuda"),
                      torch.zeros((1, 1), dtype=torch.float32, device="cuda"), e)
    torch.cuda.synchronize()


# ---------------------------------------------------------------- quantizer
def _quant_inputs(R, K, seed):
    rng = np.random.default_rng(seed)
    x = rng.normal(0.0, 1.0, size=(R, K)) * np.exp2(rng.integers(-8, 8, size=(R, 1)))
    x = x.astype(np.float16)
    x[rng.random((R, K)) < 0.01] = 0
    if R > 2 and K > 0:
        x[1, :min(K, BLOCK)] = 0                      # an all-zero block
        x[2, 0] = np.float16(65504.0)                 # the largest binary16
    return x


@pytest.mark.parametrize("block_rows", [1, 128])
def test_quant_bitexact(block_rows):
    torch = torch_cuda()
    # rows of 32 or more blocks take two blocks per lane group (wrapping across rows,
    # partial last workgroup and partial last block included): 4104, 5000 and 8200
    for s, (R, K) in enumerate([(5, 300), (64, 4096), (129, 1000), (3, 8), (300, 256), (1, 128),
                                (7, 4104), (33, 5000), (2, 8200)]):
        x = _quant_inputs(R, K, 800 + s)
        Qr, Sr = oracle.quant_fp8(x, block_rows)
        for pad in (0, 3):  # pad 3: odd row stride, element loads and stores
            buf = np.zeros((R, K + pad), dtype=np.float16)
            buf[:, :K] = x
            xd = to_dev(buf)[:, :K]
            log(f"quant block_rows={block_rows} {R}x{K} ldx={K + pad}")
            q, sc = tg.quant_fp8_block(xd, block_rows)
            torch.cuda.synchronize()
            assert np.array_equal(sc.cpu().numpy().view(np.uint32), Sr.view(np.uint32)), f"scales {R}x{K}"
            assert np.array_equal(q.cpu().numpy(), Qr), f"codes {R}x{K} block_rows={block_rows}"


def test_quant_every_rounding_tie():
    """A block whose maximum is 448 has scale 1, so x / s = x: rows holding every E4M3
    midpoint (all exact in binary16) and its binary16 neighbours exercise every
    round-to-nearest-even decision of the encoder, subnormals and the top binade included."""
    torch = torch_cuda()
    codes = np.arange(0x7F, dtype=np.uint8)
    v = oracle.e4m3_decode(codes)
    mids = ((v[:-1] + v[1:]) / 2).astype(np.float16)
    assert np.array_equal(mids.astype(np.float64), (v[:-1] + v[1:]) / 2)
    vals = np.concatenate([mids, np.nextafter(mids, np.float16(0)), np.nextafter(mids, np.float16(1000)),
                           v.astype(np.float16)]).astype(np.float16)
    vals = np.concatenate([vals, -vals])
    K = 128
    rows = -(-len(vals) // (K - 1))
    x = np.zeros((rows, K), np.float16)
    x[:, 0] = np.float16(448.0)
    flat = np.zeros(rows * (K - 1), np.float16)
    flat[:len(vals)] = vals
    x[:, 1:] = flat.reshape(rows, K - 1)
    for block_rows in (1, 128):
        Qr, Sr = oracle.quant_fp8(x, block_rows)
        assert np.all(Sr == 1.0)
        q, sc = tg.quant_fp8_block(to_dev(x), block_rows)
        torch.cuda.synchronize()
        assert np.array_equal(sc.cpu().numpy(), Sr)
        assert np.array_equal(q.cpu().numpy(), Qr), f"block_rows={block_rows}"


def test_fp8_linear_end_to_end():
    torch = torch_cuda()
    M, N, K = 257, 384, 1040
    x, Wc, SW = W.make_fp8_linear_inputs(M, N, K, seed=900)
    xq_ref, sx_ref = oracle.quant_fp8(x, 1)
    ref = oracle.gemm_fp8(xq_ref, sx_ref, Wc, SW, relu=False)
    xd, wd, swd = to_dev(x), to_dev(Wc), to_dev(SW)
    xq, sx = tg.quant_fp8_block(xd, 1)
    y = tg.fp8_block_scaled_linear(xd, wd, swd)
    torch.cuda.synchronize()
    assert np.array_equal(xq.cpu().numpy(), xq_ref) and np.array_equal(sx.cpu().numpy(), sx_ref)
    rep = oracle.compare_fp8(y.cpu().numpy().view(np.uint16), ref, oracle.fp8_bound(xq_ref, sx_ref, Wc, SW))
    assert rep["fails"] == 0, rep
    with pytest.raises(ValueError):
        tg.fp8_block_scaled_linear(xd, wd, swd, block=64)


# ---------------------------------------------------------------- default choice
@pytest.mark.parametrize("prefix", ["f256x256", "f128x128", "f256x128"])
def test_default_choice_shapes_sampled(prefix):
    """Each config the selector's table picks, on the smallest timed shape where it is the
    table's choice (the library must pick it by itself), against the oracle on sampled
    rows, columns and random entries."""
    shape = smallest_exact_shape(prefix, [c["name"] for c in tg.fp8_configs()], kind="kFp8")
    if shape is None:
        pytest.skip(f"the selector's table picks no {prefix} config")
    M, N, K, cfg = shape
    assert tg.tgemm_fp8_select_config(M, N, K) == cfg
    A, SA, B, SB = W.make_fp8_inputs(M, N, K, seed=78)
    log(f"fp8 default choice {M}x{N}x{K} cfg {cfg}")
    c = _gemm(A, SA, B, SB, True)
    rows, cols = sample_entries(M, N, np.random.default_rng(M + K), n_rows=3, n_cols=3, n_rand=4096)
    rep = oracle.compare_fp8(c[rows, cols], oracle.gemm_fp8_entries(A, SA, B, SB, rows, cols, True),
                             oracle.fp8_bound_entries(A, SA, B, SB, rows, cols))
    assert rep["fails"] == 0, rep


# ---------------------------------------------------------------- measured workloads
@pytest.mark.parametrize("name", ["fp8_block_4096", "fp8_block_relu_8192"])
def test_workload_sampled(name):
    w = W.FP8_WORKLOADS[name]
    A, SA, B, SB = w.inputs()
    cfg = tg.tgemm_fp8_select_config(w.M, w.N, w.K)
    log(f"fp8 workload {name} cfg {cfg}")
    c = _gemm(A, SA, B, SB, w.relu)
    rng = np.random.default_rng(77)
    rows, cols = sample_entries(w.M, w.N, rng)
    ref = oracle.gemm_fp8_entries(A, SA, B, SB, rows, cols, w.relu)
    E = oracle.fp8_bound_entries(A, SA, B, SB, rows, cols)
    rep = oracle.compare_fp8(c[rows, cols], ref, E)
    log(f"fp8 workload {name}: {rep}")
    assert rep["fails"] == 0, rep
    # rows beyond the sample: finite everywhere (no NaN from stale LDS or missed tiles)
    assert np.isfinite(c.view(np.float16)).all()


def test_workload_linear_sampled():
    torch = torch_cuda()
    w = W.FP8_WORKLOADS["fp8_linear_4096"]
    x, Wc, SW = w.inputs()
    xq_ref, sx_ref = oracle.quant_fp8(x, 1)
    xd = to_dev(x)
    y = tg.fp8_block_scaled_linear(xd, to_dev(Wc), to_dev(SW))
    xq, sx = tg.quant_fp8_block(xd, 1)
    torch.cuda.synchronize()
    assert np.array_equal(xq.cpu().numpy(), xq_ref) and np.array_equal(sx.cpu().numpy(), sx_ref)
    rng = np.random.default_rng(78)
    rows, cols = sample_entries(w.M, w.N, rng)
    ref = oracle.gemm_fp8_entries(xq_ref, sx_ref, Wc, SW, rows, cols, False)
    E = oracle.fp8_bound_entries(xq_ref, sx_ref, Wc, SW, rows, cols)
    rep = oracle.compare_fp8(y.cpu().numpy().view(np.uint16)[rows, cols], ref, E)
    log(f"fp8 linear: {rep}")
    assert rep["fails"] == 0, rep


def test_block_sum_precision_under_cancellation():
    """Products that cancel: every row of A and of B holds pairs (x, -x) against (y, y), so
    each block sums large products to a small exact value and the fp8 matrix instructions'
    deviation (relative to the block's largest product) shows through the fp16 output.
    Checks it against the tolerance's per-block allowance 2^-8 and reports the largest
    deviation seen."""
    rng = np.random.default_rng(950)
    M, N, K = 256, 256, 1024
    KB = K // BLOCK
    big = rng.integers(0x60, 0x78, size=(M, K // 2)).astype(np.uint8)     # |a| in 2^5 .. 2^8
    A = np.empty((M, K), np.uint8)
    A[:, 0::2] = big
    A[:, 1::2] = big | 0x80                                               # a_{2i+1} = -a_{2i}
    small = rng.integers(0x08, 0x30, size=(M, K)).astype(np.uint8) | (rng.integers(0, 2, (M, K)) << 7).astype(np.uint8)
    A[:, 0::16] = small[:, 0::16]                                         # every 8th pair: two small
    A[:, 1::16] = small[:, 1::16]                                         # values, a small exact sum
    B = rng.integers(0x30, 0x58, size=(N, K)).astype(np.uint8)
    B[:, 1::2] = B[:, 0::2]                                               # b_{2i+1} = b_{2i}
    SA = np.ones((M, KB), np.float32)
    SB = np.ones((N // BLOCK, KB), np.float32)
    c = _gemm(A, SA, B, SB, False)
    ref = oracle.gemm_fp8(A, SA, B, SB, relu=False)
    E = oracle.fp8_bound(A, SA, B, SB)
    got = oracle.f16_decode(c)
    dev = np.abs(got - ref) - 2.0 ** -11 * np.abs(ref)                    # beyond fp16 rounding
    worst = float(np.max(dev / E))
    log(f"fp8 block sums under cancellation: largest deviation {worst:.3g} of E (2^{np.log2(max(worst, 1e-30)):.1f}), "
        f"allowance 2^-8")
    rep = oracle.compare_fp8(c, ref, E)
    assert rep["fails"] == 0, rep
