"""GPU parity for the 32-weight formats IQ4_NL and Q4_0 (18-byte blocks),
through the C ABI (iq4xs_gemm_fmt), against the oracle's formulation for the
same format: within max|y - y_ref| / max|y_ref| <= 1e-4 per row, every output
poisoned first and checked written; bitwise invariants on every kernel; and
an identity across formats: IQ4_NL weights repacked from IQ4_XS sub-blocks
whose scale d*(ls-32) is exact in fp16 must give the IQ4_XS result bit for bit
(the kernels then compute the same products and the same fp32 scales)."""
import numpy as np
import pytest
import torch

import iq4_xs_q8_amd as iq
import oracle
import oracle_pins
import synth
from gpu_util import assert_rows_close, dev, poisoned

pytestmark = pytest.mark.gpu

O = None
FMTS = [iq.FMT_IQ4_NL, iq.FMT_Q4_0]
FMT_IDS = ["IQ4_NL", "Q4_0"]


def setup_module(_):
    global O
    O = oracle.get()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _inputs(M, N, K, seed=0, sigma=1.0, outliers=0.0):
    W = synth.weights18((960, N, K, seed), N, K)
    X = synth.activations((961, M, K, seed), M, K, sigma=sigma, outlier_frac=outliers)
    return W, X


def _double_d(W, K):
    W2 = W.copy().reshape(W.shape[0], K // 32, 18)
    d = W2[..., 0:2].copy().view(np.uint16)
    assert np.all((d & 0x7C00) < 0x7800)
    W2[..., 0:2] = (d + np.uint16(0x400)).view(np.uint8)
    return W2.reshape(W.shape)


SHAPES = [
    # (M, N, K): ragged tails; odd K/256 (the streaming kernel takes any K/256
    # for 144-byte units); several tiles; the tile kernel's tile shapes
    (1, 1, 256), (1, 257, 1024), (2, 100, 768), (3, 300, 1280), (4, 2048, 2048),
    (5, 33, 256), (8, 129, 768), (12, 300, 1280), (16, 300, 2048), (17, 64, 512),
    (32, 96, 1024), (33, 130, 1280), (64, 97, 768), (70, 300, 1280), (96, 200, 2048),
    (128, 160, 512), (200, 75, 256), (300, 129, 512),
]


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_format_paths_match_oracle(fmt, M, N, K):
    W, X = _inputs(M, N, K, seed=M)
    ref = O.gemm_fmt_q8_1(fmt, W, O.quantize_q8_1(X), K)
    Wd, Xd = dev(W), dev(X)
    paths = [iq.PATH_MMQ, iq.PATH_AUTO] + ([iq.PATH_GEMV] if M <= 4 else [])
    for p in paths:
        what = f"{FMT_IDS[fmt - 1]} {iq.path_name(p)} M={M} N={N} K={K}"
        y = iq.gemm_fmt(Wd, Xd, fmt, path=p, out=poisoned((M, N))).cpu().numpy()
        assert_rows_close(y, ref, what=what)
        ws = torch.randint(0, 256, (iq.fmt_workspace_bytes(fmt, M, N, K, p),), dtype=torch.uint8).cuda()
        y2 = iq.gemm_fmt(Wd, Xd, fmt, path=p, out=poisoned((M, N)), workspace=ws).cpu().numpy()
        assert np.array_equal(y, y2), f"{what}: caller workspace differs"


# the tile kernel's work splits (see test_gpu_parity.INVARIANT_CASES) and the
# streaming kernel with shared tiles and runs starting at odd super-blocks
SPLIT_CASES = [
    ("GEMV", iq.PATH_GEMV, 3, 300, 1536),
    ("streaming", iq.PATH_MMQ, 20, 300, 1536),
    ("streaming, shared tiles, odd K/256", iq.PATH_MMQ, 16, 10240, 4864),
    ("tile 64x256, two owners", iq.PATH_MMQ, 40, 40000, 256),
    ("tile 64x256, workspace", iq.PATH_MMQ, 64, 600, 4096),
    ("tile 128x128, two owners", iq.PATH_MMQ, 65, 16768, 256),
    ("tile 128x128, workspace", iq.PATH_MMQ, 100, 200, 4096),
    ("tile 128x128, one owner", iq.PATH_MMQ, 130, 8320, 1024),
]


@pytest.mark.parametrize("fmt", FMTS, ids=FMT_IDS)
@pytest.mark.parametrize("what,path,M,N,K", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_format_invariants_bitwise(fmt, what, path, M, N, K):
    W, X = _inputs(M, N, K, seed=7)
    Wd, W2d, Xd = dev(W), dev(_double_d(W, K)), dev(X)
    g = lambda w, x: iq.gemm_fmt(w, x, fmt, path=path).cpu()  # noqa: E731
    y = iq.gemm_fmt(Wd, Xd, fmt, path=path, out=poisoned((M, N))).cpu()
    assert torch.isfinite(y).all(), f"{what}: outputs not written"
    assert torch.equal(g(Wd, Xd), y), f"{what}: two runs differ"
    assert torch.equal(g(Wd, -Xd), -y), f"{what}: y(-X) != -y"
    assert torch.equal(g(Wd, 2 * Xd), 2 * y), f"{what}: y(2X) != 2y"
    assert torch.equal(g(W2d, Xd), 2 * y), f"{what}: y(2 d) != 2y"
    m = M // 2
    Xo = torch.randn_like(Xd)
    Xo[m] = Xd[m]
    assert torch.equal(g(Wd, Xo)[m], y[m]), f"{what}: row {m} depends on the other rows"
    cols = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(M).integers(0, N, 128)]))
    ref = O.gemm_fmt_q8_1(fmt, W[cols], O.quantize_q8_1(X), K)
    assert_rows_close(y.numpy()[:, cols], ref, what=what)


def _repack_xs_as_nl(M, N, K, seed):
    """IQ4_XS weights whose sub-block scales d*(ls-32) are exact in fp16
    (|ls-32| a power of two), and the same weights as IQ4_NL blocks."""
    rng = np.random.default_rng(seed)
    nb = K // 256
    Wxs = synth.weights((962, N, K, seed), N, K).reshape(N, nb, 136)
    ls = rng.choice([0, 16, 24, 28, 30, 31, 33, 34, 36, 40, 48], size=(N, nb, 8))
    sh = np.zeros((N, nb), dtype=np.uint32)
    Wxs[:, :, 4:8] = 0
    for b in range(8):
        sh |= ((ls[:, :, b] >> 4) & 3).astype(np.uint32) << (2 * b)
        Wxs[:, :, 4 + b // 2] |= ((ls[:, :, b] & 15) << (4 * (b % 2))).astype(np.uint8)
    Wxs[:, :, 2] = (sh & 0xFF).astype(np.uint8)
    Wxs[:, :, 3] = (sh >> 8).astype(np.uint8)
    d = Wxs[:, :, 0:2].copy().view(np.float16).astype(np.float64)[..., 0]
    Wnl = np.zeros((N, nb, 8, 18), dtype=np.uint8)
    for b in range(8):
        db = (d * (ls[:, :, b] - 32)).astype(np.float16)
        assert np.array_equal(db.astype(np.float64), d * (ls[:, :, b] - 32))
        Wnl[:, :, b, 0:2] = db.view(np.uint8).reshape(N, nb, 2)
        Wnl[:, :, b, 2:18] = Wxs[:, :, 8 + 16 * b:8 + 16 * b + 16]
    X = synth.activations((963, M, K, seed), M, K)
    return Wxs.reshape(N, nb * 136), Wnl.reshape(N, nb * 144), X


@pytest.mark.parametrize("M,N,K,path", [(2, 300, 1024, iq.PATH_GEMV), (16, 10240, 1024, iq.PATH_MMQ),
                                        (96, 700, 2048, iq.PATH_MMQ), (512, 2048, 512, iq.PATH_MMQ)])
def test_iq4_nl_repacked_from_iq4_xs_is_bit_identical(M, N, K, path):
    Wxs, Wnl, X = _repack_xs_as_nl(M, N, K, seed=M)
    Xq = O.quantize_q8_1(X)
    assert np.array_equal(O.gemm_fmt_q8_1(iq.FMT_IQ4_NL, Wnl, Xq, K), O.gemm_q8_1(Wxs, Xq, K))
    Xd = dev(X)
    y_xs = iq.gemm_fmt(dev(Wxs), Xd, iq.FMT_IQ4_XS, path=path, out=poisoned((M, N))).cpu().numpy()
    y_nl = iq.gemm_fmt(dev(Wnl), Xd, iq.FMT_IQ4_NL, path=path, out=poisoned((M, N))).cpu().numpy()
    assert np.array_equal(y_xs, iq.gemm(dev(Wxs), Xd, path=path).cpu().numpy()), "IQ4_XS via gemm_fmt != gemm"
    assert np.array_equal(y_nl, y_xs), "IQ4_NL repacked from IQ4_XS differs from IQ4_XS"


FULL = [(iq.FMT_IQ4_NL, 1, 10240, 5120), (iq.FMT_Q4_0, 16, 10240, 5120), (iq.FMT_IQ4_NL, 64, 17408, 5120),
        (iq.FMT_Q4_0, 12, 5120, 17408), (iq.FMT_Q4_0, 96, 5120, 17408), (iq.FMT_IQ4_NL, 512, 248320, 5120)]


@pytest.mark.parametrize("fmt,M,N,K", FULL, ids=[f"{FMT_IDS[f - 1]}-{m}x{n}x{k}" for f, m, n, k in FULL])
def test_format_full_size_sampled(fmt, M, N, K):
    """The workloads' shapes in these formats (AUTO path), sampled columns."""
    W = synth.weights18((964, N, K), N, K)
    X = synth.activations((965, M, K), M, K, outlier_frac=0.01)
    cols = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(M).integers(0, N, 160)]))
    ref = O.gemm_fmt_q8_1(fmt, W[cols], O.quantize_q8_1(X), K)
    Wd = dev(W)
    y = iq.gemm_fmt(Wd, dev(X), fmt, out=poisoned((M, N))).cpu().numpy()
    assert np.all(np.isfinite(y)), "outputs not written"
    assert_rows_close(y[:, cols], ref, what=f"{FMT_IDS[fmt - 1]} M={M} N={N} K={K}")
    del Wd
    torch.cuda.empty_cache()


def test_format_closed_forms():
    """Q4_0 with every index 8 is the zero matrix; a single non-zero
    activation picks one column of W~ (scaled by d_x * 127)."""
    N, K = 96, 512
    rng = np.random.default_rng(3)
    d_bits, codes = oracle_pins.random_fields18(rng, N * K // 32)
    W, V = oracle_pins.build_matrix18(iq.FMT_Q4_0, d_bits, np.full_like(codes, 8), N, K)
    X = rng.standard_normal((5, K)).astype(np.float32)
    for p in (iq.PATH_GEMV if X.shape[0] <= 4 else iq.PATH_MMQ, iq.PATH_AUTO):
        assert np.all(iq.gemm_fmt(dev(W), dev(X), iq.FMT_Q4_0, path=p).cpu().numpy() == 0)
    for fmt in FMTS:
        W, V = oracle_pins.build_matrix18(fmt, d_bits, codes, N, K)
        for kstar in (0, 17, 31, 300):
            X1 = np.zeros((1, K), np.float32)
            X1[0, kstar] = -1.25
            y = iq.gemm_fmt(dev(W), dev(X1), fmt, path=iq.PATH_GEMV).cpu().numpy()[0]
            d16 = float(np.float16(np.float32(1.25) / np.float32(127)))
            assert_rows_close(y[None, :], (V[:, kstar] * d16 * -127)[None, :], tol=1e-6)
