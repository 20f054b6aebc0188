"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: Q8_1 bytes bit-exact; dequantized bf16 weights bit-exact; every GEMM
path within max|y - y_ref| / max|y_ref| <= 1e-4 per output row against the
oracle of its own formulation (integer dot for GEMV and MMQ, bf16 products
for DEQ_BF16); a reference row that is exactly zero must come back exactly
zero.  Every output buffer is poisoned first and checked to be fully written.
"""
import os
import subprocess
import sys

import numpy as np
import pytest
import torch

import iq4_xs_q8_amd as iq
import oracle
import oracle_pins
import synth
from gpu_util import ROW_TOL, assert_rows_close, dev, poisoned, row_errors

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu

O = None


def setup_module(_):
    global O
    O = oracle.get()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _inputs(M, N, K, seed=0, sigma=1.0, outliers=0.0):
    W = synth.weights((900, N, K, seed), N, K)
    X = synth.activations((901, M, K, seed), M, K, sigma=sigma, outlier_frac=outliers)
    return W, X


# ------------------------------------------------------------------ Q8_1
@pytest.mark.parametrize("M,K,sigma,outl", [(1, 256, 1.0, 0.0), (4, 2048, 1.0, 0.0),
                                             (16, 5120, 1.0, 0.01), (7, 17408, 0.5, 0.0),
                                             (3, 96, 1.0, 0.0)])
def test_quantize_bit_exact(M, K, sigma, outl):
    X = synth.activations((902, M, K), M, K, sigma=sigma, outlier_frac=outl)
    want = O.quantize_q8_1(X)
    got = iq.quantize_q8_1(dev(X), out=poisoned(want.shape, torch.uint8)).cpu().numpy()
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]


def test_quantize_edge_cases_bit_exact():
    hand, hand_bytes = oracle_pins.read_handworked_q8_1()
    rng = np.random.default_rng(31)
    rows = [hand.reshape(-1)]
    d = np.float32(0.7) / np.float32(127)
    ties = ((rng.integers(-126, 126, 160) + 0.5) * d).astype(np.float32)
    ties[::32] = np.float32(0.7)
    rows += [ties, np.nextafter(ties, np.float32(np.inf)), np.nextafter(ties, np.float32(-np.inf))]
    rows.append(rng.standard_normal(160).astype(np.float32) * np.float32(1e-4))   # subnormal d
    rows.append(np.zeros(160, np.float32))
    X = np.stack(rows)
    want = O.quantize_q8_1(X)
    assert np.array_equal(want[0].reshape(-1, 36), hand_bytes)
    got = iq.quantize_q8_1(dev(X), out=poisoned(want.shape, torch.uint8)).cpu().numpy()
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]


# ------------------------------------------------------------------ dequant
@pytest.mark.parametrize("N,K", [(1, 256), (37, 1280), (300, 2048)])
def test_dequant_bf16_bit_exact(N, K):
    W = synth.weights((903, N, K), N, K)
    want = O.dequantize_bf16(W, K)
    got = iq.dequantize_bf16(dev(W), K, out=poisoned((N, K), torch.bfloat16))
    got = got.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want)


# ------------------------------------------------------------------ GEMM paths
SMALL_SHAPES = [
    # (M, N, K): several 32x32 tiles plus ragged tails in M and N
    (1, 1, 256), (1, 257, 1024), (2, 100, 512), (3, 300, 1280), (4, 2048, 2048),
    (5, 33, 256), (8, 129, 768), (12, 300, 1280), (16, 300, 2048), (17, 64, 512),
    (32, 96, 1024), (33, 130, 1280), (64, 97, 768), (70, 300, 1280), (96, 200, 2048),
    (128, 160, 512), (200, 75, 256), (300, 129, 512),
]


def _paths_for(M):
    ps = [iq.PATH_MMQ, iq.PATH_DEQ_BF16, iq.PATH_AUTO]
    if M <= 4:
        ps.insert(0, iq.PATH_GEMV)
    return ps


@pytest.mark.parametrize("M,N,K", SMALL_SHAPES)
def test_gemm_paths_match_oracle(M, N, K):
    W, X = _inputs(M, N, K)
    Xq = O.quantize_q8_1(X)
    ref_int = O.gemm_q8_1(W, Xq, K)
    ref_bf16 = O.gemm_bf16(W, Xq, K)
    Wd, Xd = dev(W), dev(X)
    for p in _paths_for(M):
        y = iq.gemm(Wd, Xd, path=p, out=poisoned((M, N))).cpu().numpy()
        ref = ref_bf16 if p == iq.PATH_DEQ_BF16 else ref_int
        assert_rows_close(y, ref, what=f"{iq.path_name(p)} M={M} N={N} K={K}")
        # the same through the pre-quantized entry point (oracle's Q8_1 bytes)
        y2 = iq.gemm_q8_1(Wd, dev(Xq), K, path=p, out=poisoned((M, N))).cpu().numpy()
        assert np.array_equal(y, y2), f"{iq.path_name(p)}: gemm and gemm_q8_1 differ"
        if p != iq.PATH_DEQ_BF16:
            # and through prepared activations (one quantization, one matmul launch)
            act = iq.prepare_act(Xd)
            y3 = iq.gemm_act(Wd, act, M, K, path=p, out=poisoned((M, N))).cpu().numpy()
            assert np.array_equal(y, y3), f"{iq.path_name(p)}: gemm and gemm_act differ"
            # Y_ZEROED: same result on a zeroed Y, without the zeroing kernel
            y5 = iq.gemm_act(Wd, act, M, K, path=p, out=torch.zeros((M, N), device="cuda"),
                             y_zeroed=True).cpu().numpy()
            assert np.array_equal(y, y5), f"{iq.path_name(p)}: gemm_act with Y_ZEROED differs"
        # and with caller-provided scratch (no allocation inside the call)
        ws = torch.empty(iq.workspace_bytes(M, N, K, p), dtype=torch.uint8, device="cuda")
        y4 = iq.gemm(Wd, Xd, path=p, out=poisoned((M, N)), workspace=ws).cpu().numpy()
        assert np.array_equal(y, y4), f"{iq.path_name(p)}: gemm and gemm_ws differ"


@pytest.mark.parametrize("path", [iq.PATH_GEMV, iq.PATH_MMQ])
def test_zero_scales_give_exact_zero(path):
    # all ls = 32: every weight is zero, so every output must be exactly 0
    rng = np.random.default_rng(41)
    N, K, M = 70, 512, 3
    d_bits, ls, codes = oracle_pins.random_fields(rng, N * K // 256)
    W, _ = oracle_pins.build_matrix(d_bits, np.full_like(ls, 32), codes, N, K)
    X = rng.standard_normal((M, K)).astype(np.float32)
    y = iq.gemm(dev(W), dev(X), path=path, out=poisoned((M, N))).cpu().numpy()
    assert np.all(y == 0)


@pytest.mark.parametrize("path", [iq.PATH_GEMV, iq.PATH_MMQ])
def test_zero_activation_row(path):
    W, X = _inputs(4, 200, 1024, seed=3)
    X[2] = 0
    y = iq.gemm(dev(W), dev(X), path=path, out=poisoned((4, 200))).cpu().numpy()
    assert np.all(y[2] == 0)
    assert_rows_close(y, O.gemm(W, X))


@pytest.mark.parametrize("path", [iq.PATH_GEMV, iq.PATH_MMQ])
def test_single_nonzero_activation(path):
    # closed form: y[n] = W~[n, k*] * d16 * 127 for x = v at k* only
    N, K = 64, 512
    W = synth.weights((904, N, K), N, K)
    V = O.dequantize(W, K)
    for kstar in (0, 15, 16, 31, 200, 511):
        X = np.zeros((1, K), np.float32)
        X[0, kstar] = 1.75
        y = iq.gemm(dev(W), dev(X), path=path, out=poisoned((1, N))).cpu().numpy()[0]
        d16 = float(np.float16(np.float32(1.75) / np.float32(127)))
        # the kernel rounds (d_w*(ls-32)*d16) and its product with D in fp32
        assert_rows_close(y[None, :], (V[:, kstar] * d16 * 127)[None, :], tol=1e-6)


def _double_dw(W: np.ndarray, K: int) -> np.ndarray:
    """The same weights with every super-block's fp16 d doubled (exponent + 1;
    the synthetic d never reaches the top exponent)."""
    nb = K // 256
    W2 = W.copy().reshape(W.shape[0], nb, 136)
    d = W2[..., 0:2].copy().view(np.uint16)
    assert np.all((d & 0x7C00) < 0x7800)
    W2[..., 0:2] = (d + np.uint16(0x400)).view(np.uint8)
    return W2.reshape(W.shape)


def _check_invariants(Wd, W2d, Xd, path, what):
    """Bitwise: deterministic, X -> -X gives -y, X -> 2X gives 2y, d_w -> 2 d_w
    gives 2y, and a row does not depend on the other rows' values (same M,
    so the same plan)."""
    y1 = iq.gemm(Wd, Xd, path=path, out=poisoned(Xd.shape[:1] + Wd.shape[:1])).cpu()
    assert torch.isfinite(y1).all(), f"{what}: outputs not written"
    assert torch.equal(iq.gemm(Wd, Xd, path=path).cpu(), y1), f"{what}: two runs differ"
    assert torch.equal(iq.gemm(Wd, -Xd, path=path).cpu(), -y1), f"{what}: y(-X) != -y(X)"
    assert torch.equal(iq.gemm(Wd, 2 * Xd, path=path).cpu(), 2 * y1), f"{what}: y(2X) != 2y(X)"
    assert torch.equal(iq.gemm(W2d, Xd, path=path).cpu(), 2 * y1), f"{what}: y(2 d_w) != 2y"
    m = Xd.shape[0] // 2
    Xo = torch.randn_like(Xd) * 3
    Xo[m] = Xd[m]
    assert torch.equal(iq.gemm(Wd, Xo, path=path).cpu()[m], y1[m]), f"{what}: row {m} depends on other rows"
    return y1


# Every kernel and work split of the integer paths.  The tile-kernel cases
# were chosen with the host plan's rules (grid size, run length, tile shape):
# 64 x 256 tiles up to M = 64, 128 x 128 above, 128 x 256 from M = 128 and
# 256 x 128 from M = 256 (unless only they would need a workspace, with runs
# shorter than a super-block); "two owners": runs longer
# than a tile, shared tiles added into a zeroed Y; "workspace": runs shorter
# than a tile, 2..16 owners per tile summed in run order by the second kernel.
INVARIANT_CASES = [
    ("GEMV", iq.PATH_GEMV, 3, 300, 1536),
    ("streaming M=20", iq.PATH_MMQ, 20, 300, 1536),
    ("streaming M=16, shared tiles", iq.PATH_MMQ, 16, 10240, 5120),
    ("tile 64x256, two owners", iq.PATH_MMQ, 40, 40000, 256),
    ("tile 64x256, workspace (16 owners)", iq.PATH_MMQ, 64, 600, 4096),
    ("tile 64x256, workspace (5 owners)", iq.PATH_MMQ, 64, 17408, 5120),
    ("tile 128x128, one owner", iq.PATH_MMQ, 130, 8320, 1024),
    ("tile 128x128, two owners", iq.PATH_MMQ, 65, 16768, 256),
    ("tile 128x128, workspace (16 owners)", iq.PATH_MMQ, 100, 200, 4096),
    ("tile 128x128, workspace (5 owners)", iq.PATH_MMQ, 96, 5120, 5120),
    ("tile 256x128, workspace (2-3 owners), M=512, paired runs", iq.PATH_MMQ, 512, 10240, 5120),
    # the tiles with four activation subtiles per wavefront; ragged M and N,
    # two owners per shared tile
    ("tile 256x128, two owners, ragged", iq.PATH_MMQ, 300, 65613, 256),
    ("tile 256x128, M=512, paired runs", iq.PATH_MMQ, 512, 65536, 256),
    ("tile 128x256, two owners, ragged", iq.PATH_MMQ, 150, 65613, 256),
    ("tile 256x128, workspace (3-4 owners)", iq.PATH_MMQ, 300, 5120, 5120),
    ("tile 128x256, workspace (8 owners)", iq.PATH_MMQ, 130, 2000, 8192),
]


@pytest.mark.parametrize("what,path,M,N,K", INVARIANT_CASES, ids=[c[0] for c in INVARIANT_CASES])
def test_invariants_bitwise(what, path, M, N, K):
    W, X = _inputs(M, N, K, seed=5)
    Wd, W2d, Xd = dev(W), dev(_double_dw(W, K)), dev(X)
    y = _check_invariants(Wd, W2d, Xd, path, what).numpy()
    cols = _sample_cols(N, n=128, seed=M)
    assert_rows_close(y[:, cols], O.gemm_q8_1(W[cols], O.quantize_q8_1(X), K), what=what)


def test_bf16_path_invariants_within_tolerance():
    # the bf16 MFMA's fp32 accumulation is not sign-symmetric bit for bit:
    # only the tolerance-level invariances hold
    W, X = _inputs(20, 300, 1536, seed=5)
    Wd, Xd = dev(W), dev(X)
    p = iq.PATH_DEQ_BF16
    y1 = iq.gemm(Wd, Xd, path=p).cpu()
    assert torch.equal(iq.gemm(Wd, Xd, path=p).cpu(), y1), "two runs differ"
    ref = y1.double().numpy()
    assert_rows_close(-iq.gemm(Wd, -Xd, path=p).cpu().numpy(), ref, tol=1e-6)
    assert_rows_close(0.5 * iq.gemm(Wd, 2 * Xd, path=p).cpu().numpy(), ref, tol=1e-6)


def test_rows_independent_of_m_streaming_and_gemv():
    """The streaming kernel gives row m the same bits for every M it serves
    (each M band has its own chunk length and register layout, but every
    output sums the same products in the same order), here on the decode
    shape whose runs start at odd super-blocks; so does the GEMV for M <= 4.
    The tile kernel (M > 32) keeps this only within one M: its tile shape and
    stream-K split follow M."""
    N, K = 10240, 5120
    W = synth.weights((905, N, K), N, K)
    X = synth.activations((906, 32, K), 32, K, outlier_frac=0.01)
    Wd, Xd = dev(W), dev(X)
    full = iq.gemm(Wd, Xd, path=iq.PATH_MMQ).cpu()
    for M in (1, 2, 3, 4, 5, 8, 9, 16, 17, 31):
        y = iq.gemm(Wd, Xd[:M].contiguous(), path=iq.PATH_MMQ).cpu()
        assert torch.equal(y, full[:M]), f"streaming kernel: rows of M={M} differ from M=32"
    g4 = iq.gemm(Wd, Xd[:4].contiguous(), path=iq.PATH_GEMV).cpu()
    for M in (1, 2, 3):
        assert torch.equal(iq.gemm(Wd, Xd[:M].contiguous(), path=iq.PATH_GEMV).cpu(), g4[:M]), f"GEMV M={M}"


@pytest.mark.parametrize("M,N,K", [(300, 2800, 512), (97, 8200, 256), (130, 8320, 1024),
                                   (100, 200, 4096), (130, 1000, 2048), (257, 384, 8192), (200, 300, 2816),
                                   (40, 1000, 2048), (64, 600, 4096), (50, 5000, 512), (33, 300, 2816),
                                   (65, 16768, 256), (130, 11392, 768), (700, 520, 1280), (1030, 270, 768),
                                   (97, 40003, 256), (97, 40004, 256), (300, 20480, 768), (512, 4096, 1024),
                                   (512, 2048, 2560)])
def test_tile_kernel_shapes(M, N, K):
    """Shapes the tile kernel takes (64 x 256 tiles for 32 < M <= 64, 128 x 128
    above, 128 x 256 or 256 x 128 from M = 128 or 256, also past M = 512):
    ragged M and N; K of one super-block (runs of more than a
    tile: two owners per shared tile, adding into a zeroed Y; N = 40003 and
    40004 for the zeroing of shared tiles with and without 16-byte rows); few tiles and
    long K (runs shorter than a tile: two to eight workgroups share a tile,
    their partial tiles summed in run order by the second kernel); run bounds
    on and off tile and super-block boundaries; several activation blocks
    whose runs over the same weight columns are paired on one XCD (300 x
    20480 x 768: two 256-row blocks, the second ragged, two-owner tiles;
    512 x 4096 x 1024: four 128-row blocks; 512 x 2048 x 2560: two blocks
    with partial tiles summed); through gemm and gemm_act
    (with and without the Y-zeroed hint), bit-identical."""
    W, X = _inputs(M, N, K, seed=M + N)
    ref = O.gemm_q8_1(W, O.quantize_q8_1(X), K)
    Wd, Xd = dev(W), dev(X)
    y = iq.gemm(Wd, Xd, path=iq.PATH_MMQ, out=poisoned((M, N))).cpu().numpy()
    assert np.all(np.isfinite(y)), "outputs not written"
    assert_rows_close(y, ref, what=f"tile M={M} N={N} K={K}")
    act = iq.prepare_act(Xd)
    y2 = iq.gemm_act(Wd, act, M, K, path=iq.PATH_MMQ, out=poisoned((M, N))).cpu().numpy()
    y3 = iq.gemm_act(Wd, act, M, K, path=iq.PATH_MMQ, out=torch.zeros((M, N), device="cuda"),
                     y_zeroed=True).cpu().numpy()
    assert np.array_equal(y, y2) and np.array_equal(y, y3)
    assert torch.equal(iq.gemm(Wd, Xd, path=iq.PATH_MMQ).cpu(), torch.from_numpy(y)), "two runs differ"


def test_ksplit_kernel_when_the_others_are_switched_off(tmp_path):
    """The K-split kernel of the MMQ path (the fallback for shapes the
    streaming and tile kernels do not take, and for odd K/256 at M <= 32),
    forced for every M by switching the other two off; it runs in a child
    process because the switches are read once per process."""
    shapes = [(8, 300, 1024), (48, 300, 1280), (64, 97, 768), (100, 200, 2048), (20, 64, 8192)]
    inputs = {}
    for i, (M, N, K) in enumerate(shapes):
        W, X = _inputs(M, N, K, seed=40 + i)
        Xo = X.copy()
        Xo[np.arange(M) != M // 2] = synth.activations((41, M, K, i), M, K)[np.arange(M) != M // 2]
        np.save(tmp_path / f"w{i}.npy", W)
        np.save(tmp_path / f"w2{i}.npy", _double_dw(W, K))
        np.save(tmp_path / f"x{i}.npy", X)
        np.save(tmp_path / f"xo{i}.npy", Xo)
        inputs[i] = (W, X)
    # in the child: y(X), y(-X), y(2X), y with every d_w doubled, and y(X')
    # where X' differs from X in every row but M/2
    code = (
        "import sys, numpy as np, torch\n"
        "import iq4_xs_q8_amd as iq\n"
        f"d = {str(tmp_path)!r}\n"
        f"for i in range({len(shapes)}):\n"
        "    W = torch.from_numpy(np.load(f'{d}/w{i}.npy')).cuda()\n"
        "    W2 = torch.from_numpy(np.load(f'{d}/w2{i}.npy')).cuda()\n"
        "    X = torch.from_numpy(np.load(f'{d}/x{i}.npy')).cuda()\n"
        "    Xo = torch.from_numpy(np.load(f'{d}/xo{i}.npy')).cuda()\n"
        "    for tag, w, x in (('y', W, X), ('neg', W, -X), ('dbl', W, 2 * X), ('dw', W2, X), ('oth', W, Xo)):\n"
        "        Y = torch.full((X.shape[0], W.shape[0]), float('nan'), device='cuda')\n"
        "        iq.gemm(w, x, path=iq.PATH_MMQ, out=Y)\n"
        "        np.save(f'{d}/{tag}{i}.npy', Y.cpu().numpy())\n")
    env = dict(os.environ, IQ4XS_MMV="0", IQ4XS_TILE="0",
               PYTHONPATH=os.pathsep.join([ROOT, os.environ.get("PYTHONPATH", "")]))
    subprocess.run([sys.executable, "-c", code], env=env, check=True, timeout=120)
    for i, (M, N, K) in enumerate(shapes):
        W, X = inputs[i]
        y = np.load(tmp_path / f"y{i}.npy")
        what = f"k_mmq M={M} N={N} K={K}"
        assert_rows_close(y, O.gemm_q8_1(W, O.quantize_q8_1(X), K), what=what)
        assert np.array_equal(np.load(tmp_path / f"neg{i}.npy"), -y), f"{what}: y(-X) != -y"
        assert np.array_equal(np.load(tmp_path / f"dbl{i}.npy"), 2 * y), f"{what}: y(2X) != 2y"
        assert np.array_equal(np.load(tmp_path / f"dw{i}.npy"), 2 * y), f"{what}: y(2 d_w) != 2y"
        assert np.array_equal(np.load(tmp_path / f"oth{i}.npy")[M // 2], y[M // 2]), f"{what}: row independence"


def test_negative_control_corrupted_weight_fails():
    # a one-byte change in W must push the affected row outside the bound
    M, N, K = 4, 64, 1024
    W, X = _inputs(M, N, K, seed=7)
    ref = O.gemm(W, X)
    Wbad = W.copy()
    Wbad[10, 1] ^= 0x04                              # row 10, block 0: d scaled by 2 or 1/2
    y = iq.gemm(dev(Wbad), dev(X), path=iq.PATH_MMQ).cpu().numpy()
    with pytest.raises(AssertionError):
        assert_rows_close(y[:, 10:11], ref[:, 10:11])
    # and the poison check itself fires on an untouched buffer
    with pytest.raises(AssertionError):
        assert_rows_close(poisoned((M, N)).cpu().numpy(), ref)


def test_large_m_grid():
    # many 32-row tiles along M and a single column
    W, X = _inputs(1000, 1, 512, seed=9)
    y = iq.gemm(dev(W), dev(X), path=iq.PATH_MMQ, out=poisoned((1000, 1))).cpu().numpy()
    assert_rows_close(y.T, O.gemm(W, X).T)


def test_weights_above_2gib():
    """A weight matrix larger than 2 GiB (N = 2^20 rows, K = 4096): the
    streaming and tile kernels address W with 32-bit offsets and decline it,
    so MMQ runs the K-split kernel (a buffer descriptor per 32-row tile); the
    GEMV addresses rows with 64-bit pointers.  Sampled columns against the
    oracle, the last rows included."""
    M, N, K = 2, 1 << 20, 4096
    W = synth.weights((55, N, K), N, K)
    assert W.nbytes > (2 << 30)
    X = synth.activations((56, M, K), M, K)
    Wd, Xd = dev(W), dev(X)
    cols = np.unique(np.concatenate([_sample_cols(N, n=96, seed=5), np.arange(N - 40, N)]))
    ref = O.gemm_q8_1(W[cols], O.quantize_q8_1(X), K)
    for p in (iq.PATH_MMQ, iq.PATH_GEMV):
        y = iq.gemm(Wd, Xd, path=p, out=poisoned((M, N)))
        torch.cuda.synchronize()
        ys = y[:, torch.from_numpy(cols).cuda()].cpu().numpy()
        assert np.all(np.isfinite(y.cpu().numpy())), f"{iq.path_name(p)}: outputs not written"
        assert_rows_close(ys, ref, what=f"{iq.path_name(p)} N={N} K={K}")
        del y
    del Wd
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ full sizes
def _sample_cols(N, n=192, seed=0):
    rng = np.random.default_rng(seed)
    cols = np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, n)]))
    return cols


FULL = []
for wl in synth.WORKLOADS:
    for (N, K) in wl.shapes:
        for M in wl.ms:
            FULL.append((wl.cid, N, K, M))


@pytest.mark.parametrize("cid,N,K,M", FULL, ids=[f"C{c}-{n}x{k}-M{m}" for c, n, k, m in FULL])
def test_full_size_sampled(cid, N, K, M):
    """The workloads at their real sizes, in the launch configuration the
    benchmark times (AUTO path), checked on sampled output columns.  The
    prefill points also run the bf16 path against its own oracle."""
    wl = {w.cid: w for w in synth.WORKLOADS}[cid]
    W = _weights_cached(wl, N, K)
    X = wl.x(M, K, N=N)
    Wd = _wdev_cached(wl, N, K, W)
    cols = _sample_cols(N, seed=M)
    Xq = O.quantize_q8_1(X)
    ref = O.gemm_q8_1(W[cols], Xq, K)
    y = iq.gemm(Wd, dev(X), out=poisoned((M, N))).cpu().numpy()
    assert np.all(np.isfinite(y)), "outputs not written"
    assert_rows_close(y[:, cols], ref, what=f"AUTO C{cid} M={M} N={N} K={K}")
    if M <= 32:
        # the matmul launch alone (tiles shared by two workgroups at these
        # sizes): bit-identical, with Y zeroed by the library or by the caller
        act = iq.prepare_act(dev(X))
        y2 = iq.gemm_act(Wd, act, M, K, out=poisoned((M, N))).cpu().numpy()
        y3 = iq.gemm_act(Wd, act, M, K, out=torch.zeros((M, N), device="cuda"), y_zeroed=True).cpu().numpy()
        assert np.array_equal(y, y2) and np.array_equal(y, y3), "gemm_act differs from gemm"
    if cid == 5 and M in (64, 512):
        yb = iq.gemm(Wd, dev(X), path=iq.PATH_DEQ_BF16, out=poisoned((M, N))).cpu().numpy()
        assert np.all(np.isfinite(yb))
        assert_rows_close(yb[:, cols], O.gemm_bf16(W[cols], Xq, K), what="DEQ_BF16")
        # the same output against the integer formulation: bf16 keeps 8
        # significant bits of W~ and X~, so the per-row ratio sits near
        # 2-3e-3, far above the 1e-4 of the exact paths
        ratio = row_errors(yb[:, cols], ref)
        print(f"[bf16-vs-integer-oracle] N={N} K={K} M={M} per-row ratio max {ratio.max():.3e} "
              f"median {np.median(ratio):.3e}", flush=True)
        assert 1e-4 < ratio.max() < 2e-2


_cache = {}


def _weights_cached(wl, N, K):
    key = ("w", wl.cid, N, K)
    if key not in _cache:
        _cache.clear()
        torch.cuda.empty_cache()
        _cache[key] = wl.w(N, K)
    return _cache[key]


def _wdev_cached(wl, N, K, W):
    key = ("d", wl.cid, N, K)
    if key not in _cache:
        _cache[key] = dev(W)
    return _cache[key]


# More 32-column tiles than compute units: the streaming kernel's balanced runs
# end inside tiles, and each such tile's two owners add their partial tiles
# into a Y that the quantize kernel of the same call zeroed (0 + a + b ==
# 0 + b + a).  The pre-quantized and prepared-activation entry points and the
# caller-workspace entry point run the same matmul kernel, so all of them must
# agree bit for bit, whatever the workspace held before.
SHARED_SHAPES = [(1, 8224, 512), (2, 10240, 1024), (3, 8224, 1024), (4, 10240, 2048),
                 (7, 8224, 512), (16, 10240, 1024), (32, 8224, 512)]


@pytest.mark.parametrize("M,N,K", SHARED_SHAPES)
def test_shared_tiles_match_oracle(M, N, K):
    W, X = _inputs(M, N, K, seed=5)
    Xq = O.quantize_q8_1(X)
    ref = O.gemm_q8_1(W, Xq, K)
    Wd, Xd = dev(W), dev(X)
    p = iq.PATH_MMQ
    y = iq.gemm(Wd, Xd, path=p, out=poisoned((M, N))).cpu().numpy()
    assert_rows_close(y, ref, what=f"MMQ shared tiles M={M} N={N} K={K}")
    y2 = iq.gemm_q8_1(Wd, dev(Xq), K, path=p, out=poisoned((M, N))).cpu().numpy()
    assert np.array_equal(y, y2), "gemm and gemm_q8_1 differ"
    act = iq.prepare_act(Xd)
    y3 = iq.gemm_act(Wd, act, M, K, path=p, out=poisoned((M, N))).cpu().numpy()
    assert np.array_equal(y, y3), "gemm and gemm_act differ"
    # the workspace may hold anything on entry, also what a call left behind
    ws = torch.empty(iq.workspace_bytes(M, N, K, p), dtype=torch.uint8, device="cuda")
    for fill in (0, 255, None, None):
        if fill is None:
            ws.copy_(torch.randint(0, 256, ws.shape, dtype=torch.uint8).cuda())
        else:
            ws.fill_(fill)
        y4 = iq.gemm(Wd, Xd, path=p, out=poisoned((M, N)), workspace=ws).cpu().numpy()
        assert np.array_equal(y, y4), f"gemm_ws differs (workspace fill {fill})"
        y5 = iq.gemm(Wd, Xd, path=p, out=poisoned((M, N)), workspace=ws).cpu().numpy()
        assert np.array_equal(y, y5), "second call on the same workspace differs"


# One X against several weight matrices (one quantization, one streaming
# launch over the tiles of all of them): ragged sizes, a group with more tiles
# than compute units (runs that cross from one matrix into the next, shared
# tiles), and shapes that fall back to one call per matrix (M > 32, odd K/256).
GROUP_CASES = [(1, (300, 520), 1024), (3, (256, 64, 96), 512), (8, (4100, 2050, 3000, 1000), 512),
               (16, (2048, 2048), 2048), (32, (6200, 2100), 512), (40, (300, 200), 512),
               (4, (257, 100), 1280)]


@pytest.mark.parametrize("M,Ns,K", GROUP_CASES)
def test_gemm_group_matches_oracle(M, Ns, K):
    Ws = [synth.weights((903, N, K, g), N, K) for g, N in enumerate(Ns)]
    X = synth.activations((904, M, K, 0), M, K)
    Xq = O.quantize_q8_1(X)
    Wd = [dev(W) for W in Ws]
    Xd = dev(X)
    outs = iq.gemm_group(Wd, Xd, [poisoned((M, N)) for N in Ns])
    again = iq.gemm_group(Wd, Xd, [poisoned((M, N)) for N in Ns])
    # caller workspace with arbitrary contents: nothing allocated, same result
    ws = torch.randint(0, 256, (iq.group_workspace_bytes(list(Ns), M, K),), dtype=torch.uint8).cuda()
    with_ws = iq.gemm_group(Wd, Xd, [poisoned((M, N)) for N in Ns], workspace=ws)
    for g, (W, N) in enumerate(zip(Ws, Ns)):
        y = outs[g].cpu().numpy()
        assert np.all(np.isfinite(y)), f"matrix {g}: outputs not written"
        assert_rows_close(y, O.gemm_q8_1(W, Xq, K), what=f"group matrix {g} M={M} N={N} K={K}")
        assert np.array_equal(y, again[g].cpu().numpy()), f"matrix {g}: repeated call differs"
        assert np.array_equal(y, with_ws[g].cpu().numpy()), f"matrix {g}: call with a workspace differs"


def test_gemm_group_graph_replays_match_eager():
    """The grouped call recorded in a HIP graph (its scratch is stream-ordered):
    every replay, with new inputs in between, equals the eager call."""
    M, Ns, K = 8, (4100, 2050, 3000, 1000), 512
    Ws = [dev(synth.weights((905, N, K, g), N, K)) for g, N in enumerate(Ns)]
    Xd = dev(synth.activations((906, M, K, 0), M, K))
    outs = [poisoned((M, N)) for N in Ns]
    ws = torch.empty(iq.group_workspace_bytes(list(Ns), M, K), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        iq.gemm_group(Ws, Xd, outs, workspace=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        iq.gemm_group(Ws, Xd, outs, workspace=ws)
    for rep in range(4):
        Xd.copy_(dev(synth.activations((907, M, K, rep), M, K, sigma=1.0 + rep)))
        for o in outs:
            o.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = iq.gemm_group(Ws, Xd)
        for i in range(len(Ns)):
            assert np.array_equal(outs[i].cpu().numpy(), want[i].cpu().numpy()), f"replay {rep} matrix {i}"


def test_two_streams_at_once():
    """Calls in flight on two streams at the same time share no state (scratch
    is per call and stream-ordered): each equals its result run alone."""
    cases = [(16, 10240, 512), (4, 8224, 1024), (64, 2048, 1024), (2, 1000, 2048)]
    data = []
    for i, (M, N, K) in enumerate(cases):
        W, X = _inputs(M, N, K, seed=40 + i)
        data.append((dev(W), dev(X), M, N, K))
    alone = [iq.gemm(W, X).cpu().numpy() for W, X, *_ in data]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [poisoned((M, N)) for _, _, M, N, _ in data]
    torch.cuda.synchronize()
    for rep in range(3):
        for i, (W, X, M, N, K) in enumerate(data):
            with torch.cuda.stream(streams[i % 2]):
                iq.gemm(W, X, out=outs[i])
        torch.cuda.synchronize()
        for i in range(len(data)):
            assert np.array_equal(outs[i].cpu().numpy(), alone[i]), f"case {cases[i]} on stream {i % 2}"


@pytest.mark.parametrize("M,N,K", [(1, 1024, 2048), (3, 520, 1280), (8, 2048, 2048), (40, 640, 4096),
                                   (4, 8224, 1024), (16, 10240, 512)])
def test_graph_replays_match_eager(M, N, K):
    """The caller-workspace entry point recorded in a HIP graph: every replay,
    with eager work and new inputs in between, equals the eager call."""
    W, X = _inputs(M, N, K, seed=3)
    Wd = dev(W)
    Xd = dev(X)
    Y = poisoned((M, N))
    ws = torch.empty(iq.workspace_bytes(M, N, K), dtype=torch.uint8, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        iq.gemm(Wd, Xd, out=Y, workspace=ws)          # warm up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        iq.gemm(Wd, Xd, out=Y, workspace=ws)
    for rep in range(4):
        Xn = synth.activations((902, M, K, rep), M, K, sigma=1.0 + rep, outlier_frac=0.01 * rep)
        Xd.copy_(dev(Xn))
        Y.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = Y.cpu().numpy()
        want = iq.gemm(Wd, Xd).cpu().numpy()          # eager, allocating entry point
        assert np.array_equal(got, want), f"replay {rep} differs from the eager call"
        ref = O.gemm_q8_1(W, O.quantize_q8_1(Xn), K)
        assert_rows_close(got, ref, what=f"graph replay {rep} M={M}")


@pytest.mark.parametrize("M,N,K", [(64, 5120, 1024), (100, 200, 4096), (130, 1000, 2048), (512, 10240, 5120),
                                   (300, 2800, 512), (3, 520, 1280), (8, 2048, 2048)])
def test_gemm_act_caller_workspace_and_graph(M, N, K):
    """Prepared activations with a caller workspace (iq4xs_gemm_act_ws): the
    tile kernel with summed partial tiles (the first shapes), with two-owner
    tiles added into Y (300 x 2800 x 512), the streaming kernel and GEMV.
    Bit-identical to the allocating gemm_act whatever the workspace holds, and
    recorded in a HIP graph: every replay, with new activations, garbage in
    Y and the workspace, and eager work in between, equals the eager call."""
    W, X = _inputs(M, N, K, seed=17)
    Wd, Xd = dev(W), dev(X)
    path = iq.PATH_GEMV if M <= 4 else iq.PATH_MMQ
    act = iq.prepare_act(Xd)
    need = iq.act_workspace_bytes(M, N, K, path)
    if (M, N, K) in ((64, 5120, 1024), (100, 200, 4096), (512, 10240, 5120)):
        assert need > 0, "expected a shape with summed partial tiles"
    ws = torch.full((need,), 0xA5, dtype=torch.uint8, device="cuda")
    want = iq.gemm_act(Wd, act, M, K, path=path, out=poisoned((M, N))).cpu().numpy()
    got = iq.gemm_act(Wd, act, M, K, path=path, out=poisoned((M, N)), workspace=ws).cpu().numpy()
    assert np.array_equal(got, want), "gemm_act with a caller workspace differs"
    assert_rows_close(got, O.gemm_q8_1(W, O.quantize_q8_1(X), K), what=f"gemm_act_ws M={M} N={N} K={K}")
    Y = poisoned((M, N))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        iq.gemm_act(Wd, act, M, K, path=path, out=Y, workspace=ws)      # warm up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        iq.gemm_act(Wd, act, M, K, path=path, out=Y, workspace=ws)
    for rep in range(3):
        Xn = synth.activations((903, M, K, rep), M, K, sigma=1.0 + rep)
        iq.prepare_act(dev(Xn), out=act)
        Y.fill_(float("nan"))
        ws.fill_(0x5A + rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eager = iq.gemm_act(Wd, act, M, K, path=path).cpu().numpy()
        assert np.array_equal(Y.cpu().numpy(), eager), f"replay {rep} differs from the eager call"
    del g


def test_table_for_another_compute_unit_count_is_refused(tmp_path):
    """A dispatch table measured on another number of compute units does not
    drive AUTO on this device (fail-closed: ETABLE); explicit paths still run."""
    t = tmp_path / "t.txt"
    t.write_text("arch gfx950\ncus 7\nband MMQ 1 1000000000 * *\n")
    W, X = _inputs(4, 300, 1024, seed=2)
    Wd, Xd = dev(W), dev(X)
    try:
        iq.load_dispatch_table(str(t))
        with pytest.raises(iq.Iq4xsError) as e:
            iq.gemm(Wd, Xd)
        assert e.value.code == iq.ETABLE and "compute units" in str(e.value)
        y = iq.gemm(Wd, Xd, path=iq.PATH_MMQ, out=poisoned((4, 300))).cpu().numpy()
        assert_rows_close(y, O.gemm(W, X))
    finally:
        iq.load_dispatch_table(None)
    props = torch.cuda.get_device_properties(0)
    assert props.multi_processor_count == 256, "the built-in table was measured on 256 compute units"
    assert_rows_close(iq.gemm(Wd, Xd, out=poisoned((4, 300))).cpu().numpy(), O.gemm(W, X))
