"""GPU parity of the fused dequantize-in-LDS path (IQ4XS_PATH_BF16X3).

The path carries W~ and X~ as bf16 hi + lo and sums three products per term
on the matrix cores.  Two references, both from the oracle:
  * the compensated bf16 formulation itself (oracle.gemm_bf16x3, the same
    hi/lo numbers summed exactly): only the fp32 accumulation differs, so the
    per-row ratio max|y - y_ref| / max|y_ref| stays near 1e-6 (a dropped or
    doubled product would be near 1e-3);
  * the integer formulation (oracle.gemm_q8_1), the contract of every path:
    per-row ratio <= 1e-4.
Shapes span several 256 x 256 workgroup tiles with ragged M and N tails.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import iq4_xs_q8_amd as iq
import oracle
import oracle_pins
import synth
from gpu_util import assert_rows_close, dev, poisoned, row_errors

pytestmark = pytest.mark.gpu

P = iq.PATH_BF16X3


def x3_tol(K):
    """Per-row bound against the compensated formulation: only the fp32
    accumulation of 3K products differs, an error that grows like sqrt(K)
    (measured 4.2e-6 at K = 17408); a dropped or doubled product would be
    near 1e-3."""
    return 4e-6 * max(1.0, (K / 2048) ** 0.5)


X3_TOL = x3_tol(2048)
O = None


def setup_module(_):
    global O
    O = oracle.get()
    assert torch.cuda.is_available(), "GPU tests need a GPU"


def _inputs(M, N, K, seed=0, sigma=1.0, outliers=0.0):
    W = synth.weights((950, N, K, seed), N, K)
    X = synth.activations((951, M, K, seed), M, K, sigma=sigma, outlier_frac=outliers)
    return W, X


SHAPES = [(1, 1, 256), (5, 64, 512), (64, 256, 256), (255, 300, 512), (256, 256, 1024),
          (257, 513, 256), (300, 1000, 768), (520, 200, 2048), (512, 2048, 512), (33, 4000, 256)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_matches_both_formulations(M, N, K):
    W, X = _inputs(M, N, K, seed=M + N)
    Xq = O.quantize_q8_1(X)
    Wd, Xd = dev(W), dev(X)
    y = iq.gemm(Wd, Xd, path=P, out=poisoned((M, N))).cpu().numpy()
    assert_rows_close(y, O.gemm_bf16x3(W, Xq, K), tol=x3_tol(K), what=f"BF16X3 vs compensated M={M} N={N} K={K}")
    r = assert_rows_close(y, O.gemm_q8_1(W, Xq, K), what=f"BF16X3 vs integer M={M} N={N} K={K}")
    print(f"[bf16x3-vs-integer-oracle] M={M} N={N} K={K} per-row ratio max {r:.3e}", flush=True)
    # the pre-quantized and caller-workspace entry points: the same launches
    y2 = iq.gemm_q8_1(Wd, dev(Xq), K, path=P, out=poisoned((M, N))).cpu().numpy()
    assert np.array_equal(y, y2), "gemm and gemm_q8_1 differ"
    ws = torch.empty(iq.workspace_bytes(M, N, K, P), dtype=torch.uint8, device="cuda")
    ws.fill_(0x7F)
    y3 = iq.gemm(Wd, Xd, path=P, out=poisoned((M, N)), workspace=ws).cpu().numpy()
    assert np.array_equal(y, y3), "gemm and gemm_ws differ"


def test_outliers_and_small_sigma():
    for sigma, outl in ((0.5, 0.0), (1.0, 0.01), (1e-3, 0.0), (300.0, 0.0)):
        W, X = _inputs(300, 700, 1024, seed=7, sigma=sigma, outliers=outl)
        Xq = O.quantize_q8_1(X)
        y = iq.gemm(dev(W), dev(X), path=P, out=poisoned((300, 700))).cpu().numpy()
        assert_rows_close(y, O.gemm_bf16x3(W, Xq, 1024), tol=X3_TOL, what=f"sigma={sigma}")
        assert_rows_close(y, O.gemm_q8_1(W, Xq, 1024), what=f"sigma={sigma} integer")


def test_zero_scales_and_zero_rows_give_exact_zero():
    rng = np.random.default_rng(43)
    N, K, M = 300, 512, 260
    d_bits, ls, codes = oracle_pins.random_fields(rng, N * K // 256)
    W0, _ = oracle_pins.build_matrix(d_bits, np.full_like(ls, 32), codes, N, K)
    X = rng.standard_normal((M, K)).astype(np.float32)
    y = iq.gemm(dev(W0), dev(X), path=P, out=poisoned((M, N))).cpu().numpy()
    assert np.all(y == 0)
    W, _ = oracle_pins.build_matrix(d_bits, ls, codes, N, K)
    X[3] = 0
    X[259] = 0
    y = iq.gemm(dev(W), dev(X), path=P, out=poisoned((M, N))).cpu().numpy()
    assert np.all(y[3] == 0) and np.all(y[259] == 0)
    assert_rows_close(y, O.gemm_q8_1(W, O.quantize_q8_1(X), K))


def test_exact_when_operands_are_bf16_numbers():
    """Power-of-two d and ls - 32 and power-of-two activation scales: every
    W~ and X~ is a bf16 number (all lo parts zero) and every partial sum is a
    small multiple of one power of two, exact in fp32: the result equals the
    integer formulation bit for bit."""
    rng = np.random.default_rng(47)
    N, K, M = 260, 256, 258      # |partial sums| < 2^24 units of 2^-14: exact in fp32
    nblk = N * K // 256
    d_bits = np.full(nblk, 0x1800, dtype=np.uint16)
    ls = rng.choice([30, 31, 33, 34], size=(nblk, 8)).astype(np.int64)
    codes = rng.integers(0, 16, size=(nblk, 256))
    W, _ = oracle_pins.build_matrix(d_bits, ls, codes, N, K)
    q = rng.integers(-127, 128, size=(M, K)).astype(np.float32)
    q[:, ::32] = 127
    X = q * np.float32(2.0**-5)
    y = iq.gemm(dev(W), dev(X), path=P, out=poisoned((M, N))).cpu().numpy()
    want = O.gemm_q8_1(W, O.quantize_q8_1(X), K)
    assert np.array_equal(y.astype(np.float64), want)


def test_invariants():
    """2X -> 2Y exactly (the splits and the fp32 sums scale by powers of two);
    rows and columns do not depend on the other rows and columns in the call;
    two calls agree bit for bit.  -X -> -Y only to within the accumulation
    error: the matrix core's fp32 sum of bf16 products is not sign-symmetric
    in its last bit (the same holds for the plain bf16 path)."""
    M, N, K = 300, 600, 1024
    W, X = _inputs(M, N, K, seed=11)
    Wd, Xd = dev(W), dev(X)
    y = iq.gemm(Wd, Xd, path=P).cpu()
    assert torch.equal(iq.gemm(Wd, Xd, path=P).cpu(), y)
    assert torch.equal(iq.gemm(Wd, 2 * Xd, path=P).cpu(), 2 * y)
    yn = iq.gemm(Wd, -Xd, path=P).cpu().numpy()
    assert_rows_close(-yn, y.numpy().astype(np.float64), tol=X3_TOL, what="-X")
    for lo, hi in ((0, 1), (17, 40), (255, 300)):
        assert torch.equal(iq.gemm(Wd, Xd[lo:hi].contiguous(), path=P).cpu(), y[lo:hi])
    rb = W.shape[1]
    sub = iq.gemm(dev(np.ascontiguousarray(W[300:600])), Xd, path=P).cpu()
    assert torch.equal(sub, y[:, 300:600])
    assert rb == K // 256 * 136


def test_auto_and_prepared_activations():
    """AUTO may route to this path by the table; the prepared-activation entry
    point never does (it feeds the integer kernels) and refuses it when asked."""
    M, N, K = 256, 512, 512
    W, X = _inputs(M, N, K, seed=5)
    act = iq.prepare_act(dev(X))
    with pytest.raises(RuntimeError):
        iq.gemm_act(dev(W), act, M, K, path=P, out=poisoned((M, N)))
    y = iq.gemm_act(dev(W), act, M, K, out=poisoned((M, N))).cpu().numpy()
    assert_rows_close(y, O.gemm(W, X))


def test_other_formats_refused():
    W = synth.weights18((952, 64, 512), 64, 512)
    X = torch.zeros((4, 512), device="cuda")
    with pytest.raises(RuntimeError):
        iq.gemm_fmt(dev(W), X, iq.FMT_IQ4_NL, path=P)


def _sample_cols(N, n=96, seed=0):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, N - 1], rng.integers(0, N, n)]))


PREFILL = [(N, K, M) for (N, K) in synth.PREFILL.shapes for M in synth.PREFILL.ms]


@pytest.mark.parametrize("N,K,M", PREFILL, ids=[f"{n}x{k}-M{m}" for n, k, m in PREFILL])
def test_prefill_full_size_sampled(N, K, M):
    """Every prefill shape at its real size, checked on sampled columns against
    the compensated formulation and the integer contract."""
    if _cache.get("key") != (N, K):
        _cache.clear()
        torch.cuda.empty_cache()
        _cache["key"] = (N, K)
        _cache["W"] = synth.PREFILL.w(N, K)
        _cache["Wd"] = dev(_cache["W"])
    W, Wd = _cache["W"], _cache["Wd"]
    X = synth.PREFILL.x(M, K, N=N)
    cols = _sample_cols(N, seed=M)
    Xq = O.quantize_q8_1(X)
    y = iq.gemm(Wd, dev(X), path=P, out=poisoned((M, N))).cpu().numpy()
    assert np.all(np.isfinite(y)), "outputs not written"
    assert_rows_close(y[:, cols], O.gemm_bf16x3(W[cols], Xq, K), tol=x3_tol(K), what="vs compensated")
    r = row_errors(y[:, cols], O.gemm_q8_1(W[cols], Xq, K))
    print(f"[bf16x3-vs-integer-oracle] N={N} K={K} M={M} per-row ratio max {r.max():.3e} "
          f"median {np.median(r):.3e}", flush=True)
    assert r.max() <= 1e-4


_cache = {}
