"""The allocation-free entry point iq4xs_gemm_noalloc (scratch in the
library's static per-device array) against the allocating iq4xs_gemm_path,
through the C ABI: bit-identical results (same kernels, same plan) and the
oracle's bound, on two calls in a row where the second is smaller than the
first (the array keeps the first call's contents: partial tiles, activation
planes)."""
import ctypes

import numpy as np
import pytest
import torch

import iq4_xs_q8_amd as iq
import oracle
import synth
from gpu_util import assert_rows_close, dev, poisoned

pytestmark = pytest.mark.gpu

L = None
O = None


def setup_module(_):
    global L, O
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    L = iq.lib
    O = oracle.get()


# (M, N, K, path) pairs: a large call, then a smaller one
PAIRS = [
    # tile kernel, few tiles and long K: partial tiles summed from the scratch
    ((128, 5120, 17408, iq.PATH_MMQ), (40, 1000, 2048, iq.PATH_MMQ)),
    # streaming kernel with tiles shared by two workgroups (Y zeroed by the quantizer)
    ((16, 10240, 5120, iq.PATH_AUTO), (3, 300, 1280, iq.PATH_AUTO)),
    # tile kernel, many tiles (two owners add into Y), then a ragged small one
    ((512, 2048, 1024, iq.PATH_MMQ), (33, 130, 1280, iq.PATH_MMQ)),
    # GEMV
    ((4, 2048, 2048, iq.PATH_GEMV), (1, 257, 1024, iq.PATH_GEMV)),
    # fused dequantize-in-LDS path: compensated activation planes in the scratch
    ((300, 1000, 2048, iq.PATH_BF16X3), (37, 260, 512, iq.PATH_BF16X3)),
]


def _call(fn, W, X, Y, M, N, K, path):
    s = torch.cuda.current_stream().cuda_stream
    rc = fn(W.data_ptr(), X.data_ptr(), Y.data_ptr(), M, N, K, path, s)
    assert rc == iq.OK, (rc, L.iq4xs_last_error())


@pytest.mark.parametrize("pair", PAIRS, ids=[f"{a[0]}x{a[1]}x{a[2]}-then-{b[0]}x{b[1]}x{b[2]}" for a, b in PAIRS])
def test_noalloc_matches_allocating_entry_point(pair):
    for rep in range(2):
        for i, (M, N, K, path) in enumerate(pair):
            W = synth.weights((950, N, K, i), N, K)
            X = synth.activations((951, M, K, i, rep), M, K, outlier_frac=0.01)
            Wd, Xd = dev(W), dev(X)
            print(f"noalloc M={M} N={N} K={K} path={iq.path_name(path)} rep={rep}", flush=True)
            y_na = poisoned((M, N))
            _call(L.iq4xs_gemm_noalloc, Wd, Xd, y_na, M, N, K, path)
            y_ref = poisoned((M, N))
            _call(L.iq4xs_gemm_path, Wd, Xd, y_ref, M, N, K, path)
            torch.cuda.synchronize()
            a, b = y_na.cpu().numpy(), y_ref.cpu().numpy()
            assert np.all(np.isfinite(a)), "outputs not written"
            assert np.array_equal(a, b), f"noalloc differs from iq4xs_gemm_path (M={M} N={N} K={K})"
            cols = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(M).integers(0, N, 96)]))
            Xq = O.quantize_q8_1(X)
            ref = O.gemm_q8_1(W[cols], Xq, K)
            assert_rows_close(a[:, cols], ref, what=f"noalloc M={M} N={N} K={K}")
            if path == iq.PATH_BF16X3:
                assert_rows_close(a[:, cols], O.gemm_bf16x3(W[cols], Xq, K), tol=4e-6,
                                  what=f"noalloc BF16X3 M={M} N={N} K={K}")


def test_noalloc_refuses_oversized_scratch_on_the_device():
    M, N, K = 8192, 64, 17408          # activation planes alone: 160 MB > 128 MiB
    W = torch.zeros((N, K // 256 * 136), dtype=torch.uint8, device="cuda")
    X = torch.zeros((M, K), dtype=torch.float32, device="cuda")
    Y = poisoned((M, N))
    s = torch.cuda.current_stream().cuda_stream
    assert L.iq4xs_gemm_noalloc(W.data_ptr(), X.data_ptr(), Y.data_ptr(), M, N, K, iq.PATH_MMQ, s) == iq.EINVAL
    torch.cuda.synchronize()
    assert torch.isnan(Y).all(), "a refused call must launch nothing"
