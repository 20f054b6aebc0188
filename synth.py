"""Seeded synthetic inputs for the IQ4_XS x Q8_1 matmul.

This module only draws random numbers and lays them out as bytes or fp32
arrays.  It holds none of the method's arithmetic (no decoding, no
quantization, no products): both the GPU library's tests/benchmark and the
CPU oracle take their inputs from here, and nothing here depends on either.

Weights.  An IQ4_XS super-block is 136 bytes.  Its first two bytes are the
fp16 super-block scale d; the remaining 134 bytes (the 16-bit high-scale
word, the four low-scale bytes and the 128 bytes of 4-bit indices) use
every bit, so drawing them as uniform random bytes is exactly the same as
drawing every 6-bit sub-block scale uniformly from {0..63} and every 4-bit
index uniformly from {0..15}.  d is drawn from U[1e-3, 4e-3] in fp64 and
stored as the nearest fp16 (numpy's round-to-nearest-even cast).

Activations.  fp32 N(0, sigma^2); the "outlier" variant scales round(1% of
K) input channels, chosen once per seed without replacement, by 20 in
every row.

Seeds.  Every array comes from numpy's PCG64 seeded by a SeedSequence of
integers that name the workload, so any process reproduces the same bytes.
"""

from __future__ import annotations

import dataclasses
from typing import Sequence

import numpy as np

QK_K = 256          # elements per IQ4_XS super-block
BLOCK_BYTES = 136   # bytes per IQ4_XS super-block
_ROW_CHUNK = 4096   # rows drawn per generator call (fixed: it is part of the stream)


def _rng(key: Sequence[int]) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def weight_bytes(N: int, K: int) -> int:
    """Size in bytes of an N x K IQ4_XS matrix (K a multiple of 256)."""
    if K % QK_K:
        raise ValueError("K must be a multiple of 256")
    return N * (K // QK_K) * BLOCK_BYTES


def weights(key: Sequence[int], N: int, K: int,
            d_lo: float = 1e-3, d_hi: float = 4e-3) -> np.ndarray:
    """Random IQ4_XS weights as a uint8 array of shape [N, (K/256)*136].

    Row n holds the K/256 super-blocks of output row n, in order.
    """
    if K % QK_K or N < 0:
        raise ValueError("need N >= 0 and K a multiple of 256")
    nb = K // QK_K
    out = np.empty((N, nb, BLOCK_BYTES), dtype=np.uint8)
    rng = _rng(key)
    for r0 in range(0, N, _ROW_CHUNK):
        r1 = min(N, r0 + _ROW_CHUNK)
        out[r0:r1] = rng.integers(0, 256, size=(r1 - r0, nb, BLOCK_BYTES), dtype=np.uint8)
        d = rng.uniform(d_lo, d_hi, size=(r1 - r0, nb)).astype(np.float16)
        out[r0:r1, :, 0:2] = d.view(np.uint8).reshape(r1 - r0, nb, 2)
    return out.reshape(N, nb * BLOCK_BYTES)


BLOCK18_BYTES = 18  # bytes per IQ4_NL / Q4_0 block of 32 weights


def weights18(key: Sequence[int], N: int, K: int,
              d_lo: float = 1e-3, d_hi: float = 4e-3) -> np.ndarray:
    """Random IQ4_NL or Q4_0 weights (both store a block of 32 weights as an
    fp16 d and 16 bytes of 4-bit indices) as uint8 [N, (K/32)*18].  The 16
    index bytes use every bit, so uniform random bytes are exactly uniform
    indices; d is drawn as for IQ4_XS."""
    if K % 32 or N < 0:
        raise ValueError("need N >= 0 and K a multiple of 32")
    nb = K // 32
    out = np.empty((N, nb, BLOCK18_BYTES), dtype=np.uint8)
    rng = _rng(key)
    for r0 in range(0, N, _ROW_CHUNK):
        r1 = min(N, r0 + _ROW_CHUNK)
        out[r0:r1] = rng.integers(0, 256, size=(r1 - r0, nb, BLOCK18_BYTES), dtype=np.uint8)
        d = rng.uniform(d_lo, d_hi, size=(r1 - r0, nb)).astype(np.float16)
        out[r0:r1, :, 0:2] = d.view(np.uint8).reshape(r1 - r0, nb, 2)
    return out.reshape(N, nb * BLOCK18_BYTES)


def activations(key: Sequence[int], M: int, K: int, sigma: float = 1.0,
                outlier_frac: float = 0.0, outlier_scale: float = 20.0) -> np.ndarray:
    """fp32 activations [M, K] ~ N(0, sigma^2), optionally with outlier channels."""
    rng = _rng(key)
    x = rng.standard_normal((M, K), dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    n_out = int(round(outlier_frac * K))
    if n_out:
        cols = rng.choice(K, size=n_out, replace=False)
        x[:, cols] *= np.float32(outlier_scale)
    return x


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: a weight shape, the M values it is run at and
    the activation distribution."""
    cid: int
    name: str
    shapes: tuple            # tuple of (N, K)
    ms: tuple                # M values
    sigma: float = 1.0
    outlier_frac: float = 0.0

    def w(self, N: int, K: int, seed: int = 0) -> np.ndarray:
        return weights((self.cid, N, K, seed), N, K)

    def x(self, M: int, K: int, seed: int = 0, N: int = 0) -> np.ndarray:
        return activations((self.cid, N, K, M, seed), M, K, self.sigma, self.outlier_frac)


# The five workloads of the measurement plan.
SMALL = Workload(1, "single GEMM N=2048 K=2048 M=4", ((2048, 2048),), (4,))
DECODE_ATTN = Workload(2, "attention/GDN input projection N=10240 K=5120, decode M=1..16",
                       ((10240, 5120),), (1, 2, 4, 8, 16), outlier_frac=0.01)
MLP_UP = Workload(3, "MLP gate/up N=17408 K=5120, batched decode M=8..96",
                  ((17408, 5120),), (8, 16, 32, 64, 96))
MLP_DOWN = Workload(4, "MLP down N=5120 K=17408, M=1..96",
                    ((5120, 17408),), (1, 12, 32, 64, 96), sigma=0.5)
PREFILL = Workload(5, "prefill sweep over nine weight shapes, M=64..512",
                   ((5120, 5120), (10240, 5120), (17408, 5120), (5120, 17408), (1024, 5120),
                    (6144, 5120), (5120, 6144), (248320, 5120), (5120, 1024)),
                   (64, 128, 256, 512))

WORKLOADS = (SMALL, DECODE_ATTN, MLP_UP, MLP_DOWN, PREFILL)
