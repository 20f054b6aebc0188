"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each pin takes an ``oracle.Oracle`` instance and raises AssertionError on a
mismatch, so the same pins run against the real oracle (test_oracle_pins.py)
and against deliberately broken builds of it (test_oracle_mutants.py).

What pins what:
  * fp16 decode / encode and bf16 rounding: numpy's and torch's own IEEE
    conversions (library routines, exhaustive or near-exhaustive).
  * IQ4_XS decode: a super-block whose bytes and selected weights were worked
    out by hand (tests/golden/iq4xs_handworked.txt), plus blocks built here by
    an *encoder* from chosen fields, so decode is checked against the inverse
    direction rather than against a second decoder.
  * Q8_1: hand-worked blocks (tests/golden/q8_1_handworked.txt) and a check
    against numpy's IEEE fp32 division.
  * GEMM: exact rational arithmetic (fractions.Fraction) on tiny inputs, the
    closed forms ls=32 => Y=0 and single-non-zero activation, and the exact
    invariances Y(-X) = -Y(X), Y(2X) = 2Y(X), Y(2 d_w) = 2Y.
  * bf16 GEMM variant: torch's bf16 cast and an fp64 matmul of the rounded
    operands.
  * IQ4_NL and Q4_0 (18-byte blocks of 32 weights): hand-worked blocks
    (tests/golden/b18_handworked.txt), an encoder, exact rationals, closed
    forms, invariants, and the identity "an IQ4_XS sub-block is an IQ4_NL
    block with d = d*(ls-32)" against the IQ4_XS oracle.
"""

from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# GGUF kvalues_iq4nl codebook (the pages name the table but do not print it).
KV = (-127, -104, -83, -65, -49, -35, -22, -10, 1, 13, 25, 38, 53, 69, 89, 113)


# ------------------------------------------------------------------ encoder
def encode_block(d_bits: int, ls, codes) -> np.ndarray:
    """Build the 136 bytes of one IQ4_XS super-block from its fields.

    d_bits: fp16 bit pattern of d; ls: 8 six-bit scales; codes: 256 indices
    0..15, codes[32b+t] being element t of sub-block b.
    """
    ls = [int(v) for v in ls]
    codes = [int(v) for v in codes]
    assert len(ls) == 8 and len(codes) == 256
    out = np.zeros(136, dtype=np.uint8)
    out[0] = d_bits & 0xFF
    out[1] = (d_bits >> 8) & 0xFF
    sh = 0
    for b in range(8):
        sh |= (ls[b] >> 4) << (2 * b)
        out[4 + b // 2] |= (ls[b] & 15) << (4 * (b % 2))
    out[2] = sh & 0xFF
    out[3] = sh >> 8
    for b in range(8):
        for t in range(16):
            out[8 + 16 * b + t] = codes[32 * b + t] | (codes[32 * b + 16 + t] << 4)
    return out


def block_values(d: float, ls, codes) -> np.ndarray:
    """W~ of a block from its fields (no byte decoding)."""
    return np.array([d * (ls[e // 32] - 32) * KV[codes[e]] for e in range(256)])


def handworked_fields():
    ls = [33, 31, 32, 0, 63, 40, 16, 48]
    codes = []
    for b in range(8):
        lo = [t if b == 0 else (t + b) & 15 for t in range(16)]
        hi = [15 - t if b == 0 else (3 * t + b) & 15 for t in range(16)]
        codes += lo + hi
    return ls, codes


def read_handworked_iq4xs():
    header, weights = None, {}
    with open(os.path.join(GOLDEN, "iq4xs_handworked.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line.startswith("header"):
                header = [int(t, 16) for t in line.split("=")[1].split()]
            elif line.startswith("weight"):
                _, e, v = line.split()
                weights[int(e)] = int(v)
    return header, weights


def read_handworked_q8_1():
    xs, bs = [], []
    with open(os.path.join(GOLDEN, "q8_1_handworked.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            tag, *rest = line.split()
            if tag == "x":
                x = np.zeros(32, dtype=np.float32)
                for item in rest:
                    i, v = item.split(":")
                    x[int(i)] = np.float32(float(v))
                xs.append(x)
            elif tag == "bytes":
                bs.append(np.array([int(t, 16) for t in rest], dtype=np.uint8))
    assert len(xs) == len(bs)
    return np.stack(xs), np.stack(bs)


def random_fields(rng, nblocks):
    d_bits = rng.uniform(1e-3, 4e-3, nblocks).astype(np.float16).view(np.uint16)
    ls = rng.integers(0, 64, (nblocks, 8))
    codes = rng.integers(0, 16, (nblocks, 256))
    return d_bits, ls, codes


def build_matrix(d_bits, ls, codes, N, K):
    """Encode N rows of K/256 blocks; returns (bytes [N, K/256*136], W~ [N,K])."""
    nb = K // 256
    W = np.zeros((N, nb * 136), dtype=np.uint8)
    V = np.zeros((N, K))
    for n in range(N):
        for j in range(nb):
            i = n * nb + j
            W[n, j * 136:(j + 1) * 136] = encode_block(int(d_bits[i]), ls[i], codes[i])
            d = float(np.array(d_bits[i], dtype=np.uint16).view(np.float16))
            V[n, j * 256:(j + 1) * 256] = block_values(d, ls[i], codes[i])
    return W, V


# ------------------------------------------------------------ fp16 / bf16
def pin_half_decode(o):
    h = np.arange(65536, dtype=np.uint16)
    got = o.half_to_double_array(h)
    want = h.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], want[~nan])
    # sign of zero
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def _half_encode_inputs():
    # every fp16 value, every midpoint between neighbours and the fp32
    # neighbours of each midpoint (the cases a wrong tie rule gets wrong),
    # plus random fp32 bit patterns over the whole range.
    h = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = ((h[:-1] + h[1:]) / 2).astype(np.float32)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    rng = np.random.default_rng(7)
    rnd = rng.integers(0, 2**32, 300000, dtype=np.uint64).astype(np.uint32).view(np.float32)
    rnd = rnd[np.isfinite(rnd)]
    big = np.array([65504, 65519.996, 65520, 65536, 1e30, np.inf], dtype=np.float32)
    x = np.concatenate([h.astype(np.float32), mids, up, dn, rnd, big])
    return np.concatenate([x, -x])


def pin_half_encode(o):
    x = _half_encode_inputs()
    got = o.float_to_half_array(x)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, want), np.flatnonzero(got != want)[:10]


def pin_bf16(o):
    import torch
    rng = np.random.default_rng(11)
    # exact fp32 values (the oracle rounds W~ and X~, which are exact in fp32)
    x = rng.standard_normal(200000).astype(np.float32) * np.float32(1e3)
    x = np.concatenate([x, rng.uniform(-1, 1, 50000).astype(np.float32) * np.float32(1e-6)])
    # fp32 values just around bf16 midpoints (tie and near-tie cases)
    base = rng.integers(0, 2**16, 20000, dtype=np.uint32) << 16 | 0x8000
    base = base[(base >> 23 & 0xFF) != 0xFF]
    ties = np.concatenate([base, base + 1, base - 1]).astype(np.uint32).view(np.float32)
    ties = ties[np.isfinite(ties) & (np.abs(ties) > 1e-30)]
    x = np.concatenate([x, ties]).astype(np.float64)
    got = o.double_to_bf16_array(x)
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy()
    assert np.array_equal(got, want.view(np.uint16))


# ------------------------------------------------------------ IQ4_XS decode
def pin_codebook(o):
    assert tuple(o.kvalues()) == KV


def pin_handworked_block(o):
    header, weights = read_handworked_iq4xs()
    ls, codes = handworked_fields()
    blk = encode_block(0x3C00, ls, codes)
    assert list(blk[:8]) == header, "encoder disagrees with the hand-derived header"
    vals = o.dequantize(blk[None, :], 256)[0]
    for e, v in weights.items():
        assert vals[e] == v, (e, vals[e], v)
    assert np.array_equal(vals, block_values(1.0, ls, codes))
    # the super-block scale multiplies everything: d = 0.5 and d = -2
    for bits, d in ((0x3800, 0.5), (0xC000, -2.0)):
        v2 = o.dequantize(encode_block(bits, ls, codes)[None, :], 256)[0]
        assert np.array_equal(v2, d * vals)


def pin_random_blocks(o):
    rng = np.random.default_rng(3)
    d_bits, ls, codes = random_fields(rng, 24)
    W, V = build_matrix(d_bits, ls, codes, 6, 1024)
    assert np.array_equal(o.dequantize(W, 1024), V)
    # each 6-bit scale value and each code in isolation
    for s in range(64):
        v = o.dequantize(encode_block(0x3C00, [s] * 8, [8] * 256)[None, :], 256)[0]
        assert np.all(v == (s - 32) * KV[8]), s


# ------------------------------------------------------------ Q8_1
def pin_q8_1_handworked(o):
    X, want = read_handworked_q8_1()
    got = o.quantize_q8_1(X.reshape(1, -1))
    assert np.array_equal(got.reshape(-1, 36), want), np.argwhere(got.reshape(-1, 36) != want)


def _q8_1_numpy(X):
    """Q8_1 with numpy's IEEE fp32 division and numpy's fp16 cast."""
    M, K = X.shape
    xb = X.reshape(M, K // 32, 32)
    amax = np.max(np.abs(xb), axis=2)
    d = (amax / np.float32(127)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = (xb / d[..., None]).astype(np.float32).astype(np.float64)
    q = np.sign(quot) * np.floor(np.abs(quot) + 0.5)
    q = np.where(d[..., None] == 0, 0, np.clip(q, -127, 127)).astype(np.int64)
    d16 = d.astype(np.float16)
    s16 = (d16.astype(np.float32) * q.sum(axis=2).astype(np.float32)).astype(np.float16)
    out = np.zeros((M, K // 32, 36), dtype=np.uint8)
    out[..., 0:2] = d16.view(np.uint8).reshape(M, K // 32, 2)
    out[..., 2:4] = s16.view(np.uint8).reshape(M, K // 32, 2)
    out[..., 4:] = q.astype(np.int8).view(np.uint8)
    return out.reshape(M, -1)


def pin_q8_1_ieee(o):
    rng = np.random.default_rng(5)
    X = rng.standard_normal((16, 4096)).astype(np.float32)
    X[3] *= np.float32(1e-4)          # fp16-subnormal d
    X[4, :64] = 0                     # all-zero blocks
    X[5, 7] = 1e4                     # large amax
    # values close to .5 multiples of d: x = (k + 1/2 +- tiny) * d
    d = np.float32(0.7) / np.float32(127)
    X[6] = ((rng.integers(-126, 126, 4096) + 0.5) * d).astype(np.float32)
    X[6, ::32] = np.float32(0.7)
    X[7] = np.nextafter(X[6], np.float32(np.inf))
    X[8] = np.nextafter(X[6], np.float32(-np.inf))
    got = o.quantize_q8_1(X)
    want = _q8_1_numpy(X)
    assert np.array_equal(got, want), np.argwhere(got != want)[:5]


def pin_q8_1_division_not_reciprocal(o):
    """Blocks whose activations sit at (k + 1/2) * d, where rounding the IEEE
    quotient x/d and rounding x * fp32(1/d) give different q; the oracle must
    follow the IEEE quotient (numpy's fp32 division)."""
    rng = np.random.default_rng(9)
    found = []
    for it in range(400):
        amax = np.float32(rng.uniform(0.1, 10))
        d = np.float32(amax / np.float32(127))
        k = rng.integers(-126, 126, 31)
        x = ((k + 0.5) * np.float64(d)).astype(np.float32)
        if it % 2:
            x = np.nextafter(x, np.where(rng.random(31) < 0.5, np.inf, -np.inf).astype(np.float32))
        x = np.concatenate([[amax], x]).astype(np.float32)
        q1 = np.floor(np.abs((x / d).astype(np.float32)).astype(np.float64) + 0.5)
        q2 = np.floor(np.abs((x * (np.float32(1) / d)).astype(np.float32)).astype(np.float64) + 0.5)
        if np.any(q1 != q2):
            found.append(x)
        if len(found) >= 32:
            break
    assert len(found) >= 32, "too few blocks with x/d != x*(1/d) after rounding"
    X = np.stack(found).reshape(1, -1)
    assert np.array_equal(o.quantize_q8_1(X), _q8_1_numpy(X))


# ------------------------------------------------------------ GEMM
def _exact_gemm(V, Xq_bytes, M, K):
    """sum_k W~[n,k] * d_x[m,k/32] * q[m,k] in exact rationals."""
    N = V.shape[0]
    xb = Xq_bytes.reshape(M, K // 32, 36)
    d = xb[..., 0:2].copy().view(np.float16).reshape(M, K // 32).astype(np.float64)
    q = xb[..., 4:].view(np.int8).reshape(M, K).astype(np.int64)
    Y = [[Fraction(0)] * N for _ in range(M)]
    A = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        xt = [Fraction(float(d[m, k // 32])) * int(q[m, k]) for k in range(K)]
        for n in range(N):
            terms = [Fraction(float(V[n, k])) * xt[k] for k in range(K)]
            Y[m][n] = sum(terms, Fraction(0))
            A[m][n] = sum((abs(t) for t in terms), Fraction(0))
    return Y, A


def pin_gemm_exact(o):
    rng = np.random.default_rng(13)
    for (M, N, K) in ((3, 4, 256), (2, 3, 512)):
        d_bits, ls, codes = random_fields(rng, N * K // 256)
        W, V = build_matrix(d_bits, ls, codes, N, K)
        X = rng.standard_normal((M, K)).astype(np.float32)
        Xq = o.quantize_q8_1(X)
        assert np.array_equal(Xq, _q8_1_numpy(X))
        Y = o.gemm_q8_1(W, Xq, K)
        exact, absum = _exact_gemm(V, Xq, M, K)
        for m in range(M):
            for n in range(N):
                err = abs(Fraction(float(Y[m, n])) - exact[m][n])
                assert err <= absum[m][n] * Fraction(1, 2**50), (m, n, float(err))


def pin_gemm_closed_forms(o):
    rng = np.random.default_rng(17)
    N, K, M = 5, 512, 3
    d_bits, ls, codes = random_fields(rng, N * K // 256)
    # (i) every ls = 32 -> the output is exactly zero, whatever X and codes are
    W0, _ = build_matrix(d_bits, np.full_like(ls, 32), codes, N, K)
    X = rng.standard_normal((M, K)).astype(np.float32)
    Y0 = o.gemm(W0, X)
    assert np.all(Y0 == 0)
    # (ii) one non-zero activation at column k*: Y[n] = W~[n,k*] * d16 * (+-127)
    W, V = build_matrix(d_bits, ls, codes, N, K)
    for kstar in (0, 15, 16, 31, 32, 100, 255, 256, 300, 511):
        for v in (3.0, -0.37):
            X1 = np.zeros((1, K), dtype=np.float32)
            X1[0, kstar] = v
            d16 = float(np.float16(np.float32(abs(v)) / np.float32(127)))
            want = V[:, kstar] * d16 * (127 if v > 0 else -127)
            assert np.array_equal(o.gemm(W, X1)[0], want), (kstar, v)
    # (iii) a single sub-block with a non-unit scale: only its columns count
    ls1 = np.full_like(ls, 32)
    ls1[1, 3] = 45                       # row 0, block 1, sub-block 3
    W1, V1 = build_matrix(d_bits, ls1, codes, N, K)
    X = rng.standard_normal((2, K)).astype(np.float32)
    Y1 = o.gemm(W1, X)
    assert np.all(Y1[:, 1:] == 0)
    Xq = o.quantize_q8_1(X).reshape(2, K // 32, 36)
    cols = slice(256 + 96, 256 + 128)
    d = Xq[:, 11, 0:2].copy().view(np.float16).astype(np.float64).reshape(2)
    q = Xq[:, 11, 4:].view(np.int8).astype(np.float64)
    want = (V1[0, cols] * q).sum(axis=1) * d
    assert np.array_equal(Y1[:, 0], want)


def pin_gemm_invariants(o):
    rng = np.random.default_rng(19)
    N, K, M = 7, 768, 4
    d_bits, ls, codes = random_fields(rng, N * K // 256)
    W, _ = build_matrix(d_bits, ls, codes, N, K)
    X = rng.standard_normal((M, K)).astype(np.float32)
    Y = o.gemm(W, X)
    assert np.array_equal(o.gemm(W, -X), -Y)
    assert np.array_equal(o.gemm(W, 2 * X), 2 * Y)
    W2, _ = build_matrix((d_bits.astype(np.uint32) + 0x400).astype(np.uint16), ls, codes, N, K)
    assert np.array_equal(o.gemm(W2, X), 2 * Y)
    for m in range(M):
        assert np.array_equal(o.gemm(W, X[m:m + 1])[0], Y[m])
    # output is [M, N]: row m is activation row m
    assert Y.shape == (M, N)


def pin_gemm_bf16(o):
    import torch
    rng = np.random.default_rng(23)
    N, K, M = 6, 512, 3
    d_bits, ls, codes = random_fields(rng, N * K // 256)
    W, V = build_matrix(d_bits, ls, codes, N, K)
    X = rng.standard_normal((M, K)).astype(np.float32)
    Xq = o.quantize_q8_1(X)
    xb = Xq.reshape(M, K // 32, 36)
    d = xb[..., 0:2].copy().view(np.float16).astype(np.float32).reshape(M, K // 32)
    q = xb[..., 4:].view(np.int8).astype(np.float32).reshape(M, K)
    Xt = q * np.repeat(d, 32, axis=1)                      # exact in fp32
    wb = torch.from_numpy(V.astype(np.float32)).to(torch.bfloat16).double()
    xbf = torch.from_numpy(Xt).to(torch.bfloat16).double()
    want = (xbf @ wb.T).numpy()
    got = o.gemm_bf16(W, Xq, K)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-12 * np.abs(want).max())
    # the bf16 weights themselves
    assert np.array_equal(o.dequantize_bf16(W, K),
                          torch.from_numpy(V.astype(np.float32)).to(torch.bfloat16)
                          .view(torch.int16).numpy().view(np.uint16))


def _x_values(Xq, M, K):
    """X~ = d_x * q of Q8_1 bytes, exact in fp64 ([M, K])."""
    xb = Xq.reshape(M, K // 32, 36)
    d = xb[..., 0:2].copy().view(np.float16).astype(np.float64).reshape(M, K // 32)
    q = xb[..., 4:].view(np.int8).astype(np.float64).reshape(M, K)
    return q * np.repeat(d, 32, axis=1)


def pin_gemm_bf16x3_bound(o):
    """Each of W~ and X~ is within 2^-16 (relative) of its hi + lo, and the
    dropped lo*lo product is below 2^-16 |W~ X~|: every term of the
    compensated sum is within 3.02 * 2^-16 of the exact product.  One-hot
    activation rows make each output a single term, so a dropped or doubled
    product (about 2^-9 of the term) shows; dense rows check the sum."""
    rng = np.random.default_rng(29)
    N, K = 9, 512
    d_bits, ls, codes = random_fields(rng, N * K // 256)
    W, V = build_matrix(d_bits, ls, codes, N, K)
    ks = (0, 1, 15, 16, 31, 33, 100, 255, 256, 300, 477, 511)
    X1 = np.zeros((len(ks), K), dtype=np.float32)
    for i, k in enumerate(ks):
        X1[i, k] = rng.standard_normal() * 3
    Xq1 = o.quantize_q8_1(X1)
    xt1 = _x_values(Xq1, len(ks), K)
    got = o.gemm_bf16x3(W, Xq1, K)
    exact = xt1 @ V.T                                 # one non-zero term per output
    terms = np.abs(xt1) @ np.abs(V).T
    assert np.all(np.abs(got - exact) <= 3.02 * 2.0**-16 * terms)
    # not the plain bf16 formulation: somewhere it is closer than bf16 can be
    plain = o.gemm_bf16(W, Xq1, K)
    assert np.max(np.abs(plain - exact) / np.maximum(terms, 1e-300)) > 2.0**-12
    assert np.max(np.abs(got - exact) / np.maximum(terms, 1e-300)) < 2.0**-14
    # dense activations: the sum of the per-term bounds
    M = 3
    X = rng.standard_normal((M, K)).astype(np.float32)
    Xq = o.quantize_q8_1(X)
    exact, absum = _exact_gemm(V, Xq, M, K)
    got = o.gemm_bf16x3(W, Xq, K)
    for m in range(M):
        for n in range(N):
            err = abs(Fraction(float(got[m, n])) - exact[m][n])
            assert err <= absum[m][n] * (Fraction(302, 100) * Fraction(1, 2**16) + Fraction(1, 2**50))


def pin_gemm_bf16x3_exact_when_representable(o):
    """Weights with power-of-two d and ls - 32 and activations whose Q8_1
    scale is a power of two: every W~ and X~ is a bf16 number, every lo part
    is zero, and the compensated sum equals the exact integer-path result."""
    rng = np.random.default_rng(31)
    N, K, M = 4, 512, 3
    nblk = N * K // 256
    d_bits = np.full(nblk, 0x1800, dtype=np.uint16)          # fp16 2^-9
    ls = rng.choice([16, 24, 28, 30, 31, 33, 34, 36, 40, 48, 0], size=(nblk, 8)).astype(np.int64)
    codes = rng.integers(0, 16, size=(nblk, 256))
    W, V = build_matrix(d_bits, ls, codes, N, K)
    q = rng.integers(-127, 128, size=(M, K)).astype(np.float32)
    q[:, ::32] = 127                                          # amax = 127 * 2^-5 in every block
    X = q * np.float32(2.0**-5)
    Xq = o.quantize_q8_1(X)
    assert np.all(Xq.reshape(M, K // 32, 36)[..., 0:2].copy().view(np.float16) == np.float16(2.0**-5))
    want = o.gemm_q8_1(W, Xq, K)
    assert np.array_equal(o.gemm_bf16x3(W, Xq, K), want)
    assert np.array_equal(o.gemm_bf16(W, Xq, K), want)


# ------------------------------------------------- IQ4_NL and Q4_0 blocks
FMT_IQ4_XS, FMT_IQ4_NL, FMT_Q4_0 = 0, 1, 2


def encode_block18(d_bits: int, codes) -> np.ndarray:
    """The 18 bytes of one IQ4_NL / Q4_0 block from its fields: d's fp16 bit
    pattern and 32 indices, codes[t] being element t."""
    codes = [int(v) for v in codes]
    assert len(codes) == 32
    out = np.zeros(18, dtype=np.uint8)
    out[0], out[1] = d_bits & 0xFF, (d_bits >> 8) & 0xFF
    for t in range(16):
        out[2 + t] = codes[t] | (codes[16 + t] << 4)
    return out


def block18_values(fmt: int, d: float, codes) -> np.ndarray:
    """W~ of one block from its fields (no byte decoding)."""
    return np.array([d * (KV[c] if fmt == FMT_IQ4_NL else c - 8) for c in codes], dtype=np.float64)


def build_matrix18(fmt, d_bits, codes, N, K):
    """Encode N rows of K/32 blocks; returns (bytes [N, K/32*18], W~ [N, K])."""
    nb = K // 32
    W = np.zeros((N, nb * 18), dtype=np.uint8)
    V = np.zeros((N, K))
    for n in range(N):
        for j in range(nb):
            i = n * nb + j
            W[n, 18 * j:18 * j + 18] = encode_block18(int(d_bits[i]), codes[i])
            d = float(np.array(d_bits[i], dtype=np.uint16).view(np.float16))
            V[n, 32 * j:32 * j + 32] = block18_values(fmt, d, codes[i])
    return W, V


def random_fields18(rng, nblocks):
    d_bits = rng.uniform(1e-3, 4e-3, nblocks).astype(np.float16).view(np.uint16)
    codes = rng.integers(0, 16, (nblocks, 32))
    return d_bits, codes


def read_handworked_b18():
    blocks, vals = {}, []
    with open(os.path.join(GOLDEN, "b18_handworked.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            if line.startswith("block"):
                name = line.split()[1]
                blocks[name] = np.array([int(t, 16) for t in line.split("=")[1].split()], dtype=np.uint8)
            else:
                tag, name, e, v = line.split()
                vals.append((FMT_IQ4_NL if tag == "nl" else FMT_Q4_0, name, int(e), float(v)))
    return blocks, vals


def pin_b18_handworked(o):
    blocks, vals = read_handworked_b18()
    assert len(vals) >= 28
    assert np.array_equal(blocks["A"], encode_block18(0x3800, list(range(16)) + [15 - t for t in range(16)]))
    for fmt, name, e, v in vals:
        got = o.dequantize_fmt(fmt, blocks[name][None, :], 32)[0]
        assert got[e] == v, (fmt, name, e, got[e], v)


def pin_b18_random_blocks(o):
    rng = np.random.default_rng(29)
    for fmt in (FMT_IQ4_NL, FMT_Q4_0):
        d_bits, codes = random_fields18(rng, 5 * 24)
        W, V = build_matrix18(fmt, d_bits, codes, 5, 768)
        assert np.array_equal(o.dequantize_fmt(fmt, W, 768), V)
        # every index in isolation, at every position
        for c in range(16):
            for t in (0, 7, 15, 16, 24, 31):
                cs = [c if i == t else 8 for i in range(32)]
                v = o.dequantize_fmt(fmt, encode_block18(0x3C00, cs)[None, :], 32)[0]
                want = KV[c] if fmt == FMT_IQ4_NL else c - 8
                assert v[t] == want, (fmt, c, t)
    assert o.row_bytes(FMT_IQ4_NL, 5120) == o.row_bytes(FMT_Q4_0, 5120) == 160 * 18


def pin_b18_gemm_exact(o):
    rng = np.random.default_rng(31)
    for fmt in (FMT_IQ4_NL, FMT_Q4_0):
        for (M, N, K) in ((3, 4, 64), (2, 3, 256)):
            d_bits, codes = random_fields18(rng, N * K // 32)
            W, V = build_matrix18(fmt, d_bits, codes, N, K)
            X = rng.standard_normal((M, K)).astype(np.float32)
            Xq = o.quantize_q8_1(X)
            Y = o.gemm_fmt_q8_1(fmt, W, Xq, K)
            exact, absum = _exact_gemm(V, Xq, M, K)
            for m in range(M):
                for n in range(N):
                    err = abs(Fraction(float(Y[m, n])) - exact[m][n])
                    assert err <= absum[m][n] * Fraction(1, 2**50), (fmt, m, n, float(err))


def pin_b18_closed_forms(o):
    rng = np.random.default_rng(37)
    N, K = 6, 256
    for fmt in (FMT_IQ4_NL, FMT_Q4_0):
        d_bits, codes = random_fields18(rng, N * K // 32)
        W, V = build_matrix18(fmt, d_bits, codes, N, K)
        # one non-zero activation at column k*: Y[n] = W~[n,k*] * d16 * (+-127)
        for kstar in (0, 15, 16, 31, 32, 100, 255):
            for v in (2.5, -0.61):
                X1 = np.zeros((1, K), dtype=np.float32)
                X1[0, kstar] = v
                d16 = float(np.float16(np.float32(abs(v)) / np.float32(127)))
                want = V[:, kstar] * d16 * (127 if v > 0 else -127)
                assert np.array_equal(o.gemm_fmt(fmt, W, X1)[0], want), (fmt, kstar, v)
        # d = 0 everywhere: Y == 0
        W0, _ = build_matrix18(fmt, np.zeros_like(d_bits), codes, N, K)
        assert np.all(o.gemm_fmt(fmt, W0, rng.standard_normal((2, K)).astype(np.float32)) == 0)
    # Q4_0 index 8 is the value 0
    Wz, _ = build_matrix18(FMT_Q4_0, d_bits, np.full_like(codes, 8), N, K)
    assert np.all(o.gemm_fmt(FMT_Q4_0, Wz, rng.standard_normal((3, K)).astype(np.float32)) == 0)


def pin_b18_invariants(o):
    rng = np.random.default_rng(41)
    N, K, M = 5, 512, 3
    for fmt in (FMT_IQ4_NL, FMT_Q4_0):
        d_bits, codes = random_fields18(rng, N * K // 32)
        W, _ = build_matrix18(fmt, d_bits, codes, N, K)
        X = rng.standard_normal((M, K)).astype(np.float32)
        Y = o.gemm_fmt(fmt, W, X)
        assert Y.shape == (M, N)
        assert np.array_equal(o.gemm_fmt(fmt, W, -X), -Y)
        assert np.array_equal(o.gemm_fmt(fmt, W, 2 * X), 2 * Y)
        W2, _ = build_matrix18(fmt, (d_bits.astype(np.uint32) + 0x400).astype(np.uint16), codes, N, K)
        assert np.array_equal(o.gemm_fmt(fmt, W2, X), 2 * Y)
        for m in range(M):
            assert np.array_equal(o.gemm_fmt(fmt, W, X[m:m + 1])[0], Y[m])


def pin_iq4_nl_is_an_iq4_xs_sub_block(o):
    """An IQ4_XS sub-block whose scale d*(ls-32) is exact in fp16 (|ls-32| a
    power of two) is an IQ4_NL block with that d and the same 16 nibble bytes
    (the engine log's batched-kernel section: same block geometry and the
    same kvalues lookup, only the scale is stored differently).  The IQ4_NL
    matrix repacked from IQ4_XS must give the IQ4_XS oracle's output bit for
    bit, tying the new format to the already pinned IQ4_XS decode."""
    rng = np.random.default_rng(43)
    N, K, M = 6, 768, 4
    d_bits, _, codes = random_fields(rng, N * K // 256)
    ls = rng.choice([32 - 32, 32 - 16, 32 - 8, 32 - 4, 32 - 2, 32 - 1, 33, 34, 36, 40, 48], size=(len(d_bits), 8))
    Wxs, Vxs = build_matrix(d_bits, ls, codes, N, K)
    Wnl = np.zeros((N, K // 32 * 18), dtype=np.uint8)
    nb = K // 256
    for n in range(N):
        for j in range(nb):
            i = n * nb + j
            d = np.array(d_bits[i], dtype=np.uint16).view(np.float16).astype(np.float64)
            for b in range(8):
                db = np.float16(d * (ls[i, b] - 32))
                assert float(db) == d * (ls[i, b] - 32)          # exact in fp16
                off = (8 * j + b) * 18
                Wnl[n, off:off + 18] = encode_block18(int(np.array(db).view(np.uint16)),
                                                      codes[i][32 * b:32 * b + 32])
    assert np.array_equal(o.dequantize_fmt(FMT_IQ4_NL, Wnl, K), Vxs)
    X = rng.standard_normal((M, K)).astype(np.float32)
    Xq = o.quantize_q8_1(X)
    assert np.array_equal(o.gemm_fmt_q8_1(FMT_IQ4_NL, Wnl, Xq, K), o.gemm_q8_1(Wxs, Xq, K))
    assert np.array_equal(o.gemm_fmt_q8_1(FMT_IQ4_XS, Wxs, Xq, K), o.gemm_q8_1(Wxs, Xq, K))


B18_PINS = (pin_b18_handworked, pin_b18_random_blocks, pin_b18_gemm_exact, pin_b18_closed_forms,
            pin_b18_invariants, pin_iq4_nl_is_an_iq4_xs_sub_block)

ALL_PINS = (pin_half_decode, pin_half_encode, pin_bf16, pin_codebook, pin_handworked_block,
            pin_random_blocks, pin_q8_1_handworked, pin_q8_1_ieee,
            pin_q8_1_division_not_reciprocal, pin_gemm_exact, pin_gemm_closed_forms,
            pin_gemm_invariants, pin_gemm_bf16, pin_gemm_bf16x3_bound,
            pin_gemm_bf16x3_exact_when_representable) + B18_PINS
