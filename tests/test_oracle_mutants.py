"""Negative controls for the oracle's pins.

Each mutant is a copy of oracle.c with one plausible mistake planted in it
(a swapped nibble, a wrong bias, a dropped term, a transposed operand, a wrong
rounding rule ...).  The copy is compiled on the CPU and every mutant must
fail at least one pin; the unmodified source must pass them all.  This shows
the pins would catch such a mistake in the oracle itself.
"""
import pytest

import oracle
import oracle_pins

MUTANTS = {
    "nibble order swapped":
        ("return t < 16 ? (byte & 15) : (byte >> 4);",
         "return t < 16 ? (byte >> 4) : (byte & 15);"),
    "scale bias 31": ("return d * (double)(ls - 32);", "return d * (double)(ls - 31);"),
    "scales_l interleaved": ("int lo4 = (blk[4 + b / 2] >> (4 * (b % 2))) & 15;",
                             "int lo4 = (blk[4 + b % 4] >> (4 * (b / 4))) & 15;"),
    "scales_h reversed": ("int hi2 = (scales_h >> (2 * b)) & 3;",
                          "int hi2 = (scales_h >> (2 * (7 - b))) & 3;"),
    "high scale bits shifted by 3": ("int ls = lo4 | (hi2 << 4);", "int ls = lo4 | (hi2 << 3);"),
    "index bytes start at 4": ("uint8_t byte = blk[8 + 16 * b + (t % 16)];",
                               "uint8_t byte = blk[4 + 16 * b + (t % 16)];"),
    "codebook typo": ("-127, -104, -83, -65,", "-127, -104, -82, -65,"),
    "q8 scale amax/128": ("float d = amax / 127.0f;", "float d = amax / 128.0f;"),
    "q8 ties to even": ("q = (int)roundf(quot);", "q = (int)rintf(quot);"),
    "q8 reciprocal multiply": ("float quot = x[i] / d;", "float quot = x[i] * (1.0f / d);"),
    "q8 sum uses fp32 d": ("uint16_t s16 = oracle_float_to_half(dst * (float)sum);",
                           "uint16_t s16 = oracle_float_to_half(d * (float)sum);"),
    "q8 fields swapped": ("o[0] = (uint8_t)(d16 & 0xFF);\n            o[1] = (uint8_t)(d16 >> 8);",
                          "o[2] = (uint8_t)(d16 & 0xFF);\n            o[3] = (uint8_t)(d16 >> 8);"
                          "\n            o[0] = 0; o[1] = 0;"),
    "gemm wrong sub-block scale": ("double sw = sb_scale(blk, (int)(b % 8));",
                                   "double sw = sb_scale(blk, (int)((b + 1) % 8));"),
    "gemm dropped last sub-block": ("for (int64_t b = 0; b < nsub; b++) {\n                const uint8_t *blk",
                                    "for (int64_t b = 0; b < nsub - 1; b++) {\n                const uint8_t *blk"),
    "gemm unsigned activations": ("(int64_t)(int8_t)xb[4 + t];", "(int64_t)(uint8_t)xb[4 + t];"),
    "gemm activation/weight element mismatch": ("(int64_t)(int8_t)xb[4 + t];",
                                                "(int64_t)(int8_t)xb[4 + (t + 16) % 32];"),
    "gemm output transposed": ("            Y[m * N + n] = acc;\n        }\n}\n\n/* Dequantize-to-bf16",
                               "            Y[n * M + m] = acc;\n        }\n}\n\n/* Dequantize-to-bf16"),
    "gemm activation scale from block 0": ("const uint8_t *xb = Xq + (m * nsub + b) * ORACLE_XBLK;",
                                           "const uint8_t *xb = Xq + (m * nsub + b) * ORACLE_XBLK;"
                                           " const uint8_t *xb0 = Xq + m * nsub * ORACLE_XBLK;"
                                           " (void)xb0;\n#define xb_d xb0"),
    "half decode bias": ("v = ldexp((double)(1024 + f), e - 25);", "v = ldexp((double)(1024 + f), e - 24);"),
    "half encode ties away": ("double m = rint(ldexp(x, 10 - e));",
                              "double m = floor(ldexp(x, 10 - e) + 0.5);"),
    "bf16 truncates": ("double m = rint(ldexp(f, 8));", "double m = trunc(ldexp(f, 8));"),
    "bf16 gemm drops activation rounding": (
        "double x = oracle_bf16_to_double(\n                    oracle_double_to_bf16(dx * (double)(int8_t)xb[4 + k % ORACLE_SB]));",
        "double x = dx * (double)(int8_t)xb[4 + k % ORACLE_SB];"),
    "bf16x3 drops the Wl*Xh product": ("total += wh * xh + wh * xl + wl * xh;", "total += wh * xh + wh * xl;"),
    "bf16x3 lo*lo in place of Wl*Xh": ("total += wh * xh + wh * xl + wl * xh;",
                                        "total += wh * xh + wh * xl + wl * xl;"),
    "bf16x3 lo rounds the value, not the residual": (
        "*lo = oracle_bf16_to_double(oracle_double_to_bf16(v - *hi));",
        "*lo = oracle_bf16_to_double(oracle_double_to_bf16(v)) - *hi;"),
    "bf16x3 activation scale of the next block": (
        "const uint8_t *xblk = Xq + (m * nsub + k / ORACLE_SB) * ORACLE_XBLK;",
        "const uint8_t *xblk = Xq + (m * nsub + (k / ORACLE_SB + 1) % nsub) * ORACLE_XBLK;"),
    "bf16x3 weight of the next sub-block": (
        "split_bf16(sb_scale(wblk, e / ORACLE_SB) * ORACLE_KV[code_at(wblk, e)], &wh, &wl);",
        "split_bf16(sb_scale(wblk, (e / ORACLE_SB + 1) % 8) * ORACLE_KV[code_at(wblk, e)], &wh, &wl);"),
    # IQ4_NL and Q4_0 (18-byte blocks)
    "b18 nibble order swapped": ("int c = t < 16 ? (byte & 15) : (byte >> 4);",
                                 "int c = t < 16 ? (byte >> 4) : (byte & 15);"),
    "q4_0 offset 7": ("return fmt == ORACLE_FMT_IQ4_NL ? ORACLE_KV[c] : c - 8;",
                      "return fmt == ORACLE_FMT_IQ4_NL ? ORACLE_KV[c] : c - 7;"),
    "iq4_nl and q4_0 values swapped": ("return fmt == ORACLE_FMT_IQ4_NL ? ORACLE_KV[c] : c - 8;",
                                       "return fmt == ORACLE_FMT_Q4_0 ? ORACLE_KV[c] : c - 8;"),
    "b18 index bytes start at 0": ("uint8_t byte = blk[2 + (t % 16)];", "uint8_t byte = blk[(t % 16)];"),
    "b18 scale from the last two bytes": ("return oracle_half_to_double((uint16_t)(blk[0] | (blk[1] << 8)));\n}\n\n/* Bytes",
                                          "return oracle_half_to_double((uint16_t)(blk[16] | (blk[17] << 8)));\n}\n\n/* Bytes"),
    "b18 gemm block stride 16": ("const uint8_t *blk = W + n * rb + j * ORACLE_B18;",
                                 "const uint8_t *blk = W + n * rb + j * 16;"),
    "b18 gemm activation block of the next weight block": (
        "const uint8_t *xq = Xq + (m * nblk + j) * ORACLE_XBLK;",
        "const uint8_t *xq = Xq + (m * nblk + (j + 1) % nblk) * ORACLE_XBLK;"),
    "b18 dequant block stride 16": ("const uint8_t *blk = W + n * rb + (k / ORACLE_SB) * ORACLE_B18;",
                                    "const uint8_t *blk = W + n * rb + (k / ORACLE_SB) * 16;"),
    "b18 gemm drops the weight scale": ("sum += scale18(blk) * d_x * (double)dot;", "sum += d_x * (double)dot;"),
    "b18 row bytes of 16 per block": ("return K / ORACLE_SB * ORACLE_B18;", "return K / ORACLE_SB * 16;"),
}

# one mutant above needs a second edit to take effect
EXTRA = {
    "gemm activation scale from block 0": (
        "double dx = oracle_half_to_double((uint16_t)(xb[0] | (xb[1] << 8)));\n                int64_t D",
        "double dx = oracle_half_to_double((uint16_t)(xb_d[0] | (xb_d[1] << 8)));\n                int64_t D"),
}


def _run_pins(o):
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except Exception:          # a mismatch, or a mutant whose output cannot even be read
            failed.append(pin.__name__)
    return failed


@pytest.fixture(scope="module")
def source():
    with open(oracle.SRC) as f:
        return f.read()


def test_unmodified_source_passes(tmp_path, source):
    path = tmp_path / "oracle.c"
    path.write_text(source)
    lib = oracle.build(out=str(tmp_path / "lib.so"), src=str(path))
    assert _run_pins(oracle.Oracle(lib)) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, source, name):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation site not unique for {name!r}"
    text = source.replace(old, new)
    if name in EXTRA:
        o2, n2 = EXTRA[name]
        assert text.count(o2) >= 1
        text = text.replace(o2, n2, 1)
    path = tmp_path / "oracle.c"
    path.write_text(text)
    lib = oracle.build(out=str(tmp_path / "lib.so"), src=str(path), extra=("-Wno-error",))
    failed = _run_pins(oracle.Oracle(lib))
    assert failed, f"no pin catches the mutant {name!r}"
