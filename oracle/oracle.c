/*
 * oracle.c -- plain, slow CPU oracle for the IQ4_XS x Q8_1 quantized matmul
 *             Y[M,N] = X[M,K] * W[N,K]^T.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the GPU library includes, links or
 * calls this file, and this file includes nothing from the GPU library.  The
 * only users are the test suite, the package smoke check and the CPU-baseline
 * leg of the benchmark.
 *
 * Sources (cited by page and section; the pages print no code):
 *   [E]  "V100TPS engine log" (agent-report.daedalus.work/V100TPS/engine.html),
 *        section on the batched IQ4_XS kernel: a 32-element IQ4_XS sub-block has
 *        the geometry of a Q4_0 block (four 32-bit words of packed nibbles, low
 *        nibbles are elements 0-15 and high nibbles elements 16-31); the scale
 *        stored per sub-block is d*(ls-32); the 4-bit value indexes the
 *        kvalues_iq4nl table instead of being used as q-8; activations are
 *        quantized to Q8_1 by quantize_q8_1.
 *   [G]  GGUF IQ4_XS / Q8_1 block formats (public ggml format description):
 *        the 136-byte super-block {fp16 d, u16 scales_h, u8 scales_l[4],
 *        u8 qs[128]}, the 16 kvalues_iq4nl constants, and the 36-byte Q8_1
 *        block {fp16 d, fp16 s, int8 qs[32]}.  The pages name these formats
 *        but print neither the byte layout nor the constants.
 *
 *   [S]  "SGLang MoE port thread" (lcz.me/post/31556), the passage that takes
 *        back an earlier conclusion about TP block alignment: an IQ4_NL block
 *        holds 32 values in 18 bytes (it had been mistaken for a 256-value
 *        block); and the passage on the per-layer embedding table, whose
 *        IQ4_NL rows were checked bit for bit against an independent decoder.
 *   The engine log's batched-kernel section also fixes the two 32-weight
 *   formats beside IQ4_XS: a Q4_0 block is exactly the geometry of an IQ4_XS
 *   sub-block (four 32-bit words of nibbles, low nibbles elements 0-15, high
 *   nibbles 16-31) with one scale d per block and the value q-8; IQ4_NL
 *   (the format the kvalues_iq4nl codebook is named for) has the same block
 *   with the value kvalues_iq4nl[q].
 *
 * Readings where the pages are silent (each one stated where it is used):
 *   R1  field order and 6-bit scale assembly follow [G];
 *   R2  Q8_1 of a 32-element block: amax = max|x| (fp32), d = amax/127 as an
 *       IEEE fp32 division, q = round-half-away-from-zero of the IEEE fp32
 *       quotient x/d (q = 0 when d == 0), clamped to [-127,127]; stored d is
 *       fp16(d) rounded to nearest even; stored s is fp16(d_stored * sum(q)),
 *       the sum of the values the block represents (exact in fp32 before the
 *       single rounding to fp16);
 *   R3  the GEMM uses the stored fp16 d of each Q8_1 block and ignores s;
 *   R4  the dequantize-to-bf16 variant rounds W~ = d*(ls-32)*kv and
 *       X~ = d_x*q to bf16 (nearest even) and sums their exact products;
 *   R5  an IQ4_NL or Q4_0 block of 18 bytes is {fp16 d, u8 qs[16]} (the GGUF
 *       order: the scale first, then the 16 nibble bytes laid out as in an
 *       IQ4_XS sub-block); a row of K weights is K/32 consecutive blocks;
 *   R6  the compensated bf16 variant (this library's route to putting the
 *       dequantize-then-GEMM path under the same per-row bound as the
 *       integer path) splits each of W~ and X~ into hi = bf16(v) and
 *       lo = bf16(v - hi), both nearest even, and sums
 *       Wh*Xh + Wh*Xl + Wl*Xh per element (the lo*lo product is dropped).
 *
 * Arithmetic.  Every decoded weight d*(ls-32)*kv needs at most 11+6+7 = 24
 * significant bits and every product term d_w*(ls-32)*d_x*D at most 48, so
 * each term is exact in fp64; the only rounding in the GEMM is the fp64 sum,
 * taken in ascending sub-block (or element) order.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_QK 256      /* elements per IQ4_XS super-block          */
#define ORACLE_SB 32       /* elements per sub-block and per Q8_1 block */
#define ORACLE_WBLK 136    /* bytes per IQ4_XS super-block              */
#define ORACLE_XBLK 36     /* bytes per Q8_1 block                      */

/* [G] kvalues_iq4nl: the non-linear codebook the 4-bit indices select from. */
static const int ORACLE_KV[16] = {-127, -104, -83, -65, -49, -35, -22, -10,
                                  1,    13,   25,  38,  53,  69,  89,  113};

int oracle_kvalue(int i) { return (i >= 0 && i < 16) ? ORACLE_KV[i] : 0; }

/* ---------------------------------------------------------------- fp16 */

/* IEEE binary16 -> value: sign, 5-bit exponent (bias 15), 10-bit fraction. */
double oracle_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);                 /* zero or subnormal */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);     /* 1.f * 2^(e-15) */
    return sign ? -v : v;
}

/* value -> IEEE binary16, round to nearest, ties to even (R2). */
uint16_t oracle_float_to_half(float xf)
{
    double x = (double)xf;                        /* exact */
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    if (isnan(x))
        return (uint16_t)(sign | 0x7E00);
    x = fabs(x);
    if (isinf(x))
        return (uint16_t)(sign | 0x7C00);
    if (x < ldexp(1.0, -14)) {
        /* subnormal range: multiples of 2^-24 */
        double m = rint(ldexp(x, 24));            /* default mode: ties-to-even */
        return (uint16_t)(sign | (uint16_t)m);    /* m == 1024 is the smallest normal */
    }
    int e;
    frexp(x, &e);                                 /* x = f * 2^e, f in [0.5, 1) */
    e -= 1;                                       /* x = 1.xxx * 2^e */
    double m = rint(ldexp(x, 10 - e));            /* 11 significant bits */
    if (m == 2048.0) {
        m = 1024.0;
        e += 1;
    }
    if (e > 15)
        return (uint16_t)(sign | 0x7C00);         /* overflow to infinity */
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)(m - 1024.0));
}

/* value (a normal fp32 number) -> bfloat16 bits, nearest even (R4). */
uint16_t oracle_double_to_bf16(double x)
{
    if (x == 0.0)
        return signbit(x) ? 0x8000 : 0;
    int e;
    double f = frexp(x, &e);                      /* |f| in [0.5, 1) */
    double m = rint(ldexp(f, 8));                 /* 8 significant bits */
    float r = (float)ldexp(m, e - 8);             /* exact in fp32 */
    uint32_t bits;
    memcpy(&bits, &r, 4);
    return (uint16_t)(bits >> 16);
}

double oracle_bf16_to_double(uint16_t b)
{
    uint32_t bits = (uint32_t)b << 16;
    float r;
    memcpy(&r, &bits, 4);
    return (double)r;
}

/* --------------------------------------------------------- IQ4_XS decode */

static double sb_scale(const uint8_t *blk, int b)
{
    /* R1/[G]: d at bytes 0-1, scales_h (little-endian u16) at 2-3,
       scales_l[4] at 4-7.  Sub-block b's 6-bit scale: low 4 bits from
       nibble (b%2) of scales_l[b/2], high 2 bits from bits 2b..2b+1 of
       scales_h.  [E]: effective scale d*(ls-32). */
    double d = oracle_half_to_double((uint16_t)(blk[0] | (blk[1] << 8)));
    unsigned scales_h = (unsigned)blk[2] | ((unsigned)blk[3] << 8);
    int lo4 = (blk[4 + b / 2] >> (4 * (b % 2))) & 15;
    int hi2 = (scales_h >> (2 * b)) & 3;
    int ls = lo4 | (hi2 << 4);
    return d * (double)(ls - 32);
}

static int code_at(const uint8_t *blk, int i)
{
    /* [E]: sub-block b = i/32 uses 16 bytes; element t of the sub-block is the
       low nibble of byte t for t < 16 and the high nibble of byte t-16
       otherwise.  R1/[G]: the 128 index bytes start at byte 8 and sub-block b
       owns bytes 8+16b .. 8+16b+15. */
    int b = i / ORACLE_SB, t = i % ORACLE_SB;
    uint8_t byte = blk[8 + 16 * b + (t % 16)];
    return t < 16 ? (byte & 15) : (byte >> 4);
}

/* W~[n,k] = d*(ls-32)*kvalues[code], exact in fp64.  out is [N][K]. */
void oracle_dequantize(const uint8_t *W, int64_t N, int64_t K, double *out)
{
    int64_t nb = K / ORACLE_QK;
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++) {
            const uint8_t *blk = W + (n * nb + k / ORACLE_QK) * ORACLE_WBLK;
            int i = (int)(k % ORACLE_QK);
            out[n * K + k] = sb_scale(blk, i / ORACLE_SB) * ORACLE_KV[code_at(blk, i)];
        }
}

/* bf16 bits of W~ (R4).  out is [N][K]. */
void oracle_dequantize_bf16(const uint8_t *W, int64_t N, int64_t K, uint16_t *out)
{
    int64_t nb = K / ORACLE_QK;
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++) {
            const uint8_t *blk = W + (n * nb + k / ORACLE_QK) * ORACLE_WBLK;
            int i = (int)(k % ORACLE_QK);
            out[n * K + k] = oracle_double_to_bf16(sb_scale(blk, i / ORACLE_SB) *
                                                   ORACLE_KV[code_at(blk, i)]);
        }
}

/* ------------------------------------------------------------ Q8_1 */

/* R2.  X is fp32 [M][K]; out is [M][K/32] blocks of 36 bytes. */
void oracle_quantize_q8_1(const float *X, int64_t M, int64_t K, uint8_t *out)
{
    int64_t nblk = K / ORACLE_SB;
    for (int64_t m = 0; m < M; m++)
        for (int64_t b = 0; b < nblk; b++) {
            const float *x = X + m * K + b * ORACLE_SB;
            uint8_t *o = out + (m * nblk + b) * ORACLE_XBLK;
            float amax = 0.0f;
            for (int i = 0; i < ORACLE_SB; i++)
                if (fabsf(x[i]) > amax)
                    amax = fabsf(x[i]);
            float d = amax / 127.0f;                 /* IEEE fp32 division */
            int sum = 0;
            for (int i = 0; i < ORACLE_SB; i++) {
                int q = 0;
                if (d != 0.0f) {
                    float quot = x[i] / d;           /* IEEE fp32 division */
                    q = (int)roundf(quot);           /* half away from zero */
                    if (q > 127) q = 127;
                    if (q < -127) q = -127;
                }
                o[4 + i] = (uint8_t)(int8_t)q;
                sum += q;
            }
            uint16_t d16 = oracle_float_to_half(d);
            float dst = (float)oracle_half_to_double(d16);
            uint16_t s16 = oracle_float_to_half(dst * (float)sum);   /* product exact in fp32 */
            o[0] = (uint8_t)(d16 & 0xFF);
            o[1] = (uint8_t)(d16 >> 8);
            o[2] = (uint8_t)(s16 & 0xFF);
            o[3] = (uint8_t)(s16 >> 8);
        }
}

/* ------------------------------------------------------------ GEMM */

static int n_threads = 0;   /* 0: OpenMP default */

void oracle_set_threads(int t) { n_threads = t; }

int oracle_get_threads(void)
{
#ifdef _OPENMP
    return n_threads > 0 ? n_threads : omp_get_max_threads();
#else
    return 1;
#endif
}

/* Integer-dot formulation ([E], R3):
     Y[m,n] = sum_b  d_w[n,b/8]*(ls[n,b]-32) * d_x[m,b] * D[m,n,b],
     D[m,n,b] = sum_{t<32} kvalues[code(n, 32b+t)] * q[m, 32b+t]  (exact int).
   W is [N][K/256] super-blocks, Xq is [M][K/32] Q8_1 blocks, Y is [M][N]. */
void oracle_gemm_q8_1(const uint8_t *W, const uint8_t *Xq, int64_t M, int64_t N, int64_t K,
                      double *Y)
{
    int64_t nb = K / ORACLE_QK, nsub = K / ORACLE_SB;
#pragma omp parallel for schedule(static) num_threads(oracle_get_threads())
    for (int64_t n = 0; n < N; n++)
        for (int64_t m = 0; m < M; m++) {
            double acc = 0.0;
            for (int64_t b = 0; b < nsub; b++) {
                const uint8_t *blk = W + (n * nb + b / 8) * ORACLE_WBLK;
                const uint8_t *xb = Xq + (m * nsub + b) * ORACLE_XBLK;
                double sw = sb_scale(blk, (int)(b % 8));
                double dx = oracle_half_to_double((uint16_t)(xb[0] | (xb[1] << 8)));
                int64_t D = 0;
                for (int t = 0; t < ORACLE_SB; t++)
                    D += (int64_t)ORACLE_KV[code_at(blk, (int)(32 * (b % 8) + t))] *
                         (int64_t)(int8_t)xb[4 + t];
                acc += sw * dx * (double)D;
            }
            Y[m * N + n] = acc;
        }
}

/* Dequantize-to-bf16 formulation (R4):
     Y[m,n] = sum_k bf16(W~[n,k]) * bf16(d_x[m,k/32] * q[m,k]),
   products exact in fp64, summed in ascending k. */
void oracle_gemm_bf16(const uint8_t *W, const uint8_t *Xq, int64_t M, int64_t N, int64_t K,
                      double *Y)
{
    int64_t nb = K / ORACLE_QK, nsub = K / ORACLE_SB;
#pragma omp parallel for schedule(static) num_threads(oracle_get_threads())
    for (int64_t n = 0; n < N; n++)
        for (int64_t m = 0; m < M; m++) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; k++) {
                const uint8_t *blk = W + (n * nb + k / ORACLE_QK) * ORACLE_WBLK;
                int i = (int)(k % ORACLE_QK);
                double w = oracle_bf16_to_double(oracle_double_to_bf16(
                    sb_scale(blk, i / ORACLE_SB) * ORACLE_KV[code_at(blk, i)]));
                const uint8_t *xb = Xq + (m * nsub + k / ORACLE_SB) * ORACLE_XBLK;
                double dx = oracle_half_to_double((uint16_t)(xb[0] | (xb[1] << 8)));
                double x = oracle_bf16_to_double(
                    oracle_double_to_bf16(dx * (double)(int8_t)xb[4 + k % ORACLE_SB]));
                acc += w * x;
            }
            Y[m * N + n] = acc;
        }
}

/* hi and lo bf16 parts of v (R6): hi = bf16(v), lo = bf16(v - hi). */
static void split_bf16(double v, double *hi, double *lo)
{
    *hi = oracle_bf16_to_double(oracle_double_to_bf16(v));
    *lo = oracle_bf16_to_double(oracle_double_to_bf16(v - *hi));
}

/* Compensated bf16 formulation (R6):
     Y[m,n] = sum_k Wh*Xh + Wh*Xl + Wl*Xh,
   (Wh, Wl) the split of W~[n,k] = d*(ls-32)*kv, (Xh, Xl) that of
   X~[m,k] = d_x*q; products exact in fp64, summed in ascending k. */
void oracle_gemm_bf16x3(const uint8_t *W, const uint8_t *Xq, int64_t M, int64_t N, int64_t K,
                        double *Y)
{
    int64_t nb = K / ORACLE_QK, nsub = K / ORACLE_SB;
#pragma omp parallel for schedule(static) num_threads(oracle_get_threads())
    for (int64_t n = 0; n < N; n++)
        for (int64_t m = 0; m < M; m++) {
            double total = 0.0;
            for (int64_t k = 0; k < K; k++) {
                const uint8_t *wblk = W + (n * nb + k / ORACLE_QK) * ORACLE_WBLK;
                int e = (int)(k % ORACLE_QK);
                double wh, wl, xh, xl;
                split_bf16(sb_scale(wblk, e / ORACLE_SB) * ORACLE_KV[code_at(wblk, e)], &wh, &wl);
                const uint8_t *xblk = Xq + (m * nsub + k / ORACLE_SB) * ORACLE_XBLK;
                double d_act = oracle_half_to_double((uint16_t)(xblk[0] | (xblk[1] << 8)));
                split_bf16(d_act * (double)(int8_t)xblk[4 + k % ORACLE_SB], &xh, &xl);
                total += wh * xh + wh * xl + wl * xh;
            }
            Y[m * N + n] = total;
        }
}

/* ------------------------------------------ IQ4_NL and Q4_0 (R5, [E], [S]) */

#define ORACLE_B18 18      /* bytes per IQ4_NL / Q4_0 block of 32 weights */

/* Weight formats of oracle_dequantize_fmt / oracle_gemm_fmt_q8_1. */
#define ORACLE_FMT_IQ4_XS 0
#define ORACLE_FMT_IQ4_NL 1
#define ORACLE_FMT_Q4_0 2

/* Value of element t (0..31) of an 18-byte block, without its scale: the
   nibble placement of an IQ4_XS sub-block ([E]: low nibbles are elements
   0-15, high nibbles 16-31), the 16 nibble bytes after the fp16 d (R5). */
static int value18(int fmt, const uint8_t *blk, int t)
{
    uint8_t byte = blk[2 + (t % 16)];
    int c = t < 16 ? (byte & 15) : (byte >> 4);
    return fmt == ORACLE_FMT_IQ4_NL ? ORACLE_KV[c] : c - 8;   /* Q4_0: q - 8 */
}

static double scale18(const uint8_t *blk)
{
    return oracle_half_to_double((uint16_t)(blk[0] | (blk[1] << 8)));
}

/* Bytes of one row of K weights in a format (K % 256 == 0 for IQ4_XS, K % 32
   for the 32-weight formats); 0 for an unknown format. */
int64_t oracle_row_bytes(int fmt, int64_t K)
{
    if (fmt == ORACLE_FMT_IQ4_XS)
        return K / ORACLE_QK * ORACLE_WBLK;
    if (fmt == ORACLE_FMT_IQ4_NL || fmt == ORACLE_FMT_Q4_0)
        return K / ORACLE_SB * ORACLE_B18;
    return 0;
}

/* W~[n,k], exact in fp64, for any of the three formats.  out is [N][K]. */
void oracle_dequantize_fmt(int fmt, const uint8_t *W, int64_t N, int64_t K, double *out)
{
    if (fmt == ORACLE_FMT_IQ4_XS) {
        oracle_dequantize(W, N, K, out);
        return;
    }
    int64_t rb = oracle_row_bytes(fmt, K);
    for (int64_t n = 0; n < N; n++)
        for (int64_t k = 0; k < K; k++) {
            const uint8_t *blk = W + n * rb + (k / ORACLE_SB) * ORACLE_B18;
            out[n * K + k] = scale18(blk) * (double)value18(fmt, blk, (int)(k % ORACLE_SB));
        }
}

/* Integer-dot formulation for any format ([E], R3, R5):
     Y[m,n] = sum_b s_w[n,b] * d_x[m,b] * D[m,n,b],
   s_w = d of block b (IQ4_NL, Q4_0) or d*(ls-32) (IQ4_XS), D the exact
   integer dot of the 32 block values with the Q8_1 values.  Every term is
   exact in fp64 (11 + 11 + 20 significant bits); the sum runs over b in
   ascending order. */
void oracle_gemm_fmt_q8_1(int fmt, const uint8_t *W, const uint8_t *Xq, int64_t M, int64_t N, int64_t K,
                          double *Y)
{
    if (fmt == ORACLE_FMT_IQ4_XS) {
        oracle_gemm_q8_1(W, Xq, M, N, K, Y);
        return;
    }
    int64_t rb = oracle_row_bytes(fmt, K), nblk = K / ORACLE_SB;
#pragma omp parallel for schedule(static) num_threads(oracle_get_threads())
    for (int64_t n = 0; n < N; n++)
        for (int64_t m = 0; m < M; m++) {
            double sum = 0.0;
            for (int64_t j = 0; j < nblk; j++) {
                const uint8_t *blk = W + n * rb + j * ORACLE_B18;
                const uint8_t *xq = Xq + (m * nblk + j) * ORACLE_XBLK;
                double d_x = oracle_half_to_double((uint16_t)(xq[0] | (xq[1] << 8)));
                int64_t dot = 0;
                for (int t = 0; t < ORACLE_SB; t++)
                    dot += (int64_t)value18(fmt, blk, t) * (int64_t)(int8_t)xq[4 + t];
                sum += scale18(blk) * d_x * (double)dot;
            }
            Y[m * N + n] = sum;
        }
}

/* ------------------------------------------------- array helpers (tests) */

void oracle_float_to_half_array(const float *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_float_to_half(x[i]);
}

void oracle_half_to_double_array(const uint16_t *h, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_half_to_double(h[i]);
}

void oracle_double_to_bf16_array(const double *x, int64_t n, uint16_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_double_to_bf16(x[i]);
}
