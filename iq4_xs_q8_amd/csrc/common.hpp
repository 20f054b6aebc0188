// common.hpp -- internal definitions shared by the HIP kernels of libiq4xs.
//
// Format facts ("V100TPS engine log", agent-report.daedalus.work/V100TPS/engine.html,
// section on the batched IQ4_XS kernel; byte layout and codebook from the GGUF
// IQ4_XS / Q8_1 formats, which the pages name but do not print):
//   IQ4_XS super-block = 256 weights in 136 bytes {fp16 d, u16 scales_h,
//   u8 scales_l[4], u8 qs[128]}; sub-block b = 32 weights in qs[16b..16b+15],
//   low nibbles are elements 0-15, high nibbles 16-31; scale d*(ls-32);
//   weight = scale * kvalues_iq4nl[nibble].
//   Q8_1 block = 32 activations in 36 bytes {fp16 d, fp16 s, int8 q[32]}.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace iq4xs {

constexpr int QK = 256;         // weights per super-block
constexpr int SB = 32;          // weights per sub-block, activations per Q8_1 block
constexpr int SUBS = QK / SB;   // sub-blocks per super-block
constexpr int WBLK = 136;       // bytes per IQ4_XS super-block
constexpr int XBLK = 36;        // bytes per Q8_1 block
constexpr int QS_OFF = 8;       // offset of qs[] inside a super-block
static_assert(2 + 2 + 4 + QK / 2 == WBLK, "IQ4_XS super-block size");
static_assert(QS_OFF == 2 + 2 + 4, "qs follows d, scales_h, scales_l");
static_assert(2 + 2 + SB == XBLK, "Q8_1 block size");

// Rows of the internal activation planes are padded to a multiple of this,
// so the block scales of four consecutive rows are one aligned float4.
constexpr int MPAD = 4;

// ---- weight formats ---------------------------------------------------------
// IQ4_XS: 136-byte super-blocks of 256 weights (above).  IQ4_NL and Q4_0: a
// block of 32 weights is 18 bytes {fp16 d, u8 qs[16]} with the nibble layout
// of an IQ4_XS sub-block ("V100TPS engine log", batched IQ4_XS kernel
// section: a Q4_0 block has exactly that geometry, one scale d per block and
// the value q-8; "SGLang MoE port thread": an IQ4_NL block is 32 values in 18
// bytes, its values the kvalues_iq4nl codebook).  The kernels walk every
// format in units of 256 weights: eight 18-byte blocks make a 144-byte unit,
// which (unlike 136 bytes) is always 16-byte aligned.
enum : int { FMT_IQ4_XS = 0, FMT_IQ4_NL = 1, FMT_Q4_0 = 2, NUM_FMTS = 3 };
constexpr int B18 = 18;   // bytes per IQ4_NL / Q4_0 block
constexpr int sblk_bytes(int f) { return f == FMT_IQ4_XS ? 136 : 8 * B18; }
static_assert(sblk_bytes(FMT_IQ4_NL) % 16 == 0, "144-byte units stay 16-byte aligned");

// ---- kvalues_iq4nl packed for byte-permute lookups -----------------------
constexpr int8_t KVALUES[16] = {-127, -104, -83, -65, -49, -35, -22, -10,
                                1,    13,   25,  38,  53,  69,  89,  113};
constexpr uint32_t kv_word(int i)
{
    return (uint32_t)(uint8_t)KVALUES[4 * i] | ((uint32_t)(uint8_t)KVALUES[4 * i + 1] << 8) |
           ((uint32_t)(uint8_t)KVALUES[4 * i + 2] << 16) |
           ((uint32_t)(uint8_t)KVALUES[4 * i + 3] << 24);
}
constexpr uint32_t KV0 = kv_word(0), KV1 = kv_word(1), KV2 = kv_word(2), KV3 = kv_word(3);
static_assert(KV0 == 0xBFAD9881u && KV3 == 0x71594535u, "codebook packing");

// Q4_0's values q-8 as a 16-entry table of the same kind.
constexpr int8_t Q40VALUES[16] = {-8, -7, -6, -5, -4, -3, -2, -1, 0, 1, 2, 3, 4, 5, 6, 7};

// The 16-entry value table of a format, packed four bytes per word.
template <int F>
struct Values {
    static constexpr const int8_t *t = F == FMT_Q4_0 ? Q40VALUES : KVALUES;
    static constexpr uint32_t w(int i)
    {
        return (uint32_t)(uint8_t)t[4 * i] | ((uint32_t)(uint8_t)t[4 * i + 1] << 8) |
               ((uint32_t)(uint8_t)t[4 * i + 2] << 16) | ((uint32_t)(uint8_t)t[4 * i + 3] << 24);
    }
    static constexpr uint32_t W0 = w(0), W1 = w(1), W2 = w(2), W3 = w(3);
};
static_assert(Values<FMT_IQ4_XS>::W0 == KV0 && Values<FMT_IQ4_NL>::W3 == KV3, "codebook packing");
static_assert(Values<FMT_Q4_0>::W0 == 0xFBFAF9F8u && Values<FMT_Q4_0>::W3 == 0x07060504u, "q-8 packing");

// Four 4-bit indices -> four int8 values with byte permutes.  v_perm_b32
// picks byte s (0..7) of {hi:lo}, gives 0x00 for selector 5 of {0:0} and
// 0xFF for any selector >= 13: indices 0-7 come from {W1:W0}, 8-15 from
// {W3:W2}, and a mask built from bit 3 (selector 5 or 13) chooses per byte.
// The indices are bits 0-3 of each byte of t; bits 4-7 are ignored.
template <int F = FMT_IQ4_XS>
__device__ __forceinline__ uint32_t lut4(uint32_t t)
{
    using V = Values<F>;
    const uint32_t s = t & 0x07070707u;
    const uint32_t a = __builtin_amdgcn_perm(V::W1, V::W0, s);
    const uint32_t b = __builtin_amdgcn_perm(V::W3, V::W2, s);
    const uint32_t m = __builtin_amdgcn_perm(0u, 0u, (t & 0x08080808u) | 0x05050505u);
    return (m & b) | (~m & a);
}

// 8 index bytes (2 dwords of qs) -> 16 int8 weights in "chunk" order:
// out[0..1] = low nibbles (elements j..j+7), out[2..3] = high nibbles
// (elements 16+j..16+j+7) of the same bytes.
template <int F = FMT_IQ4_XS>
__device__ __forceinline__ void expand8(uint32_t w0, uint32_t w1, uint32_t out[4])
{
    out[0] = lut4<F>(w0);
    out[1] = lut4<F>(w1);
    out[2] = lut4<F>(w0 >> 4);
    out[3] = lut4<F>(w1 >> 4);
}

// Split codebook: kvalues[x] = KL[x & 7] + kh(x ^ 13), where kh(s) is what
// v_perm_b32 returns for selector s over the table KH: KH[s] for s < 8, the
// sign byte of KH[1|3|5|7] (0x00: all are positive) for s = 8..11, 0x00 for
// 12 and 0xFF (-1) for 13..15.  x ^ 13 maps x = 8..15 onto 0..7 and gives
// x = 0, 2, 3 the value -1, which KL absorbs (KL[0] = -126 where kvalues[0]
// = -127).  Both parts fit int8, so a dot product with the codebook values is
// the sum of two dot products with two byte-permute lookups, one selector
// op each: no per-byte select between two half-tables.
constexpr int8_t KL[8] = {-126, -104, -82, -64, -49, -35, -22, -10};
constexpr int8_t KH[8] = {104, 102, 123, 111, 117, 127, 102, 107};
// The same split of Q4_0's q-8 (all KH parts positive, so selectors 8-11
// give 0 and x = 0, 2, 3 get the -1 that KL absorbs).
constexpr int8_t QL[8] = {-7, -7, -5, -4, -4, -3, -2, -1};
constexpr int8_t QH[8] = {8, 8, 8, 8, 8, 7, 7, 7};
constexpr int perm_byte(const int8_t *t8, int sel)
{
    return sel >= 13 ? -1 : sel == 12 ? 0 : sel >= 8 ? (t8[2 * (sel - 8) + 1] < 0 ? -1 : 0) : t8[sel];
}
constexpr bool split_ok(const int8_t *lo, const int8_t *hi, const int8_t *want)
{
    for (int x = 0; x < 16; x++)
        if (lo[x & 7] + perm_byte(hi, x ^ 13) != want[x])
            return false;
    return true;
}
static_assert(split_ok(KL, KH, KVALUES), "split codebook");
static_assert(split_ok(QL, QH, Q40VALUES), "split q-8");
constexpr uint32_t word4(const int8_t *b)
{
    return (uint32_t)(uint8_t)b[0] | ((uint32_t)(uint8_t)b[1] << 8) | ((uint32_t)(uint8_t)b[2] << 16) |
           ((uint32_t)(uint8_t)b[3] << 24);
}
constexpr uint32_t KL0 = word4(KL), KL1 = word4(KL + 4), KH0 = word4(KH), KH1 = word4(KH + 4);
template <int F>
struct Split {
    static constexpr const int8_t *lo = F == FMT_Q4_0 ? QL : KL;
    static constexpr const int8_t *hi = F == FMT_Q4_0 ? QH : KH;
    static constexpr uint32_t L0 = word4(lo), L1 = word4(lo + 4), H0 = word4(hi), H1 = word4(hi + 4);
};
static_assert(Split<FMT_IQ4_NL>::L0 == KL0 && Split<FMT_IQ4_XS>::H1 == KH1, "split packing");

// Four indices (bits 0-3 of each byte of t; bits 4-7 ignored) -> the two
// int8 parts of their values.
template <int F = FMT_IQ4_XS>
__device__ __forceinline__ void lut4_split(uint32_t t, uint32_t &lo, uint32_t &hi)
{
    using S = Split<F>;
    lo = __builtin_amdgcn_perm(S::L1, S::L0, t & 0x07070707u);
    hi = __builtin_amdgcn_perm(S::H1, S::H0, (t & 0x0F0F0F0Fu) ^ 0x0D0D0D0Du);
}

// expand8 as two parts: a[i] + b[i] (bytewise, as integers) = out[i] of expand8.
template <int F = FMT_IQ4_XS>
__device__ __forceinline__ void expand8_split(uint32_t w0, uint32_t w1, uint32_t a[4], uint32_t b[4])
{
    lut4_split<F>(w0, a[0], b[0]);
    lut4_split<F>(w1, a[1], b[1]);
    lut4_split<F>(w0 >> 4, a[2], b[2]);
    lut4_split<F>(w1 >> 4, a[3], b[3]);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t h16)
{
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h16);
}

// Effective scale d*(ls_b - 32) of sub-block b from the first 8 header bytes
// (h0 = bytes 0-3 = d | scales_h << 16, h1 = bytes 4-7 = scales_l).  Exact in
// fp32 (11 + 6 significant bits).
__device__ __forceinline__ float sub_scale(uint32_t h0, uint32_t h1, int b)
{
    const uint32_t lo4 = (h1 >> (4 * b)) & 15u;           // nibble b%2 of scales_l[b/2]
    const uint32_t hi2 = (h0 >> (16 + 2 * b)) & 3u;       // bits 2b..2b+1 of scales_h
    const int ls = (int)(lo4 | (hi2 << 4));
    return half_bits_to_float(h0 & 0xFFFFu) * (float)(ls - 32);
}

// ---- one 256-weight unit of any format -------------------------------------
// `u` points at the unit (4-byte aligned): an IQ4_XS super-block, or eight
// IQ4_NL / Q4_0 blocks.  The 18-byte blocks put d and the index bytes at
// offsets that are only 2-byte aligned, so they are read as aligned dwords
// and shifted into place (v_alignbit), and nothing past the unit is read.

// Scale of sub-block b (0..7): d*(ls_b - 32), or the d of block b, in two
// steps so that the read can be issued with other loads and decoded later:
// the raw bytes (IQ4_XS: the 8 header bytes; else the dword holding d_b), then
// the value.  live == false gives 0 (a sub-block that only pads a group).
template <int F>
__device__ __forceinline__ uint2 unit_scale_raw(const char *u, int b)
{
    if constexpr (F == FMT_IQ4_XS)
        return *reinterpret_cast<const uint2 *>(u);
    else
        return make_uint2(*reinterpret_cast<const uint32_t *>(u + ((B18 * b) & ~3)), 0u);
}
template <int F>
__device__ __forceinline__ float unit_scale_dec(uint2 raw, int b, bool live)
{
    if constexpr (F == FMT_IQ4_XS) {
        return sub_scale(live ? raw.x : 0u, raw.y, b);
    } else {
        // d_b sits at byte 18b: the low half of its dword for even b, the
        // high half of the dword before for odd b
        const uint32_t bits = (b & 1) ? (raw.x >> 16) : (raw.x & 0xFFFFu);
        return live ? half_bits_to_float(bits) : 0.0f;
    }
}
template <int F>
__device__ __forceinline__ float unit_scale(const char *u, int b, bool live)
{
    return unit_scale_dec<F>(unit_scale_raw<F>(u, b), b, live);
}

// The 8 index bytes qs[8h..8h+7] of sub-block b (16 weights: elements
// 8h..8h+7 in the low nibbles, 16+8h..16+8h+7 in the high ones).
template <int F>
__device__ __forceinline__ uint2 unit_qs(const char *u, int b, int h)
{
    if constexpr (F == FMT_IQ4_XS) {
        return *reinterpret_cast<const uint2 *>(u + QS_OFF + 16 * b + 8 * h);
    } else {
        const int o = B18 * b + 2 + 8 * h;                     // 0 or 2 mod 4
        const uint32_t *w = reinterpret_cast<const uint32_t *>(u + (o & ~3));
        const uint32_t w0 = w[0], w1 = w[1];
        if (o & 2) {                                           // bytes o..o+7 span three dwords
            const uint32_t w2 = w[2];
            return make_uint2(__builtin_amdgcn_alignbit(w1, w0, 16), __builtin_amdgcn_alignbit(w2, w1, 16));
        }
        return make_uint2(w0, w1);
    }
}

// ---- internal activation planes ------------------------------------------
// The matmul kernels read Q8_1 activations from two sub-block-major planes
// instead of the 36-byte ABI blocks (Mp = M rounded up to MPAD):
//   qp  int8  [K/32][Mp][32]  the 32 values of block b of row m at
//                              qp[(b*Mp + m)*32], in "chunk" order: bytes 0-7 =
//                              elements 0-7, 8-15 = elements 16-23, 16-23 =
//                              elements 8-15, 24-31 = elements 24-31, so chunk h
//                              (16 bytes at 16h) holds the elements paired with
//                              the low and high nibbles of qs[16b'+8h .. +7];
//   dp  float [K/32][Mp]      the block scales d (fp16 widened).
// The 32 rows of one block are 1 KB of contiguous bytes, the MFMA operand of a
// 32-row tile.  Rows M..Mp-1 are allocated but never written: the kernels
// either read a zero row in their place or discard what they compute from
// them.
struct XPlanes {
    int8_t *qp;
    float *dp;
    int64_t M, Mp, K;
};

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
inline size_t xplanes_bytes(int64_t M, int64_t K)
{
    const int64_t Mp = round_up(M, MPAD);
    return (size_t)(Mp * K) + (size_t)(Mp * (K / SB)) * sizeof(float);
}
inline XPlanes xplanes_at(void *base, int64_t M, int64_t K)
{
    XPlanes p;
    p.M = M;
    p.Mp = round_up(M, MPAD);
    p.K = K;
    p.qp = (int8_t *)base;
    p.dp = (float *)((char *)base + p.Mp * K);
    return p;
}

// Up to MAXGRP weight matrices with the same K that share one X (the
// streaming kernel's grouped launch): matrix g has N[g] rows at w[g] and its
// own output y[g] ([M][N[g]]); its 32-column tiles are t0[g] .. t0[g+1]-1 of
// the tiles numbered across the group.
constexpr int MAXGRP = 4;
struct MmvGroup {
    const uint8_t *w[MAXGRP];
    float *y[MAXGRP];
    int n[MAXGRP];
    int t0[MAXGRP + 1];
    int count;
    __device__ __forceinline__ int matrix_of(int t) const
    {
        int gi = 0;
#pragma unroll
        for (int q = 1; q < MAXGRP; q++)
            gi += (q < count && t >= t0[q]) ? 1 : 0;
        return gi;
    }
};

// Outputs the quantize kernels zero on the way (for matmuls that add partial
// tiles into Y): up to MAXGRP ranges p[i][0..n[i]), 16-byte aligned.
// ---- compensated bf16 activations (fused.hip) ------------------------------
// The fused dequantize-in-LDS kernel reads X~ = d_x*q (exact in fp32) as two
// bf16 numbers, hi = bf16(X~) and lo = bf16(X~ - hi), from planes the
// quantizer writes: u16 [K/32][Ms][64], row m of block b at (b*Ms + m)*64,
// hi[32] then lo[32] in element order; Ms = M rounded up to FUSED_ROWS, rows
// M..Ms-1 zero.
constexpr int FUSED_ROWS = 256;
struct XSplit {
    uint16_t *p = nullptr;
    int64_t Ms = 0;
};
inline int64_t fused_ms(int64_t M) { return (M + FUSED_ROWS - 1) / FUSED_ROWS * FUSED_ROWS; }
inline size_t fused_xs_bytes(int64_t M, int64_t K) { return (size_t)(K / SB) * (size_t)fused_ms(M) * 128; }

// hi = bf16(a), bf16(b) (nearest even; v_cvt_pk_bf16_f32) and lo = the bf16
// of what hi leaves out (exact in fp32), packed low element first.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void bf16x2_split(float a, float b, uint32_t &hi, uint32_t &lo)
{
    const bf16x2_t h = {(__bf16)a, (__bf16)b};
    hi = __builtin_bit_cast(uint32_t, h);
    const float ra = a - __builtin_bit_cast(float, hi << 16);
    const float rb = b - __builtin_bit_cast(float, hi & 0xFFFF0000u);
    const bf16x2_t l = {(__bf16)ra, (__bf16)rb};
    lo = __builtin_bit_cast(uint32_t, l);
}

// Tiles of Y that two workgroups of the tile kernel add into (a stream-K run
// boundary falls inside each): zeroed before the matmul instead of all of Y.
// Tile t covers rows (t / wblocks)*bm .. +bm and columns (t % wblocks)*bn .. +bn.
constexpr int MAXZT = 256;
struct ZeroTiles {
    float *y = nullptr;
    int64_t M = 0, N = 0;
    int bm = 0, bn = 0, wblocks = 0, count = 0;
    int t[MAXZT] = {};
};

// What a quantize launch zeroes besides its work: whole ranges (one per
// matrix of a grouped call) and the shared tiles of one tile-kernel call.
struct ZeroList {
    float *p[MAXGRP] = {};
    int64_t n[MAXGRP] = {};
    int count = 0;
    ZeroTiles tiles;
};

// ---- launchers (each defined in the .hip file that holds its kernel) -----
// All return a hipError_t from hipGetLastError() after the launch.  The
// quantizers also zero yz[0..nz) when yz is given (the output of a matmul
// that adds partial tiles into it).
// xs (optional) receives the compensated bf16 planes.
hipError_t launch_quantize(const float *X, void *Xq, const XPlanes *planes, int64_t M, int64_t K, hipStream_t s,
                           float *yz = nullptr, int64_t nz = 0, const XSplit *xs = nullptr);
hipError_t launch_quantize(const float *X, void *Xq, const XPlanes *planes, int64_t M, int64_t K, hipStream_t s,
                           const ZeroList &zl, const XSplit *xs = nullptr);
hipError_t launch_q8_1_convert(const void *Xq, const XPlanes *planes, int64_t M, int64_t K, hipStream_t s,
                              float *yz = nullptr, int64_t nz = 0, const XSplit *xs = nullptr);
hipError_t launch_q8_1_convert(const void *Xq, const XPlanes *planes, int64_t M, int64_t K, hipStream_t s,
                              const ZeroList &zl, const XSplit *xs = nullptr);
hipError_t launch_zero(float *y, int64_t n, hipStream_t s);
hipError_t launch_zero_tiles(const ZeroTiles &zt, hipStream_t s);
hipError_t launch_gemv(const void *W, const XPlanes &x, float *Y, int64_t N, hipStream_t s,
                       int fmt = FMT_IQ4_XS);
// MMQ work split for a shape: TM 32-row subtiles per wavefront, KW
// wavefronts per workgroup and KS workgroups along K.  With KS > 1 the launch
// needs a workspace of workspace_bytes (KS partial [M][N] tiles).
// Streaming matrix-core kernel for M <= 32 (mmv.hip): `grid` workgroups
// (at most one per 32-column tile and per compute unit), result registers
// `live`; zero_y = some tile is shared by two workgroups, which add into a
// zeroed Y.
struct MmvPlan {
    bool ok = false, zero_y = false;
    int grid = 0, live = 0;
    int fmt = FMT_IQ4_XS;
};
MmvPlan mmv_plan(int64_t M, int64_t N, int64_t K, int cus, int fmt = FMT_IQ4_XS);
hipError_t launch_mmv(const void *W, const XPlanes &x, float *Y, int64_t N, const MmvPlan &p,
                      hipStream_t s);
// The same over a group of matrices (one launch; zero_y: every y[g] zeroed).
MmvPlan mmv_plan_group(int64_t M, const int64_t *N, int count, int64_t K, int cus, int fmt = FMT_IQ4_XS);
MmvGroup mmv_group(const void *const *W, float *const *Y, const int64_t *N, int count);
hipError_t launch_mmv_group(const MmvGroup &grp, const XPlanes &x, const MmvPlan &p, hipStream_t s);
// Tile kernel for M > 32 (mmqt.hip): 128 x 128 tiles, runs of (tile, half
// super-block) units over `grid` workgroups; tiles shared by several
// workgroups are summed from a workspace of partial tiles by a second kernel.
struct MmqtPlan {
    bool ok = false, zero_y = false;    // zero_y: shared tiles add into a zeroed Y
    int grid = 0, mblocks = 0, wblocks = 0, bm = 0, bn = 0;   // tile: bm activation rows x bn weight rows
    int64_t tiles = 0;
    int fmt = FMT_IQ4_XS;
    size_t workspace_bytes = 0;         // else partial tiles in a workspace
};
MmqtPlan mmqt_plan(int64_t M, int64_t N, int64_t K, int cus, int fmt = FMT_IQ4_XS);
// The tiles of Y a plan with zero_y needs zeroed (count 0 otherwise).
ZeroTiles mmqt_zero_tiles(const MmqtPlan &p, int64_t M, int64_t N, int64_t K, float *Y);
hipError_t launch_mmqt(const void *W, const XPlanes &x, float *Y, int64_t N, const MmqtPlan &p, void *workspace,
                       hipStream_t s);
struct MmqPlan {
    bool ok = true;            // false: no MMQ kernel takes this shape in this format
    int tm = 1, kw = 1, ks = 1;
    bool mmv = false;          // the streaming kernel runs (M <= 32)
    MmvPlan vp;
    bool tile = false;         // the 128 x 128 tile kernel runs
    MmqtPlan tp;
    bool zero_y = false;       // Y must hold zeros before the launch
    size_t workspace_bytes = 0;
};
// The K-split fallback reads IQ4_XS only: for the other formats a shape
// that neither the streaming nor the tile kernel takes (a weight matrix of
// 2 GiB or more) has no MMQ plan (ok == false).
MmqPlan mmq_plan(int64_t M, int64_t N, int64_t K, int fmt = FMT_IQ4_XS);
// y_zeroed: the caller has already zeroed Y (else the launcher does it when
// the plan needs it).
hipError_t launch_mmq(const void *W, const XPlanes &x, float *Y, int64_t N, void *workspace,
                      bool y_zeroed, hipStream_t s, int fmt = FMT_IQ4_XS);
hipError_t launch_dequant_bf16(const void *W, uint16_t *Wb, int64_t N, int64_t K, hipStream_t s);
// Fused dequantize-in-LDS GEMMs (fused.hip), from the hi/lo planes Xs (an
// XSplit with Ms = fused_ms(M)): the compensated formulation (hi and lo parts,
// three products) and the plain bf16 one (hi parts only, one product).
int64_t fused_grid(int64_t M, int64_t N);
hipError_t launch_fused_x3(const void *W, const uint16_t *Xs, float *Y, int64_t M, int64_t N, int64_t K,
                           hipStream_t s);
int64_t deq_grid(int64_t M, int64_t N);
hipError_t launch_fused_deq(const void *W, const uint16_t *Xs, float *Y, int64_t M, int64_t N, int64_t K,
                            hipStream_t s);

constexpr int GEMV_MAX_M = 4;

// Tuning override, read once: IQ4XS_MMV=0 (do not use the streaming kernel).
struct TuneOverride {
    int mmv = 1;    // IQ4XS_MMV=0: no streaming kernel for M <= 32
    int tile = 1;   // IQ4XS_TILE=0: no 128 x 128 tile kernel for M > 32
};
const TuneOverride &tune_override();

// Compute units of the current device (256 when it cannot be queried).
int device_cus();

}  // namespace iq4xs
