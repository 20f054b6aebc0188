// fused.hip -- dequantize-in-LDS GEMMs on bf16 operands: the compensated
// formulation (k_gemm_x3) and the plain one (k_gemm_deq, further down).
//
// Prior art: "V100TPS engine log" (agent-report.daedalus.work/V100TPS/engine.html),
// M=64 kernel-launch table: a dequantize kernel writes the whole weight in
// fp16 and a dense tensor-core GEMM reads it back, at a cost that does not
// fall with M; "V100TPS MTP investigation", crossover passage: past a few
// dozen rows the dense path wins because the quantized kernel cannot use the
// tensor cores.  Here nothing is written back to HBM: each workgroup expands
// the IQ4_XS sub-block it is about to use straight into LDS.  And so that
// this path meets the integer path's accuracy, every operand is carried as
// two bf16 numbers.
//
// Arithmetic (the oracle's compensated bf16 formulation):
//   W~ = d*(ls-32)*kv is exact in fp32 (11+6+7 significant bits), and so is
//   X~ = d_x*q (11+7).  Each is split into hi = bf16(v) and lo = bf16(v - hi),
//   both nearest even (v - hi is exact in fp32), so hi + lo is v to within
//   2^-16.  Per 32x32 output tile and 16-wide k step, three
//   v_mfma_f32_32x32x16_bf16 accumulate Wh*Xh + Wh*Xl + Wl*Xh in fp32; the
//   Wl*Xl product, below 2^-16 of the term, is dropped.
//
// Work split: a workgroup owns a 256 x 256 tile of Y (rows of X by rows of
// W): eight wavefronts of 128 x 64 (4 x 2 MFMA tiles, two wavefronts per
// SIMD), or four of 128 x 128 (one per SIMD, 256 accumulators each; selectable for
// measurement).  K is walked one 32-weight sub-block at a time through two
// LDS stages: the activation tile (256 rows of {hi[32], lo[32]}, written by
// the quantizer in that layout) is loaded straight into LDS by buffer loads,
// and the weight tile (256 columns) is expanded from its index bytes and its
// scale by one or two threads per column.  The loads of sub-block s+1 (and
// the weight loads of s+2) are issued before the matrix-core work on
// sub-block s and the expansion of s+1 goes to the other stage, so one
// barrier per sub-block suffices.
//
// Workgroups are numbered so that the M-tiles of one N-tile run one after the
// other on the same XCD (workgroup g goes to XCD g mod 8): the weight tile
// they share is then read from HBM once into that XCD's L2.
#include "common.hpp"
#include "stream.hpp"

#include <cstdlib>

namespace iq4xs {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // (HIP's uint4 copies as a memcpy)
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int WROW = 72;   // u16 per weight column in LDS: hi[32], lo[32], 8 of padding
static_assert(WROW * 2 % 16 == 0, "LDS columns stay 16-byte aligned");

// Tile configuration: TM x TN MFMA tiles per wavefront, WM x WN wavefronts
// per workgroup.
template <int TM_, int TN_, int WM_, int WN_>
struct XCfg {
    static constexpr int TM = TM_, TN = TN_, WM = WM_, WN = WN_;
    static constexpr int BM = 32 * TM * WM;              // rows of X per workgroup
    static constexpr int BN = 32 * TN * WN;              // rows of W per workgroup
    static constexpr int NT = 64 * WM * WN;              // threads
    static constexpr int TPC = NT / BN;                  // threads per weight column (1 or 2)
    static constexpr int XBYTES = BM * 128;              // activation tile: hi[32], lo[32] per row
    static constexpr int STAGE = XBYTES + BN * WROW * 2; // bytes per LDS stage
    static constexpr int XLOADS = XBYTES / 1024 / (WM * WN);   // 1 KB LDS-direct loads per wavefront
    static_assert(TPC == 1 || TPC == 2, "one or two threads per weight column");
    static_assert(TPC * BN == NT, "every thread expands part of one column");
    static_assert(XLOADS * 1024 * WM * WN == XBYTES && XLOADS >= 1, "activation tile in whole loads");
    static_assert(FUSED_ROWS % BM == 0, "activation planes are padded to whole workgroup tiles");
    static_assert(2 * STAGE <= 160 * 1024, "two LDS stages fit one compute unit");
};
// 4 wavefronts of 128 x 128 (one per SIMD, 256 accumulators each), or 8 of
// 128 x 64 (two per SIMD: one wavefront's expansion runs beside the other's
// matrix-core work).
using X3Big = XCfg<4, 4, 2, 2>;
using X3Pair = XCfg<4, 2, 2, 4>;

// kvalues_iq4nl + 128 (bytes 1..241), so that a byte converts to fp32 in one
// instruction and the bias is folded into the scaling FMA.
constexpr uint32_t KB0 = KV0 ^ 0x80808080u, KB1 = KV1 ^ 0x80808080u;
constexpr uint32_t KB2 = KV2 ^ 0x80808080u, KB3 = KV3 ^ 0x80808080u;

// Four 4-bit indices (bits 0-3 of each byte of t) -> four biased values.
// Same byte-permute lookup as lut4 in common.hpp, v_bfi for the select.
__device__ __forceinline__ uint32_t lut4_biased(uint32_t t)
{
    const uint32_t s = t & 0x07070707u;
    const uint32_t a = __builtin_amdgcn_perm(KB1, KB0, s);
    const uint32_t b = __builtin_amdgcn_perm(KB3, KB2, s);
    const uint32_t m = __builtin_amdgcn_perm(0u, 0u, (t & 0x08080808u) | 0x05050505u);
    return (m & b) | (~m & a);
}

// Four biased values (the bytes of u) of a sub-block with scale sw ->
// hi and lo bf16 pairs of the weights (kv*sw: the FMA with c = -128*sw is
// exact because the result is representable).
__device__ __forceinline__ void expand4(uint32_t u, float sw, float c, uint32_t &h0, uint32_t &h1, uint32_t &l0,
                                        uint32_t &l1)
{
    const float w0 = fmaf((float)(u & 0xFFu), sw, c);
    const float w1 = fmaf((float)((u >> 8) & 0xFFu), sw, c);
    const float w2 = fmaf((float)((u >> 16) & 0xFFu), sw, c);
    const float w3 = fmaf((float)(u >> 24), sw, c);
    bf16x2_split(w0, w1, h0, l0);
    bf16x2_split(w2, w3, h1, l1);
}

// Eight weights from the indices in bits 0-3 of the bytes of qa, qb ->
// hi at dst[0..7], lo at dst[32..39].
__device__ __forceinline__ void expand8_x3(uint32_t qa, uint32_t qb, float sw, float c, uint16_t *dst)
{
    uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
    expand4(lut4_biased(qa), sw, c, h0, h1, l0, l1);
    expand4(lut4_biased(qb), sw, c, h2, h3, l2, l3);
    *reinterpret_cast<u32x4 *>(dst) = u32x4{h0, h1, h2, h3};
    *reinterpret_cast<u32x4 *>(dst + 32) = u32x4{l0, l1, l2, l3};
}

// As expand8_x3 with the hi parts only (the plain bf16 formulation).
__device__ __forceinline__ void expand8_hi(uint32_t qa, uint32_t qb, float sw, float c, uint16_t *dst)
{
    const uint32_t ua = lut4_biased(qa), ub = lut4_biased(qb);
    const bf16x2_t h0 = {(__bf16)fmaf((float)(ua & 0xFFu), sw, c), (__bf16)fmaf((float)((ua >> 8) & 0xFFu), sw, c)};
    const bf16x2_t h1 = {(__bf16)fmaf((float)((ua >> 16) & 0xFFu), sw, c), (__bf16)fmaf((float)(ua >> 24), sw, c)};
    const bf16x2_t h2 = {(__bf16)fmaf((float)(ub & 0xFFu), sw, c), (__bf16)fmaf((float)((ub >> 8) & 0xFFu), sw, c)};
    const bf16x2_t h3 = {(__bf16)fmaf((float)((ub >> 16) & 0xFFu), sw, c), (__bf16)fmaf((float)(ub >> 24), sw, c)};
    *reinterpret_cast<u32x4 *>(dst) = u32x4{__builtin_bit_cast(uint32_t, h0), __builtin_bit_cast(uint32_t, h1),
                                            __builtin_bit_cast(uint32_t, h2), __builtin_bit_cast(uint32_t, h3)};
}

// A thread's share of its weight column for one sub-block: 16 index bytes
// (or 8, with two threads per column) and the super-block header.
struct WStage {
    u32x2 q0, q1, hdr;
};

template <class C>
__device__ __forceinline__ void load_w(WStage &st, const char *__restrict__ wrow, int s, int part)
{
    const char *u = wrow + (int64_t)(s / SUBS) * WBLK;
    st.hdr = *reinterpret_cast<const u32x2 *>(u);
    if constexpr (C::TPC == 1) {
        st.q0 = *reinterpret_cast<const u32x2 *>(u + QS_OFF + 16 * (s % SUBS));
        st.q1 = *reinterpret_cast<const u32x2 *>(u + QS_OFF + 16 * (s % SUBS) + 8);
    } else {
        st.q0 = *reinterpret_cast<const u32x2 *>(u + QS_OFF + 16 * (s % SUBS) + 8 * part);
    }
}

// Expands the thread's share of its column into the weight area of an LDS
// stage: index bytes 8h..8h+7 hold elements 8h..8h+7 (low nibbles) and
// 16+8h..16+8h+7 (high nibbles).
template <class C>
__device__ __forceinline__ void store_w(const WStage &st, uint16_t *__restrict__ lw, int s, int colidx, int part)
{
    const float sw = sub_scale(st.hdr.x, st.hdr.y, s % SUBS);
    const float c = -128.0f * sw;
    uint16_t *col = lw + colidx * WROW;
    if constexpr (C::TPC == 1) {
        expand8_x3(st.q0.x, st.q0.y, sw, c, col);
        expand8_x3(st.q1.x, st.q1.y, sw, c, col + 8);
        expand8_x3(st.q0.x >> 4, st.q0.y >> 4, sw, c, col + 16);
        expand8_x3(st.q1.x >> 4, st.q1.y >> 4, sw, c, col + 24);
    } else {
        expand8_x3(st.q0.x, st.q0.y, sw, c, col + 8 * part);
        expand8_x3(st.q0.x >> 4, st.q0.y >> 4, sw, c, col + 16 + 8 * part);
    }
}

// Slot of an activation row's 16-byte piece in LDS: slot p' of row r holds
// piece p' ^ swz(r) (hi pieces 0-3, lo pieces 4-7), swz(r) from bits 0-3 of
// r only.  The operand reads of 8 consecutive rows (16-row aligned groups)
// then hit 8 different 16-byte bank groups of a 128-byte line, and those of
// 16 consecutive rows 16 different groups of a 256-byte line: conflict-free
// whether the LDS serves 128 or 256 bytes per clock.
__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// The activation tile of sub-block s into an LDS stage: wavefront w's load t
// fills LDS bytes [(L*w+t)*1024, +1024) (L loads per wavefront), lane i its
// 16 bytes at 16*i, i.e. slot i%8 of tile row 8*(L*w+t) + i/8.
template <class C>
__device__ __forceinline__ void load_x(__amdgpu_buffer_rsrc_t xr, char *lx, uint32_t row_off, int wave, int lane)
{
#pragma unroll
    for (int t = 0; t < C::XLOADS; t++) {
        const int r = 8 * (C::XLOADS * wave + t) + (lane >> 3);
        const int p = (lane & 7) ^ swz(r);
        stream::load_lds16(xr, lx + 1024 * (C::XLOADS * wave + t), row_off + (uint32_t)(r * 128 + 16 * p));
    }
}

__device__ __forceinline__ v8bf lds_bf8(const void *p)
{
    return __builtin_bit_cast(v8bf, *reinterpret_cast<const u32x4 *>(p));
}

struct Ctx {
    __amdgpu_buffer_rsrc_t xr;
    const char *wrow;
    uint32_t x0;          // byte offset of the workgroup's first activation row in sub-block 0
    uint32_t xstep;       // bytes between consecutive sub-blocks of the activation planes
    int S, wave, lane, colidx, part, lx_off, lw_off;
};

// The MFMAs of one sub-block from an LDS stage: per 16-wide k half, the
// wavefront's TN weight operands (hi, lo) and TM activation operands (hi, lo),
// three products per tile.
template <class C>
__device__ __forceinline__ void mfmas(v16f (&acc)[C::TM][C::TN], const char *cur, const Ctx &cx)
{
    const char *lx = cur + cx.lx_off;
    const char *lw = cur + C::XBYTES + cx.lw_off;
    const int h = cx.lane >> 5, sw = swz(cx.lane & 31);
#pragma unroll
    for (int c = 0; c < 2; c++) {
        v8bf bh[C::TN], bl[C::TN];
#pragma unroll
        for (int j = 0; j < C::TN; j++) {
            bh[j] = lds_bf8(lw + 64 * j * WROW + 32 * c);
            bl[j] = lds_bf8(lw + 64 * j * WROW + 32 * c + 64);
        }
#pragma unroll
        for (int i = 0; i < C::TM; i++) {
            // hi piece 2c+h and lo piece 4+2c+h of row 32i + col (swz of the
            // row is swz(col): the tile offsets are multiples of 32)
            const v8bf ah = lds_bf8(lx + 32 * i * 128 + 16 * ((2 * c + h) ^ sw));
#pragma unroll
            for (int j = 0; j < C::TN; j++)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh[j], acc[i][j], 0, 0, 0);
            const v8bf al = lds_bf8(lx + 32 * i * 128 + 16 * ((4 + 2 * c + h) ^ sw));
#pragma unroll
            for (int j = 0; j < C::TN; j++)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bl[j], acc[i][j], 0, 0, 0);
#pragma unroll
            for (int j = 0; j < C::TN; j++)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, bh[j], acc[i][j], 0, 0, 0);
        }
    }
}

// One sub-block step: the activation tile of sub-block s+1 goes straight
// into the LDS stage `nxt`; the weight loads of sub-block s+2 go to
// `loading`; the MFMAs of sub-block s run from the stage `cur` and the
// weights of sub-block s+1 (`ready`, loaded one step earlier) are expanded
// into `nxt` (the compiler interleaves the two).  Indices past the last
// sub-block are clamped: what they load and expand is never read.
template <class C>
__device__ __forceinline__ void step(v16f (&acc)[C::TM][C::TN], const char *cur, char *nxt, const WStage &ready,
                                     WStage &loading, int s, const Ctx &cx)
{
    const int s1 = s + 1 < cx.S ? s + 1 : cx.S - 1;
    const int s2 = s + 2 < cx.S ? s + 2 : cx.S - 1;
    load_x<C>(cx.xr, nxt, cx.x0 + (uint32_t)s1 * cx.xstep, cx.wave, cx.lane);
    load_w<C>(loading, cx.wrow, s2, cx.part);
    mfmas<C>(acc, cur, cx);
    store_w<C>(ready, reinterpret_cast<uint16_t *>(nxt + C::XBYTES), s1, cx.colidx, cx.part);
    // this wavefront's activation loads and LDS writes are done (and its
    // weight loads, issued at the same time); the barrier makes them everyone's
    __builtin_amdgcn_s_waitcnt(stream::wait_vm_lds(0));
    stream::raw_barrier();
}

// Xs: the quantizer's hi/lo planes, [K/32][Ms][64] bf16 (Ms = M rounded up to
// FUSED_ROWS; rows M..Ms-1 are zero), fewer than 2^31 bytes.  W: [N][K/256]
// IQ4_XS super-blocks.
template <class C>
__global__ void __launch_bounds__(C::NT, 1)
k_gemm_x3(const char *__restrict__ W, const uint16_t *__restrict__ Xs, float *__restrict__ Y, int64_t M,
          int64_t N, int64_t K, int64_t Ms)
{
    __shared__ __attribute__((aligned(16))) char lds[2 * C::STAGE];
    const int tid = threadIdx.x;
    const int64_t nbm = (M + C::BM - 1) / C::BM, nbn = (N + C::BN - 1) / C::BN;
    const int64_t g = blockIdx.x;
    const int64_t nb = (g / 8) / nbm * 8 + (g % 8), mb = (g / 8) % nbm;
    if (nb >= nbn)
        return;                                     // whole workgroup
    const int64_t m0 = mb * C::BM, n0 = nb * C::BN;

    Ctx cx;
    cx.S = (int)(K / SB);                           // a multiple of 8
    cx.xr = __builtin_amdgcn_make_buffer_rsrc((void *)Xs, (short)0, (int)(cx.S * Ms * 128), stream::BUFFER_FLAGS);
    cx.x0 = (uint32_t)(m0 * 128);
    cx.xstep = (uint32_t)(Ms * 128);
    // with two threads per column, the halves of the workgroup take the two
    // halves of the columns (consecutive lanes write consecutive columns)
    cx.colidx = tid % C::BN;
    cx.part = tid / C::BN;
    const int64_t wn_row = n0 + cx.colidx < N ? n0 + cx.colidx : N - 1;   // columns past N repeat row N-1
    cx.wrow = W + wn_row * (K / QK) * WBLK;
    cx.lane = tid & 63;
    cx.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = cx.wave / C::WN, wn = cx.wave % C::WN;
    const int col = cx.lane & 31, h = cx.lane >> 5;
    cx.lx_off = (32 * C::TM * wm + col) * 128;
    cx.lw_off = ((32 * C::TN * wn + col) * WROW + 8 * h) * 2;

    v16f acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; i++)
#pragma unroll
        for (int j = 0; j < C::TN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                acc[i][j][r] = 0.0f;

    WStage wa, wb;
    load_x<C>(cx.xr, lds, cx.x0, cx.wave, cx.lane);
    load_w<C>(wa, cx.wrow, 0, cx.part);
    store_w<C>(wa, reinterpret_cast<uint16_t *>(lds + C::XBYTES), 0, cx.colidx, cx.part);
    load_w<C>(wa, cx.wrow, 1, cx.part);
    __builtin_amdgcn_s_waitcnt(stream::wait_vm_lds(0));
    stream::raw_barrier();
    // two steps per trip, so that the two LDS stages are fixed offsets
    for (int s = 0; s < cx.S; s += 2) {
        step<C>(acc, lds, lds + C::STAGE, wa, wb, s, cx);
        step<C>(acc, lds + C::STAGE, lds, wb, wa, s + 1, cx);
    }

    // lane (col, h) of tile (i, j) holds Y[m][n] for n = its column and
    // m = 8*(r/4) + 4*h + r%4, r = 0..15
#pragma unroll
    for (int j = 0; j < C::TN; j++) {
        const int64_t n = n0 + 32 * C::TN * wn + 32 * j + col;
        if (n >= N)
            continue;
#pragma unroll
        for (int i = 0; i < C::TM; i++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int64_t m = m0 + 32 * C::TM * wm + 32 * i + 8 * (r / 4) + 4 * h + (r % 4);
                if (m < M)
                    Y[m * N + n] = acc[i][j][r];
            }
    }
}

// ---------------------------------------------------------------------------
// The plain bf16 formulation (the pages' dequantize-then-GEMM arithmetic):
// W~ and X~ each rounded once to bf16, one MFMA per 32x32 tile and 16-wide k
// step.  Same tiles as the compensated kernel (256 x 256 of Y, eight
// wavefronts of 128 x 64, two threads per weight column), but a third of its
// matrix-core work and a sixth of its weight expansion per output, so what
// bounds it is getting the operands in.  Every load is a 16-byte
// LDS-writing buffer load, a lane per 16 contiguous bytes:
//  * the activation hi parts of sub-block s+2 during step s, into one of
//    three stages (64-byte rows, 16-byte pieces swizzled by swz2);
//  * the raw weights one half super-block ahead, into one of two stages: for
//    each column of the tile, bytes [0,16) of its super-block (the header)
//    and the half's 64 index bytes, an 80-byte LDS row, so that a row is
//    read in five contiguous pieces instead of a lane per column;
//  * during step s the expansion of sub-block s+1 reads the raw stage and
//    writes one of two expanded stages.
// At the end of a step a wavefront waits for all but the loads it issued in
// that step (every wavefront issues the same number: slots without a job
// load nothing into a dump area), then one barrier.
template <int TM_, int TN_, int WM_, int WN_>
struct DCfg {
    static constexpr int TM = TM_, TN = TN_, WM = WM_, WN = WN_;
    static constexpr int BM = 32 * TM * WM;              // rows of X per workgroup
    static constexpr int BN = 32 * TN * WN;              // rows of W per workgroup
    static constexpr int NWAVE = WM * WN, NT = 64 * NWAVE;
    static constexpr int TPC = NT / BN;                  // threads per weight column
    static constexpr int WROWD = 40;                     // u16 per expanded column: hi[32], 8 of padding
    static constexpr int RAWROW = 80;                    // bytes per raw weight row (header piece + 64)
    static constexpr int XBYTES = BM * 64, WBYTES = BN * WROWD * 2, RBYTES = BN * RAWROW;
    static constexpr int XOFF = 0, WOFF = 3 * XBYTES, ROFF = WOFF + 2 * WBYTES, DUMP = ROFF + 2 * RBYTES;
    static constexpr int LDS = DUMP + 1024;
    static constexpr int XL = XBYTES / 1024 / NWAVE;     // activation loads per wavefront and step
    static constexpr int RJ = RBYTES / 1024;             // 1 KB raw weight jobs per half
    static constexpr int RL = (RJ + NWAVE - 1) / NWAVE;  // raw weight loads per wavefront and half
    static_assert(TPC == 2 && TPC * BN == NT, "two threads per weight column");
    static_assert(XL * 1024 * NWAVE == XBYTES && XL >= 1, "activation tile in whole loads");
    static_assert(RBYTES % 1024 == 0, "raw weight stage in whole loads");
    static_assert(FUSED_ROWS % BM == 0, "activation planes are padded to whole workgroup tiles");
    static_assert(LDS <= 160 * 1024, "the stages fit one compute unit");
};
using DPair = DCfg<4, 2, 2, 4>;

// Slot of an activation row's 16-byte hi piece (p = 0..3) in LDS: p ^ swz2(r),
// so that the 16 rows one operand read covers land in 16 different 16-byte
// bank groups of a 256-byte line.
__device__ __forceinline__ int swz2(int r) { return (r >> 2) & 3; }

template <class C>
struct DCtx {
    __amdgpu_buffer_rsrc_t xr, wr;
    uint32_t x0, xstep;           // plane bytes: the tile's first row, between sub-blocks
    uint32_t rgo[2][C::RL];       // raw weight slots: this lane's offset for half 0 / 1 (OOB: no job)
    int rdst[C::RL];              // and the LDS offset its load fills within a raw stage
    int S, wave, lane, colidx, part, lx_off, lw_off;
};

// The activation hi parts of sub-block s into stage xs: load t of wavefront
// w fills 1 KB = 16 rows; lane i takes piece (i%4) ^ swz2(row) of row i/4.
template <class C>
__device__ __forceinline__ void load_xd(char *lds, int xs, int s, const DCtx<C> &cx)
{
#pragma unroll
    for (int t = 0; t < C::XL; t++) {
        const int chunk = C::XL * cx.wave + t;
        const int r = 16 * chunk + (cx.lane >> 2);
        const int p = (cx.lane & 3) ^ swz2(r);
        stream::load_lds16(cx.xr, lds + C::XOFF + xs * C::XBYTES + 1024 * chunk,
                           cx.x0 + (uint32_t)s * cx.xstep + (uint32_t)(r * 128 + 16 * p));
    }
}

// The raw weights of half hh (sub-blocks 4hh..4hh+3) into raw stage rs.
template <class C>
__device__ __forceinline__ void load_wd(char *lds, int rs, int hh, const DCtx<C> &cx)
{
    const uint32_t base = (uint32_t)(hh >> 1) * WBLK;
#pragma unroll
    for (int k = 0; k < C::RL; k++) {
        const uint32_t go = (hh & 1) ? cx.rgo[1][k] : cx.rgo[0][k];   // (no dynamic index: registers)
        const int dst = cx.rdst[k] < 0 ? C::DUMP : C::ROFF + rs * C::RBYTES + cx.rdst[k];
        stream::load_lds16(cx.wr, lds + dst, go == stream::OOB ? go : go + base);
    }
}

// Expands sub-block s (raw stage of its half) into expanded stage ws: the
// thread's 8 index bytes of its column, low and high nibbles.
template <class C>
__device__ __forceinline__ void expand_d(char *lds, int ws, int s, const DCtx<C> &cx)
{
    const char *raw = lds + C::ROFF + ((s >> 2) & 1) * C::RBYTES + cx.colidx * C::RAWROW;
    const u32x2 hdr = *reinterpret_cast<const u32x2 *>(raw);
    const u32x2 q = *reinterpret_cast<const u32x2 *>(raw + 16 + 16 * (s & 3) + 8 * cx.part);
    const float sw = sub_scale(hdr.x, hdr.y, s % SUBS);
    uint16_t *col = reinterpret_cast<uint16_t *>(lds + C::WOFF + ws * C::WBYTES) + cx.colidx * C::WROWD + 8 * cx.part;
    expand8_hi(q.x, q.y, sw, -128.0f * sw, col);
    expand8_hi(q.x >> 4, q.y >> 4, sw, -128.0f * sw, col + 16);
}

template <class C>
__device__ __forceinline__ void mfmas_d(v16f (&acc)[C::TM][C::TN], const char *lds, int xs, int ws,
                                        const DCtx<C> &cx)
{
    const char *lx = lds + C::XOFF + xs * C::XBYTES + cx.lx_off;
    const char *lw = lds + C::WOFF + ws * C::WBYTES + cx.lw_off;
    const int h = cx.lane >> 5, sz = swz2(cx.lane & 31);
#pragma unroll
    for (int c = 0; c < 2; c++) {
        v8bf bh[C::TN];
#pragma unroll
        for (int j = 0; j < C::TN; j++)
            bh[j] = lds_bf8(lw + 64 * j * C::WROWD + 32 * c);
#pragma unroll
        for (int i = 0; i < C::TM; i++) {
            // (swz2 of row 32i + col is swz2(col): the tile offsets are multiples of 32)
            const v8bf ah = lds_bf8(lx + 32 * i * 64 + 16 * ((2 * c + h) ^ sz));
#pragma unroll
            for (int j = 0; j < C::TN; j++)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, bh[j], acc[i][j], 0, 0, 0);
        }
    }
}

// Xs: the quantizer's hi/lo planes, [K/32][Ms][64] bf16 (Ms = M rounded up
// to FUSED_ROWS; rows M..Ms-1 are zero), fewer than 2^31 bytes; the hi parts
// are read.  W: [N][K/256] IQ4_XS super-blocks; the workgroup's 256 rows
// (fewer than 2^31 bytes) through a buffer descriptor of their own.
template <class C>
__global__ void __launch_bounds__(C::NT, 1)
k_gemm_deq(const char *__restrict__ W, const uint16_t *__restrict__ Xs, float *__restrict__ Y, int64_t M,
           int64_t N, int64_t K, int64_t Ms)
{
    __shared__ __attribute__((aligned(16))) char lds[C::LDS];
    const int tid = threadIdx.x;
    const int64_t nbm = (M + C::BM - 1) / C::BM, nbn = (N + C::BN - 1) / C::BN;
    const int64_t g = blockIdx.x;
    const int64_t nb = (g / 8) / nbm * 8 + (g % 8), mb = (g / 8) % nbm;
    if (nb >= nbn)
        return;                                     // whole workgroup
    const int64_t m0 = mb * C::BM, n0 = nb * C::BN;
    const int rows = (int)(N - n0 < C::BN ? N - n0 : C::BN);
    const uint32_t row_bytes = (uint32_t)(K / QK) * WBLK;

    DCtx<C> cx;
    cx.S = (int)(K / SB);
    cx.xr = __builtin_amdgcn_make_buffer_rsrc((void *)Xs, (short)0, (int)(cx.S * Ms * 128), stream::BUFFER_FLAGS);
    cx.wr = __builtin_amdgcn_make_buffer_rsrc((void *)(W + n0 * (int64_t)row_bytes), (short)0,
                                              (int)((uint32_t)rows * row_bytes), stream::BUFFER_FLAGS);
    cx.x0 = (uint32_t)(m0 * 128);
    cx.xstep = (uint32_t)(Ms * 128);
    cx.colidx = tid % C::BN;
    cx.part = tid / C::BN;
    cx.lane = tid & 63;
    cx.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // raw weight slot k of this wavefront: 1 KB job wave*RL + k covers LDS
    // bytes [1024 job, +1024) of a raw stage: lane i its 16 bytes at 16 i,
    // piece pc of row r (rows past the matrix repeat its last row); piece 0
    // is super-block bytes [0,16), pieces 1-4 the half's index bytes
#pragma unroll
    for (int k = 0; k < C::RL; k++) {
        const int job = C::RL * cx.wave + k;
        if (job < C::RJ) {
            const int at = 1024 * job + 16 * cx.lane;
            const int r = at / C::RAWROW, pc = (at - r * C::RAWROW) / 16;
            const uint32_t rb = (uint32_t)(r < rows ? r : rows - 1) * row_bytes;
            cx.rgo[0][k] = rb + (pc == 0 ? 0u : (uint32_t)(16 * pc - 8));
            cx.rgo[1][k] = rb + (pc == 0 ? 0u : (uint32_t)(16 * pc + 56));
            cx.rdst[k] = 1024 * job;
        } else {
            cx.rgo[0][k] = cx.rgo[1][k] = stream::OOB;
            cx.rdst[k] = -1;
        }
    }
    const int wm = cx.wave / C::WN, wn = cx.wave % C::WN;
    const int col = cx.lane & 31, h = cx.lane >> 5;
    cx.lx_off = (32 * C::TM * wm + col) * 64;
    cx.lw_off = ((32 * C::TN * wn + col) * C::WROWD + 8 * h) * 2;

    v16f acc[C::TM][C::TN];
#pragma unroll
    for (int i = 0; i < C::TM; i++)
#pragma unroll
        for (int j = 0; j < C::TN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                acc[i][j][r] = 0.0f;

    const int S = cx.S, H = S / 4;                  // S is a multiple of 8
    load_wd<C>(lds, 0, 0, cx);
    load_xd<C>(lds, 0, 0, cx);
    load_xd<C>(lds, 1, 1, cx);
    __builtin_amdgcn_s_waitcnt(stream::wait_vm_lds(C::XL));
    stream::raw_barrier();
    expand_d<C>(lds, 0, 0, cx);
    __builtin_amdgcn_s_waitcnt(stream::WAIT_LDS);
    stream::raw_barrier();
    int xs = 0;                                     // activation stage of sub-block s (s mod 3)
    for (int s = 0; s < S; s++) {
        const int xn = xs == 0 ? 2 : xs - 1;        // stage of s+2
        load_xd<C>(lds, xn, s + 2 < S ? s + 2 : S - 1, cx);
        const bool half_start = (s & 3) == 0;
        if (half_start) {
            const int hh = (s >> 2) + 1;
            load_wd<C>(lds, hh & 1, hh < H ? hh : H - 1, cx);
        }
        mfmas_d<C>(acc, lds, xs, s & 1, cx);
        expand_d<C>(lds, (s + 1) & 1, s + 1 < S ? s + 1 : S - 1, cx);
        // all but this step's loads have landed, and this wavefront's LDS
        // writes are done; the barrier makes them everyone's
        if (half_start)
            __builtin_amdgcn_s_waitcnt(stream::wait_vm_lds(C::XL + C::RL));
        else
            __builtin_amdgcn_s_waitcnt(stream::wait_vm_lds(C::XL));
        stream::raw_barrier();
        xs = xs == 2 ? 0 : xs + 1;
    }
    __builtin_amdgcn_s_waitcnt(stream::wait_vm_lds(0));

    // lane (col, h) of tile (i, j) holds Y[m][n] for n = its column and
    // m = 8*(r/4) + 4*h + r%4, r = 0..15
#pragma unroll
    for (int j = 0; j < C::TN; j++) {
        const int64_t n = n0 + 32 * C::TN * wn + 32 * j + col;
        if (n >= N)
            continue;
#pragma unroll
        for (int i = 0; i < C::TM; i++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int64_t m = m0 + 32 * C::TM * wm + 32 * i + 8 * (r / 4) + 4 * h + (r % 4);
                if (m < M)
                    Y[m * N + n] = acc[i][j][r];
            }
    }
}

// Which configuration a shape runs (IQ4XS_X3CFG=0 / 1 forces one; for
// measurements).
int x3_config()
{
    static const int forced = [] {
        const char *v = getenv("IQ4XS_X3CFG");
        return v && (v[0] == '0' || v[0] == '1') ? v[0] - '0' : -1;
    }();
    return forced >= 0 ? forced : 1;
}

template <class C>
int64_t grid_of(int64_t M, int64_t N)
{
    const int64_t nbm = (M + C::BM - 1) / C::BM, nbn = (N + C::BN - 1) / C::BN;
    return (nbn + 7) / 8 * 8 * nbm;
}

}  // namespace

int64_t fused_grid(int64_t M, int64_t N)
{
    return x3_config() == 0 ? grid_of<X3Big>(M, N) : grid_of<X3Pair>(M, N);
}

hipError_t launch_fused_x3(const void *W, const uint16_t *Xs, float *Y, int64_t M, int64_t N, int64_t K,
                           hipStream_t s)
{
    const int64_t Ms = fused_ms(M);
    const char *w = (const char *)W;
    if (x3_config() == 0)
        hipLaunchKernelGGL((k_gemm_x3<X3Big>), dim3((unsigned)grid_of<X3Big>(M, N)), dim3(X3Big::NT), 0, s, w, Xs,
                           Y, M, N, K, Ms);
    else
        hipLaunchKernelGGL((k_gemm_x3<X3Pair>), dim3((unsigned)grid_of<X3Pair>(M, N)), dim3(X3Pair::NT), 0, s, w,
                           Xs, Y, M, N, K, Ms);
    return hipGetLastError();
}

int64_t deq_grid(int64_t M, int64_t N) { return grid_of<DPair>(M, N); }

hipError_t launch_fused_deq(const void *W, const uint16_t *Xs, float *Y, int64_t M, int64_t N, int64_t K,
                            hipStream_t s)
{
    hipLaunchKernelGGL((k_gemm_deq<DPair>), dim3((unsigned)grid_of<DPair>(M, N)), dim3(DPair::NT), 0, s,
                       (const char *)W, Xs, Y, M, N, K, fused_ms(M));
    return hipGetLastError();
}

}  // namespace iq4xs
