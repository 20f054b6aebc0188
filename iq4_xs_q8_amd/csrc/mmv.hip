// mmv.hip -- IQ4_XS x Q8_1 on the int8 matrix cores for a few activation rows
// (M <= 32), streaming the weights once at close to HBM speed.
//
// Arithmetic (batched IQ4_XS kernel section of the "V100TPS engine log",
// agent-report.daedalus.work/V100TPS/engine.html): per 32-element sub-block the
// exact integer dot of the int8 codebook values with the int8 activations,
// here one v_mfma_i32_32x32x32_i8 for a 32-column x 32-row tile, then
// y += d_w*(ls-32) * d_x * dot in fp32.
//
// Work split:
//  * The weights are cut into units (32-column tile t, super-block j), ordered
//    tile-major, and every workgroup gets one contiguous run of units of equal
//    length.  The grid never has more workgroups than tiles, so a run covers at
//    least one tile's worth of units and a tile is shared by at most two
//    workgroups: every compute unit gets the same work whatever the shape.
//  * A run is walked in chunks of up to CH super-blocks of one tile, chunk
//    windows starting at even super-blocks (with K/256 even, every window is
//    16-byte aligned and ends inside its row).  A chunk's weights (32 rows x up
//    to CH*136 contiguous bytes per row) and the activations of its sub-blocks
//    (one contiguous range of the sub-block-major planes) are copied to LDS
//    with 16-byte loads that follow the memory layout, so every HBM access is
//    a long contiguous run.  Two register sets carry the copies of the next
//    two chunks while the current one is computed.
//  * Sixteen wavefronts: wavefront w computes sub-block w%8 of the chunk's
//    super-blocks w/8, w/8+2, ... from LDS (the 8 index bytes and header of its
//    lane's row, the 16 activation bytes of its lane's row; rows past M read a
//    zero row).  The chunk is computed without branches: a super-block past
//    the chunk's end reads bytes that are zero in LDS (their header gives
//    scale 0).
//  * When a tile's units end, the wavefronts' partial tiles are summed in LDS
//    in wavefront order.  A tile owned by one workgroup is stored; a tile
//    shared by two is added into Y with one atomic add per element, Y having
//    been zeroed beforehand: 0 + a + b == 0 + b + a in floating point, so the
//    result does not depend on which workgroup comes first.
#include "common.hpp"

#include <type_traits>

namespace iq4xs {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int TILE = 32;
constexpr int NW = 16;                     // wavefronts per workgroup
constexpr int NT = 64 * NW;                // threads per workgroup
constexpr int PAR = NW / SUBS;             // wavefronts per sub-block
constexpr int BUFFER_FLAGS = 0x00020000;   // raw buffer resource, gfx9 family
constexpr uint32_t OOB = 0x80000000u;      // buffer offset past every range: loads return 0

// LDS row stride of a weight chunk: room for CH+1 super-blocks (the last one
// stays zero: the slot a wavefront reads when a chunk starts at an odd
// super-block), rounded up to an odd number of 16-byte units so that the 32
// rows of an MFMA operand read spread over the banks.
constexpr int wrow_bytes(int ch)
{
    const int u = ((ch + 1) * WBLK + 15) / 16;
    return 16 * (u % 2 ? u : u + 1);
}

template <int LIVE>
struct Shape {
    static constexpr int CH = LIVE <= 4 ? 8 : LIVE == 8 ? 4 : 2;           // super-blocks per chunk
    static constexpr int MP_MAX = LIVE <= 4 ? 8 : LIVE == 8 ? 16 : 32;     // padded rows served
};

template <int LIVE>
struct Layout {
    static constexpr int CH = Shape<LIVE>::CH, MP_MAX = Shape<LIVE>::MP_MAX;
    static_assert(CH % PAR == 0, "every wavefront gets the same number of super-blocks");
    static constexpr int WROW = wrow_bytes(CH);
    // one chunk buffer: weights [32][WROW], activations [CH*8][Mp][32], a
    // 32-byte zero row (the operand of rows >= M), scales [CH*8][Mp] (+ slack
    // for the rows a lane reads past Mp)
    static constexpr int W_BYTES = TILE * WROW;
    static constexpr int A_BYTES = CH * SUBS * MP_MAX * SB;
    static constexpr int Z_OFF = W_BYTES + A_BYTES;
    static constexpr int D_OFF = Z_OFF + 32;
    static constexpr int D_BYTES = (CH + 1) * SUBS * MP_MAX * 4 + 32 * 4;
    static constexpr int BUF = D_OFF + D_BYTES;
    static constexpr int RED = NW * LIVE * 64 * 4;                            // partial tiles
    static constexpr int SINK = 2 * BUF + RED;                                // 64 x 16 bytes
    static constexpr int TOTAL = SINK + 64 * 16;
    // 16-byte pieces a thread copies per chunk: weights, then one activation
    // piece and one scale piece
    static constexpr int W_PR = CH * WBLK / 16;                               // pieces per row
    static constexpr int W_PIECES = TILE * W_PR;
    static constexpr int W_LOADS = (W_PIECES + NT - 1) / NT;
    static_assert(CH * WBLK % 16 == 0, "whole 16-byte pieces per row");
    static_assert(CH * SUBS * MP_MAX * SB / 16 <= NT && CH * SUBS * MP_MAX * 4 / 16 <= NT,
                  "one activation piece and one scale piece per thread");
    static_assert(TOTAL <= 160 * 1024 && TOTAL % 16 == 0 && BUF % 16 == 0, "LDS budget");
};

// Result register r of lane (col, h) holds row 8*(r/4) + 4*h + r%4.
template <int LIVE>
__device__ __forceinline__ void epilogue(const v16i &D, float sw, const float4 *dx, float acc[LIVE])
{
#pragma unroll
    for (int r = 0; r < LIVE; r++) {
        const float d = (r % 4 == 0) ? dx[r / 4].x : (r % 4 == 1) ? dx[r / 4].y
                      : (r % 4 == 2) ? dx[r / 4].z : dx[r / 4].w;
        acc[r] += (sw * d) * (float)D[r];
    }
}

// LIVE: result registers that can hold a real row: 1, 2, 3, 4 (rows 0..LIVE-1
// in lanes 0-31; LIVE = 4 also serves M <= 8 through lanes 32-63), 8 (M <= 16),
// 16 (M <= 32).
template <int LIVE>
__global__ void __launch_bounds__(NT, 1)
k_mmv(const uint8_t *__restrict__ W, const int8_t *__restrict__ qp, float *__restrict__ Y, int M, int N,
      int K, int Mp, int nb, int U, int G)
{
    using L = Layout<LIVE>;
    constexpr int CH = L::CH;
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int s = wave % SUBS, par = wave / SUBS;             // sub-block, first super-block
    const int col = lane & 31, h = lane >> 5;
    const int ua = (int)((int64_t)U * blockIdx.x / G), ub = (int)((int64_t)U * (blockIdx.x + 1) / G);
    const uint32_t row_bytes = (uint32_t)nb * WBLK;

    // all of LDS starts at zero: the spare super-block slot of every weight
    // row and the zero activation rows stay so (the copies never write them)
    for (int i = tid; i < L::TOTAL / 16; i += NT)
        reinterpret_cast<v4i *>(lds)[i] = v4i{0, 0, 0, 0};

    // ---- chunk copy: fixed per-lane geometry ------------------------------
    // Every lane loads and stores at every step (no branches, so the wait
    // counts are the same on every path): lanes without a piece load out of
    // range and store to a per-lane sink slot.
    const int sink = L::SINK + 16 * lane;
    uint32_t w_go[L::W_LOADS];                                // byte offset in the tile's rows
    int w_st[2][L::W_LOADS], w_c[L::W_LOADS];                 // LDS target per buffer, piece in row
#pragma unroll
    for (int i = 0; i < L::W_LOADS; i++) {
        const int p = tid + NT * i;
        const int r = p / L::W_PR, c = p - r * L::W_PR;
        const bool ok = p < L::W_PIECES;
        w_go[i] = ok ? (uint32_t)r * row_bytes + 16 * c : OOB;
        w_st[0][i] = ok ? r * L::WROW + 16 * c : sink;
        w_st[1][i] = ok ? L::BUF + r * L::WROW + 16 * c : sink;
        w_c[i] = ok ? c : 1 << 20;
    }
    // the two planes are contiguous (scales at qp + Mp*K): one descriptor
    const int dp_at = Mp * K;
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc((void *)qp, (short)0, dp_at + Mp * (K / SB) * 4, BUFFER_FLAGS);
    const int qa_full = CH * SUBS * Mp * SB / 16, da_full = CH * SUBS * Mp * 4 / 16;
    const int q_st[2] = {tid < qa_full ? L::W_BYTES + 16 * tid : sink,
                         tid < qa_full ? L::BUF + L::W_BYTES + 16 * tid : sink};
    const int d_st[2] = {tid < da_full ? L::D_OFF + 16 * tid : sink,
                         tid < da_full ? L::BUF + L::D_OFF + 16 * tid : sink};
    const int t_last = (N - 1) / TILE;

    // two register sets: the copies of two chunks are in flight at once
    v4i wreg[2][L::W_LOADS], qreg[2], dreg[2];
    // Issue the loads of chunk (t, j0, cl) into register set S.  The weight
    // window starts at super-block j0 & ~1; pieces holding none of
    // super-blocks j0..j0+cl-1 are not read.  cl == 0: no chunk (the loads
    // are still issued, all out of range, so the wait counts are the same on
    // every path).
    auto load_chunk = [&](auto set, int t, int j0, int cl) {
        constexpr int S = decltype(set)::value;
        const int rows = N - t * TILE < TILE ? N - t * TILE : TILE;
        const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
            (void *)(W + (int64_t)t * TILE * row_bytes), (short)0, (int)(rows * row_bytes), BUFFER_FLAGS);
        const int je = j0 & ~1;
        const int xo = j0 * SUBS * Mp * SB, dox = dp_at + j0 * SUBS * Mp * 4;
        // piece c of a row holds bytes [16c, 16c+16) of the window; it is read
        // when they meet the chunk's bytes [lo, hi)
        const int lo = (j0 - je) * WBLK, hi = lo + cl * WBLK;
#pragma unroll
        for (int i = 0; i < L::W_LOADS; i++) {
            const bool need = (uint32_t)(16 * w_c[i] + 15 - lo) < (uint32_t)(hi - lo + 15);
            wreg[S][i] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
                                                     wr, need ? w_go[i] : OOB, je * WBLK, 0));
        }
        // (pieces past the chunk load zeros; their LDS bytes are never read)
        const int qa = cl * SUBS * Mp * SB / 16, da = cl * SUBS * Mp * 4 / 16;
        qreg[S] = __builtin_bit_cast(
            v4i, __builtin_amdgcn_raw_buffer_load_b128(xr, tid < qa ? 16u * tid : OOB, xo, 0));
        dreg[S] = __builtin_bit_cast(
            v4i, __builtin_amdgcn_raw_buffer_load_b128(xr, tid < da ? 16u * tid : OOB, dox, 0));
        // keep the sets' loads in issue order: a set is always waited for
        // while the one issued after it stays in flight
        __builtin_amdgcn_sched_barrier(0);
    };
    auto store_chunk = [&](auto set, int buf) {
        constexpr int S = decltype(set)::value;
#pragma unroll
        for (int i = 0; i < L::W_LOADS; i++)
            *reinterpret_cast<v4i *>(lds + w_st[buf][i]) = wreg[S][i];
        *reinterpret_cast<v4i *>(lds + q_st[buf]) = qreg[S];
        *reinterpret_cast<v4i *>(lds + d_st[buf]) = dreg[S];
    };

    // ---- chunk cursors (wavefront-uniform) ------------------------------------
    // A chunk ends at the run's end, the tile's end or its window's end.
    struct Cur {
        int u, t, j;
    };
    auto len = [&](const Cur &c) {
        int l = ub - c.u;
        l = l < nb - c.j ? l : nb - c.j;
        const int wl = (c.j & ~1) + CH - c.j;
        return l < wl ? l : wl;
    };
    auto advance = [&](Cur &c) {
        const int l = len(c);
        c.u += l;
        c.j += l;
        if (c.j == nb) {
            c.j = 0;
            c.t++;
        }
    };

    float acc[LIVE];
#pragma unroll
    for (int r = 0; r < LIVE; r++)
        acc[r] = 0.0f;
    float *red = reinterpret_cast<float *>(lds + 2 * L::BUF);
    auto flush = [&](int t, bool owned) {
        __syncthreads();                                      // red is free (previous flush read)
#pragma unroll
        for (int r = 0; r < LIVE; r++) {
            red[(wave * LIVE + r) * 64 + lane] = acc[r];
            acc[r] = 0.0f;
        }
        __syncthreads();
        for (int slot = tid; slot < LIVE * 64; slot += NT) {
            const int r = slot >> 6, l2 = slot & 63;
            float v = red[r * 64 + l2];
#pragma unroll
            for (int w = 1; w < NW; w++)
                v += red[(w * LIVE + r) * 64 + l2];
            const int m = 8 * (r / 4) + 4 * (l2 >> 5) + (r % 4);
            const int n = t * TILE + (l2 & 31);
            if (m < M && n < N) {
                if (owned)
                    Y[(int64_t)m * N + n] = v;
                else
                    atomicAdd(Y + (int64_t)m * N + n, v);
            }
        }
    };

    // per-lane LDS read offsets inside a chunk buffer (rows >= M: the zero row)
    const int w_lane = col * L::WROW;
    const int a_step = col < M ? Mp * SB : 0;
    int a_off[CH / PAR], d_off[CH / PAR];
#pragma unroll
    for (int i = 0; i < CH / PAR; i++) {
        const int sb = (par + PAR * i) * SUBS + s;            // sub-block within the chunk
        a_off[i] = (col < M ? L::W_BYTES + col * SB : L::Z_OFF) + 16 * h + sb * a_step;
        d_off[i] = L::D_OFF + 16 * h + 4 * sb * Mp;
    }

    const std::integral_constant<int, 0> S0;
    const std::integral_constant<int, 1> S1;
    Cur cc, cl;                                               // compute / load cursors
    cc.u = ua;
    cc.t = ua / nb;
    cc.j = ua - cc.t * nb;
    cl = cc;
    auto load_next = [&](auto set) {
        const int l = cl.u < ub ? len(cl) : 0;
        load_chunk(set, cl.t < t_last ? cl.t : t_last, cl.j, l);
        if (l > 0)
            advance(cl);
    };
    load_next(S0);                                            // chunk 0 -> set 0
    load_next(S1);                                            // chunk 1 -> set 1
    __syncthreads();                                          // LDS zeroed
    store_chunk(S0, 0);
    load_next(S0);                                            // chunk 2 -> set 0
    __syncthreads();

    // Compute chunk k from LDS buffer k%2, then move chunk k+1 from register
    // set (k+1)%2 into the other buffer (its loads were issued two chunks
    // ago) and reuse the set for chunk k+3.
    auto step = [&](auto set, auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        if (cc.u < ub) {                                      // (uniform; no memory loads inside)
            const char *b = lds + buf * L::BUF;
            const int n_sb = len(cc);
            const char *wchunk = b + w_lane + (cc.j & 1) * WBLK;  // the window starts at cc.j & ~1
#pragma unroll
            for (int i = 0; i < CH / PAR; i++) {
                const char *wrow = wchunk + (par + PAR * i) * WBLK;
                const uint2 hdr = *reinterpret_cast<const uint2 *>(wrow);
                const uint2 q = *reinterpret_cast<const uint2 *>(wrow + QS_OFF + 16 * s + 8 * h);
                const v4i ax = *reinterpret_cast<const v4i *>(b + a_off[i]);
                float4 dx[LIVE >= 4 ? LIVE / 4 : 1];
#pragma unroll
                for (int qd = 0; qd < (LIVE >= 4 ? LIVE / 4 : 1); qd++)
                    dx[qd] = *reinterpret_cast<const float4 *>(b + d_off[i] + 32 * qd);
                uint32_t wv[4];
                expand8(q.x, q.y, wv);
                const v4i bw = {(int)wv[0], (int)wv[1], (int)wv[2], (int)wv[3]};
                const v16i zero = {0};
                const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(ax, bw, zero, 0, 0, 0);
                epilogue<LIVE>(D, sub_scale(hdr.x, hdr.y, s), dx, acc);
            }
            // the tile's units end with this chunk: reduce and write it
            if (cc.j + n_sb == nb || cc.u + n_sb == ub) {
                const bool owned = cc.t * nb >= ua && (cc.t + 1) * nb <= ub;
                flush(cc.t, owned);
            }
            advance(cc);
        }
        store_chunk(set, buf ^ 1);                            // chunk k+1 (garbage past the run)
        load_next(set);                                       // chunk k+3
        __syncthreads();
    };
    // Two chunks per iteration, the second one possibly past the run (then
    // only its copy part runs): every iteration issues the same loads in the
    // same order.
    const std::integral_constant<int, 0> B0;
    const std::integral_constant<int, 1> B1;
    do {
        step(S1, B0);                                         // even chunk; chunk k+1 is in set 1
        step(S0, B1);                                         // odd chunk; chunk k+1 is in set 0
    } while (cc.u < ub);
}

template <int LIVE>
hipError_t launch_l(const uint8_t *W, const XPlanes &x, float *Y, int64_t N, const MmvPlan &p, hipStream_t s)
{
    const int nb = (int)(x.K / QK);
    const int64_t T = (N + TILE - 1) / TILE;
    const size_t lds = (size_t)Layout<LIVE>::TOTAL;
    // (the kernel reads both planes through one descriptor)
    if ((const char *)x.dp != (const char *)x.qp + x.Mp * x.K || x.Mp > Shape<LIVE>::MP_MAX)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_mmv<LIVE>), dim3((unsigned)p.grid), dim3(NT), lds, s, W, x.qp, Y, (int)x.M,
                       (int)N, (int)x.K, (int)x.Mp, nb, (int)(T * nb), p.grid);
    return hipGetLastError();
}

}  // namespace

MmvPlan mmv_plan(int64_t M, int64_t N, int64_t K, int cus)
{
    MmvPlan p;
    const int64_t nb = K / QK, row_bytes = nb * WBLK;
    const int64_t Mp = round_up(M, MPAD);
    const int64_t T = (N + TILE - 1) / TILE;
    // K/256 even (16-byte aligned chunk windows); 32-bit buffer offsets and
    // unit counts: one tile of weights, the activation planes and T*K/256
    // stay below 2^31
    if (M < 1 || M > TILE || nb % 2 != 0 || TILE * row_bytes >= (1LL << 31) ||
        Mp * K + Mp * K / 8 >= (1LL << 31) || T * nb >= (1LL << 31))
        return p;
    const int64_t U = T * nb;
    p.grid = (int)(T < cus ? T : cus);
    p.live = M <= 4 ? (int)M : M <= 8 ? 4 : M <= 16 ? 8 : 16;
    p.zero_y = false;
    for (int64_t g = 1; g < p.grid; g++)
        if (U * g / p.grid % nb != 0) {
            p.zero_y = true;                                // some tile has two owners
            break;
        }
    p.ok = true;
    return p;
}

hipError_t launch_mmv(const void *Wv, const XPlanes &x, float *Y, int64_t N, const MmvPlan &p,
                      hipStream_t s)
{
    const uint8_t *W = (const uint8_t *)Wv;
    if (!p.ok)
        return hipErrorInvalidValue;
    switch (p.live) {
    case 1: return launch_l<1>(W, x, Y, N, p, s);
    case 2: return launch_l<2>(W, x, Y, N, p, s);
    case 3: return launch_l<3>(W, x, Y, N, p, s);
    case 4: return launch_l<4>(W, x, Y, N, p, s);
    case 8: return launch_l<8>(W, x, Y, N, p, s);
    case 16: return launch_l<16>(W, x, Y, N, p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace iq4xs
