// mmv.hip -- IQ4_XS x Q8_1 on the int8 matrix cores for a few activation rows
// (M <= 32), streaming the weights once at close to HBM speed.
//
// Arithmetic (batched IQ4_XS kernel section of the "V100TPS engine log",
// agent-report.daedalus.work/V100TPS/engine.html): per 32-element sub-block the
// exact integer dot of the int8 codebook values with the int8 activations,
// here two chained v_mfma_i32_32x32x32_i8 for a 32-column x 32-row tile (the
// codebook values enter as the two int8 parts of the split codebook, one
// byte-permute lookup each), then y += d_w*(ls-32) * d_x * dot in fp32.
//
// Work split:
//  * The weights are cut into units (32-column tile t, super-block j), ordered
//    tile-major, and every workgroup gets one contiguous run of units of equal
//    length.  The grid never has more workgroups than tiles, so a run covers at
//    least one tile's worth of units and a tile is shared by at most two
//    workgroups: every compute unit gets the same work whatever the shape.
//  * A run is walked in chunks of up to CH super-blocks of one tile, chunk
//    windows starting at even super-blocks (with K/256 even, every window is
//    16-byte aligned and ends inside its row).  The list of chunks is worked
//    out once per workgroup, by one wavefront, into LDS.
//  * A chunk's weights (32 rows x up to CH*136 contiguous bytes per row) and
//    the activations of its sub-blocks (one contiguous range of the
//    sub-block-major planes) are copied to LDS with 16-byte loads that follow
//    the memory layout: every HBM access is a long contiguous run and every
//    load instruction moves 1 KB.  The first wavefronts copy weights, the
//    others activations and scales.  Two register sets carry the copies of
//    the next two chunks while the current one is computed.
//  * Sixteen wavefronts compute: wavefront w takes sub-block w%8 of the
//    chunk's super-blocks w/8, w/8+2, ... from LDS (the 8 index bytes and
//    header of its lane's row, the 16 activation bytes of its lane's row;
//    rows past M read a zero row).
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
constexpr int MAX_CHUNKS = 128;            // chunks of one workgroup's run (checked by the plan)

// LDS row stride of a weight chunk: CH*136 bytes rounded up to an odd number
// of 16-byte units, so that the 32 rows of an MFMA operand read spread over
// the banks.
constexpr int wrow_bytes(int ch)
{
    const int u = (ch * WBLK + 15) / 16;
    return 16 * (u % 2 ? u : u + 1);
}

constexpr int chunk_sb(int live) { return live <= 4 ? 8 : live == 8 ? 4 : 2; }

// LIVE result registers, activation rows padded to MPC (>= Mp) in LDS.
template <int LIVE, int MPC>
struct Layout {
    static constexpr int CH = chunk_sb(LIVE);
    static_assert(CH % PAR == 0, "every wavefront gets the same number of super-blocks");
    static constexpr int WROW = wrow_bytes(CH);
    // one chunk buffer: weights [32][WROW], activations [CH*8][Mp][32], a
    // 32-byte zero row (the operand of rows >= M), scales [CH*8][Mp] (+ slack
    // for the rows a lane reads past Mp)
    static constexpr int W_BYTES = TILE * WROW;
    static constexpr int A_BYTES = CH * SUBS * MPC * SB;
    static constexpr int Z_OFF = W_BYTES + A_BYTES;
    static constexpr int D_OFF = Z_OFF + 32;
    static constexpr int D_BYTES = CH * SUBS * MPC * 4 + 32 * 4;
    static constexpr int BUF = D_OFF + D_BYTES;
    static constexpr int RED = NW * LIVE * 64 * 4;                            // partial tiles
    static constexpr int SCHED = 2 * BUF + RED;                               // chunk list, count
    static constexpr int SINK = SCHED + MAX_CHUNKS * 16 + 16;                 // 64 x 16 bytes
    static constexpr int TOTAL = SINK + 64 * 16;
    // The copy of a chunk is cut into jobs of one wavefront load (64 lanes x
    // 16 bytes): JW jobs of weight pieces (32 rows x CH*136 bytes), JQ of
    // activation pieces, JD of scale pieces.  Every wavefront issues SLOTS
    // loads per chunk: wavefronts 0..WA-1 take the weight jobs, the others the
    // activation jobs and then the scale jobs.
    static constexpr int W_PR = CH * WBLK / 16;                               // pieces per row
    static constexpr int W_PIECES = TILE * W_PR;
    static constexpr int JW = (W_PIECES + 63) / 64;
    static constexpr int JQ = (CH * SUBS * MPC * SB / 16 + 63) / 64;
    static constexpr int JD = (CH * SUBS * MPC * 4 / 16 + 63) / 64;
    static constexpr int SLOTS = (JW + JQ + JD + NW - 1) / NW;
    static constexpr int WA = (JW + SLOTS - 1) / SLOTS;
    static_assert(WA + (JQ + JD + SLOTS - 1) / SLOTS <= NW, "copy jobs fit the wavefronts");
    static_assert(CH * WBLK % 16 == 0, "whole 16-byte pieces per row");
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

// The chunks of the run [ua, ub) in order: {t, j0, cl, flags}, flags bit 0 =
// the tile's units end with this chunk, bit 1 = the tile belongs to this
// workgroup alone.  Returns the number of chunks.
__device__ int chunk_list(v4i *out, int ua, int ub, int nb, int ch)
{
    int u = ua, t = ua / nb, j = ua - t * nb, n = 0;
    while (u < ub && n < MAX_CHUNKS) {
        int l = ub - u;
        l = l < nb - j ? l : nb - j;
        const int wl = (j & ~1) + ch - j;
        l = l < wl ? l : wl;
        const bool ends = j + l == nb || u + l == ub;
        const bool owned = t * nb >= ua && (t + 1) * nb <= ub;
        out[n++] = v4i{t, j, l, (ends ? 1 : 0) | (owned ? 2 : 0)};
        u += l;
        j += l;
        if (j == nb) {
            j = 0;
            t++;
        }
    }
    return n;
}

// LIVE: result registers that can hold a real row: 1, 2, 3, 4 (rows 0..LIVE-1
// in lanes 0-31; LIVE = 4 also serves M <= 8 through lanes 32-63), 8 (M <= 16),
// 16 (M <= 32).  MPC: a bound on the padded activation rows Mp.
template <int LIVE, int MPC>
__global__ void __launch_bounds__(NT, 1)
k_mmv(const uint8_t *__restrict__ W, const int8_t *__restrict__ qp, float *__restrict__ Y, int M, int N,
      int K, int Mp, int nb, int U, int G)
{
    using L = Layout<LIVE, MPC>;
    constexpr int CH = L::CH;
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int s = wave % SUBS, par = wave / SUBS;             // sub-block, first super-block
    const int col = lane & 31, h = lane >> 5;
    const int ua = (int)((int64_t)U * blockIdx.x / G), ub = (int)((int64_t)U * (blockIdx.x + 1) / G);
    const uint32_t row_bytes = (uint32_t)nb * WBLK;
    v4i *sched = reinterpret_cast<v4i *>(lds + L::SCHED);

    // the chunk list (one wavefront) and the two zero activation rows
    int n_chunks = 0;
    if (wave == 0) {
        if (lane == 0)
            n_chunks = chunk_list(sched, ua, ub, nb, CH);
        n_chunks = __shfl(n_chunks, 0);
        if (lane < 16)
            reinterpret_cast<uint32_t *>(lds + (lane >> 3) * L::BUF + L::Z_OFF)[lane & 7] = 0u;
        if (lane == 0)
            reinterpret_cast<int *>(lds + L::SCHED + MAX_CHUNKS * 16)[0] = n_chunks;
    }
    __syncthreads();
    n_chunks = __builtin_amdgcn_readfirstlane(reinterpret_cast<const int *>(lds + L::SCHED + MAX_CHUNKS * 16)[0]);

    // ---- chunk copy: fixed per-lane geometry ------------------------------
    // descriptors over the whole weight matrix and over both activation planes
    // (contiguous: scales at qp + Mp*K); offsets are per lane, so rows past N
    // and pieces past a plane read as zero
    const int dp_at = Mp * K;
    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc((void *)W, (short)0, (int)((uint32_t)N * row_bytes), BUFFER_FLAGS);
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc((void *)qp, (short)0, dp_at + Mp * (K / SB) * 4, BUFFER_FLAGS);
    const bool w_group = wave < L::WA;                        // (uniform)
    const __amdgpu_buffer_rsrc_t rsrc = w_group ? wr : xr;
    const int sink = L::SINK + 16 * lane;
    // per slot: this lane's piece offset inside the chunk (global bytes), its
    // piece number inside its row (weights) or plane range (activations,
    // scales), whether it is a scale piece, and its LDS target per buffer
    uint32_t p_go[L::SLOTS];
    int p_id[L::SLOTS], p_st[2][L::SLOTS];
    bool p_scale[L::SLOTS];
    const int qa_full = CH * SUBS * Mp * SB / 16, da_full = CH * SUBS * Mp * 4 / 16;
#pragma unroll
    for (int k = 0; k < L::SLOTS; k++) {
        if (w_group) {
            const int p = 64 * (wave * L::SLOTS + k) + lane;
            const int r = p / L::W_PR, c = p - r * L::W_PR;
            const bool ok = p < L::W_PIECES;
            p_go[k] = ok ? (uint32_t)r * row_bytes + 16 * c : OOB;
            p_id[k] = ok ? c : 1 << 20;
            p_scale[k] = false;
            p_st[0][k] = ok ? r * L::WROW + 16 * c : sink;
            p_st[1][k] = ok ? L::BUF + r * L::WROW + 16 * c : sink;
        } else {
            const int job = (wave - L::WA) * L::SLOTS + k;    // activation jobs first, then scales
            const bool isq = job < L::JQ;
            const int p = 64 * (isq ? job : job - L::JQ) + lane;
            const bool ok = isq ? p < qa_full : p < da_full;
            p_go[k] = ok ? (isq ? 16u * p : (uint32_t)dp_at + 16u * p) : OOB;
            p_id[k] = ok ? p : 1 << 20;
            p_scale[k] = !isq;
            const int at = isq ? L::W_BYTES + 16 * p : L::D_OFF + 16 * p;
            p_st[0][k] = ok ? at : sink;
            p_st[1][k] = ok ? L::BUF + at : sink;
        }
    }

    // two register sets: the copies of two chunks are in flight at once
    v4i creg[2][L::SLOTS];
    // Issue the loads of chunk c into register set S.  The weight window
    // starts at super-block j0 & ~1; pieces holding none of super-blocks
    // j0..j0+cl-1, and activation or scale pieces past the chunk, are not
    // read.  Every wavefront issues SLOTS loads per chunk, also past the last
    // chunk (all out of range then), so the wait counts are the same on every
    // path.
    auto load_chunk = [&](auto set, int c) {
        constexpr int S = decltype(set)::value;
        v4i info = v4i{0, 0, 0, 0};
        if (c < n_chunks)
            info = sched[c];
        const int t = __builtin_amdgcn_readfirstlane(info[0]);
        const int j0 = __builtin_amdgcn_readfirstlane(info[1]);
        const int cl = __builtin_amdgcn_readfirstlane(info[2]);
        const int je = j0 & ~1;
        // weights: piece c of a row holds bytes [16c, 16c+16) of the window;
        // it is read when they meet the chunk's bytes [lo, hi).  Activations
        // and scales: pieces below the chunk's count are read.  (One load
        // instruction per slot for both groups: no branch around the loads.)
        const int lo = (j0 - je) * WBLK, hi = lo + cl * WBLK;
        const uint32_t wbase = (uint32_t)t * TILE * row_bytes + je * WBLK;
        const int qa = cl * SUBS * Mp * SB / 16, da = cl * SUBS * Mp * 4 / 16;
        const uint32_t qbase = j0 * SUBS * Mp * SB, dbase = j0 * SUBS * Mp * 4;
#pragma unroll
        for (int k = 0; k < L::SLOTS; k++) {
            const bool need = w_group ? (uint32_t)(16 * p_id[k] + 15 - lo) < (uint32_t)(hi - lo + 15)
                                      : p_id[k] < (p_scale[k] ? da : qa);
            const uint32_t base = w_group ? wbase : p_scale[k] ? dbase : qbase;
            creg[S][k] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(
                                                     rsrc, need ? p_go[k] + base : OOB, 0, 0));
        }
        // keep the sets' loads in issue order: a set is always waited for
        // while the one issued after it stays in flight
        __builtin_amdgcn_sched_barrier(0);
    };
    // (lanes without a piece store to their sink slot)
    auto store_chunk = [&](auto set, auto bufc) {
        constexpr int S = decltype(set)::value, buf = decltype(bufc)::value;
#pragma unroll
        for (int k = 0; k < L::SLOTS; k++)
            *reinterpret_cast<v4i *>(lds + p_st[buf][k]) = creg[S][k];
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
    const std::integral_constant<int, 0> B0;
    const std::integral_constant<int, 1> B1;
    load_chunk(S0, 0);                                        // chunk 0 -> set 0
    load_chunk(S1, 1);                                        // chunk 1 -> set 1
    store_chunk(S0, B0);
    load_chunk(S0, 2);                                        // chunk 2 -> set 0
    __syncthreads();

    // Compute chunk c from LDS buffer c%2, then move chunk c+1 from register
    // set (c+1)%2 into the other buffer (its loads were issued two chunks
    // ago) and reuse the set for chunk c+3.
    auto step = [&](auto set, auto bufc, int c) {
        constexpr int buf = decltype(bufc)::value;
        if (c < n_chunks) {                                   // (uniform; no memory loads inside)
            const v4i info = sched[c];
            const int t = __builtin_amdgcn_readfirstlane(info[0]);
            const int j0 = __builtin_amdgcn_readfirstlane(info[1]);
            const int n_sb = __builtin_amdgcn_readfirstlane(info[2]);
            const int flags = __builtin_amdgcn_readfirstlane(info[3]);
            const char *b = lds + buf * L::BUF;
            const char *wchunk = b + w_lane + (j0 & 1) * WBLK;  // the window starts at j0 & ~1
#pragma unroll
            for (int i = 0; i < CH / PAR; i++) {
                if (par + PAR * i >= n_sb)                    // (uniform) past the chunk's end
                    break;
                const char *wrow = wchunk + (par + PAR * i) * WBLK;
                const uint2 hdr = *reinterpret_cast<const uint2 *>(wrow);
                const uint2 q = *reinterpret_cast<const uint2 *>(wrow + QS_OFF + 16 * s + 8 * h);
                const v4i ax = *reinterpret_cast<const v4i *>(b + a_off[i]);
                float4 dx[LIVE >= 4 ? LIVE / 4 : 1];
#pragma unroll
                for (int qd = 0; qd < (LIVE >= 4 ? LIVE / 4 : 1); qd++)
                    dx[qd] = *reinterpret_cast<const float4 *>(b + d_off[i] + 32 * qd);
                uint32_t wa[4], wb[4];
                expand8_split(q.x, q.y, wa, wb);
                const v4i ba = {(int)wa[0], (int)wa[1], (int)wa[2], (int)wa[3]};
                const v4i bb = {(int)wb[0], (int)wb[1], (int)wb[2], (int)wb[3]};
                const v16i zero = {0};
                const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                    ax, bb, __builtin_amdgcn_mfma_i32_32x32x32_i8(ax, ba, zero, 0, 0, 0), 0, 0, 0);
                epilogue<LIVE>(D, sub_scale(hdr.x, hdr.y, s), dx, acc);
            }
            if (flags & 1)                                    // the tile's units end here
                flush(t, (flags & 2) != 0);
        }
        store_chunk(set, std::integral_constant<int, buf ^ 1>());   // chunk c+1
        load_chunk(set, c + 3);                                     // chunk c+3
        __syncthreads();
    };
    // Two chunks per iteration, the second one possibly past the run (then
    // only its copy part runs): every iteration issues the same loads.
    for (int c = 0; c < n_chunks; c += 2) {
        step(S1, B0, c);                                      // chunk c+1 is in set 1
        step(S0, B1, c + 1);                                  // chunk c+2 is in set 0
    }
}

template <int LIVE, int MPC>
hipError_t launch_l(const uint8_t *W, const XPlanes &x, float *Y, int64_t N, const MmvPlan &p, hipStream_t s)
{
    const int nb = (int)(x.K / QK);
    const int64_t T = (N + TILE - 1) / TILE;
    const size_t lds = (size_t)Layout<LIVE, MPC>::TOTAL;
    // (the kernel reads both planes through one descriptor)
    if ((const char *)x.dp != (const char *)x.qp + x.Mp * x.K || x.Mp > MPC)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_mmv<LIVE, MPC>), dim3((unsigned)p.grid), dim3(NT), lds, s, W, x.qp, Y, (int)x.M,
                       (int)N, (int)x.K, (int)x.Mp, nb, (int)(T * nb), p.grid);
    return hipGetLastError();
}

// Chunks of the longest run (the same rule as chunk_list).
int64_t max_chunks(int64_t U, int64_t nb, int grid, int ch)
{
    int64_t most = 0;
    for (int g = 0; g < grid; g++) {
        const int64_t ua = U * g / grid, ub = U * (g + 1) / grid;
        int64_t u = ua, j = ua % nb, n = 0;
        while (u < ub) {
            int64_t l = ub - u;
            l = l < nb - j ? l : nb - j;
            const int64_t wl = (j & ~1LL) + ch - j;
            l = l < wl ? l : wl;
            u += l;
            j = (j + l) % nb;
            n++;
        }
        most = n > most ? n : most;
    }
    return most;
}

}  // namespace

MmvPlan mmv_plan(int64_t M, int64_t N, int64_t K, int cus)
{
    MmvPlan p;
    const int64_t nb = K / QK, row_bytes = nb * WBLK;
    const int64_t Mp = round_up(M, MPAD);
    const int64_t T = (N + TILE - 1) / TILE;
    // K/256 even (16-byte aligned chunk windows); 32-bit buffer offsets and
    // unit counts: the weight matrix, the activation planes and T*K/256 stay
    // below 2^31
    if (M < 1 || M > TILE || nb % 2 != 0 || N * row_bytes >= (1LL << 31) ||
        Mp * K + Mp * K / 8 >= (1LL << 31) || T * nb >= (1LL << 31))
        return p;
    const int64_t U = T * nb;
    p.grid = (int)(T < cus ? T : cus);
    p.live = M <= 4 ? (int)M : M <= 8 ? 4 : M <= 16 ? 8 : 16;
    if (max_chunks(U, nb, p.grid, chunk_sb(p.live)) > MAX_CHUNKS)
        return p;
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
    case 1: return launch_l<1, 4>(W, x, Y, N, p, s);
    case 2: return launch_l<2, 4>(W, x, Y, N, p, s);
    case 3: return launch_l<3, 4>(W, x, Y, N, p, s);
    case 4: return x.Mp <= 4 ? launch_l<4, 4>(W, x, Y, N, p, s) : launch_l<4, 8>(W, x, Y, N, p, s);
    case 8: return launch_l<8, 16>(W, x, Y, N, p, s);
    case 16: return launch_l<16, 32>(W, x, Y, N, p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace iq4xs
