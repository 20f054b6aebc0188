// mmqt.hip -- IQ4_XS x Q8_1 for many activation rows (M > 32) on the int8
// matrix cores: output tiles of BM activation rows x BN weight rows, each
// output owned by one wavefront.
//
// Arithmetic (batched IQ4_XS kernel section of the "V100TPS engine log",
// agent-report.daedalus.work/V100TPS/engine.html): per 32-element sub-block
// the exact integer dot of the int8 codebook values with the int8
// activations (one v_mfma_i32_32x32x32_i8 over the full 16-entry lookup),
// then y += d_w*(ls-32) * d_x * dot in fp32.  (The split codebook of the
// streaming kernel would save lookup work for a second MFMA; here the VALU
// and matrix-core work of a SIMD add up rather than overlap, and the single
// MFMA measured faster.)
//
// Work split:
//  * Tiles (see QCfg): 64 x 256 up to M = 64, 128 x 128 above, and 256 x 128
//    (M >= 256) or 128 x 256 (M >= 128) where those larger tiles need no
//    summing of many partial tiles.  Tiles are ordered with the weight
//    block fastest, so with several activation blocks the partition repeats
//    in each of them and the runs over one weight range can share an XCD's
//    L2.  Units are (tile, half super-block), tile-major; each
//    workgroup gets one contiguous run of equal length (stream-K style:
//    every compute unit gets the same work, also when there are fewer tiles
//    than compute units).  A tile covered by one run is stored by its
//    workgroup.  When every run covers at least a tile's units, a tile has
//    two owners at most and they add into a Y whose shared tiles were zeroed
//    beforehand (0 + a + b == 0 + b + a); otherwise the owners store their
//    partial tiles (at most two per run: its first and its last) in a
//    workspace, and a second kernel adds the partials of every shared tile
//    in run order.  Either way the result does not depend on timing.
//  * Half a super-block of a tile at a time (4 sub-blocks) goes straight
//    from memory into one of NBUF LDS buffers (5, or 3 for the larger tiles)
//    with 16-byte LDS-writing buffer loads: for each of the BN weight rows
//    its header and the half's 64 index bytes (an 80-byte LDS row), the BM
//    activation rows of the 4 sub-blocks (sub-block-major planes) and their
//    scales.  The loads of a half run NBUF-1 halves ahead of its use; one
//    barrier per half.  (A wavefront that walked the run ahead touching
//    whole weight rows, to turn the 72-byte pieces into long contiguous
//    reads, made every measured shape 4-9% slower: it arrived last at every
//    barrier.)
//  * Eight wavefronts: wavefront w owns weight subtile w%(BN/32) and a group
//    of G activation subtiles w/(BN/32) (G = 2, or 4 for the larger tiles),
//    i.e. G x 16 accumulators per lane.  Per sub-block it expands its weight
//    subtile's index bytes once (byte permutes) and uses them for all G
//    activation subtiles, so the fp32 rescale of the integer dots (three
//    VALU operations per output and sub-block) is the bulk of the work.
#include "common.hpp"
#include "stream.hpp"

#include <algorithm>

namespace iq4xs {
namespace {

using namespace stream;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int TILE = 32;
constexpr int NWQ = 8, NTQ = 64 * NWQ;     // wavefronts, threads per workgroup
constexpr int HALF = SUBS / 2;             // sub-blocks per step
constexpr int WROWQ = 80;                  // LDS weight row: header, 8 unused, 64 index bytes
constexpr int NLQ = NWQ;                   // copying wavefronts

// Output tile BM activation rows x BN weight rows: 64 x 256, 128 x 128,
// 256 x 128 or 128 x 256 (mmqt_plan picks one).  Wavefront w owns weight
// subtile w % (BN/32) and the group of G activation subtiles w / (BN/32):
// G = 2, or 4 for the two large tiles, where each wavefront's codebook lookup
// serves four activation subtiles (half the lookup work per output; the
// rescale, three VALU instructions per output, is the rest).  One LDS
// buffer: weights [BN][80], activations [HALF][BM][32], scales [HALF][BM],
// 1 KB for slots without a job; NBUF buffers (5, or 3 for the large tiles).
// F: the weight format.  An 80-byte weight row holds, for IQ4_XS, the
// super-block's 8 header bytes, 8 unused bytes and the half's 64 index
// bytes; for IQ4_NL and Q4_0, bytes [0, 80) of the 144-byte unit for the
// first half and [64, 144) for the second (its four 18-byte blocks at
// 8 + 18s), so that no copy reaches past the unit.
template <int BM_, int BN_, int F_ = FMT_IQ4_XS>
struct QCfg {
    static constexpr int BM = BM_, BN = BN_, NTW = BN / TILE, F = F_;
    static constexpr int G = (BM / TILE) * NTW / NWQ;          // activation subtiles per wavefront
    static constexpr int U = G == 2 ? 2 : 1;                    // sub-blocks per compute group
    static constexpr int NBUF = G == 2 ? 5 : 3;
    static constexpr int W_BYTES = BN * WROWQ;
    static constexpr int A_OFF = W_BYTES, A_BYTES = HALF * BM * SB;
    static constexpr int D_OFF = A_OFF + A_BYTES, D_BYTES = HALF * BM * 4;
    static constexpr int DUMP = D_OFF + D_BYTES;
    static constexpr int BUFQ = DUMP + 1024;
    static constexpr int JW = W_BYTES / 1024, JA = A_BYTES / 1024, JD = D_BYTES / 1024;
    static constexpr int SLOTS = (JW + JA + JD + NLQ - 1) / NLQ;
    static_assert((G == 2 || G == 4) && NTW * (BM / (G * TILE)) == NWQ, "eight wavefronts: weight subtile x group");
    static_assert(W_BYTES % 1024 == 0 && D_BYTES % 1024 == 0 && NBUF * BUFQ + 256 <= 160 * 1024, "LDS budget");
};

// Unit cursor: one half super-block of one tile per step (j counts halves,
// nh = 2 * K/256 of them per tile).
struct UnitCursor {
    int u, t, j, ua, ub, nh;
    __device__ Chunk next()
    {
        Chunk c{t, j, 0, 0};
        if (u < ub) {
            const bool ends = j + 1 == nh || u + 1 == ub;
            const bool owned = t * nh >= ua && (t + 1) * nh <= ub;
            c.cl = 1;
            c.flags = (ends ? 1 : 0) | (owned ? 2 : 0);
            u++;
            if (++j == nh) {
                j = 0;
                t++;
            }
        }
        return c;
    }
};

// The runs whose first tile is shared and ends inside them (the last owner
// of each tile with more than one), found on the host.
struct FixRuns {
    int k[MAXG];
};

// Partial tile slot (run g, 0 = its first tile, 1 = its last): 4*G float4
// per thread, float4 e of thread tid at [e][tid] (coalesced stores and
// loads); e = 4*i + r/4 for accumulator i, result register r.
constexpr int slot_f4(int G) { return 4 * G * NTQ; }
template <int G>
__device__ __forceinline__ float4 *slot_at(float *ws, int g, int which)
{
    return reinterpret_cast<float4 *>(ws) + (size_t)(2 * g + which) * slot_f4(G);
}

template <class C>
__global__ void __launch_bounds__(NTQ, 1)
k_mmqt(const uint8_t *__restrict__ W, const int8_t *__restrict__ qp, float *__restrict__ Y,
       float *__restrict__ ws, int M, int N, int K, int Mp, int nb, int wblocks, int G, int add_into_y, Runs runs)
{
    constexpr int BM = C::BM, BN = C::BN, SLOTS = C::SLOTS, JW = C::JW, JA = C::JA, JD = C::JD;
    constexpr int A_OFF = C::A_OFF, D_OFF = C::D_OFF, BUFQ = C::BUFQ;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    constexpr int GQ = C::G, UQ = C::U, NB = C::NBUF;
    const int nt = wave % C::NTW, mq = wave / C::NTW;        // weight subtile, activation group
    const int col = lane & 31, h = lane >> 5;
    // Workgroups are dealt round-robin to the 8 XCDs (each with its own L2).
    // Tiles are numbered weight block fastest, so runs g and g + G/mblocks
    // cover the same weight columns and half super-blocks in consecutive
    // activation blocks, at the same pace.  One XCD takes such a set of runs
    // (and neighbouring sets), so the weights that one of them loads are in
    // that XCD's L2 when the others need them.
    const int mblocks = (M + BM - 1) / BM;
    int g = (int)blockIdx.x;
    if (G % (8 * mblocks) == 0) {
        const int S = G / 8, x = g % 8, s = g / 8;
        g = (s % mblocks) * (G / mblocks) + x * (S / mblocks) + s / mblocks;
    } else if (G % 8 == 0) {
        g = (g % 8) * (G / 8) + g / 8;
    }
    const int ua = runs.u[g], ub = runs.u[g + 1], t_first = runs.t[g];
    const uint32_t row_bytes = (uint32_t)nb * sblk_bytes(C::F);
    const int dp_at = Mp * K;
    const __amdgpu_buffer_rsrc_t wr =
        __builtin_amdgcn_make_buffer_rsrc((void *)W, (short)0, (int)((uint32_t)N * row_bytes), BUFFER_FLAGS);
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc((void *)qp, (short)0, dp_at + Mp * (K / SB) * 4, BUFFER_FLAGS);

    // Per slot: the LDS offset its load fills (uniform), which plane it reads
    // (uniform: 0 weights, 1 activations, 2 scales, 3 none) and this lane's
    // offset relative to the unit's base, for the first and the second half
    // of a super-block (weights: 16-byte piece p of an 80-byte LDS row holds
    // super-block bytes [0,16) for p = 0, else the half's index bytes).
    int p_dst[SLOTS], p_kind[SLOTS];
    uint32_t p_go0[SLOTS], p_go1[SLOTS];
#pragma unroll
    for (int k = 0; k < SLOTS; k++) {
        const int job = wave * SLOTS + k;
        if (job < JW) {
            const int at = 1024 * job + 16 * lane;
            const int r = at / WROWQ, pc = (at - r * WROWQ) / 16;   // row, piece (5 per row)
            p_dst[k] = 1024 * job;
            p_kind[k] = 0;
            if constexpr (C::F == FMT_IQ4_XS) {
                p_go0[k] = (uint32_t)r * row_bytes + (pc == 0 ? 0 : 16 * pc - 8);
                p_go1[k] = (uint32_t)r * row_bytes + (pc == 0 ? 0 : 16 * pc + 56);
            } else {
                p_go0[k] = (uint32_t)r * row_bytes + 16 * pc;
                p_go1[k] = (uint32_t)r * row_bytes + 64 + 16 * pc;
            }
        } else if (job < JW + JA) {
            const int a = job - JW;                               // 1 KB = 32 rows of one sub-block
            const int sb = a / (BM / TILE), r = TILE * (a % (BM / TILE)) + (lane >> 1);
            p_dst[k] = A_OFF + 1024 * a;
            p_kind[k] = 1;
            p_go0[k] = p_go1[k] = (uint32_t)((sb * Mp + r) * SB + 16 * (lane & 1));
        } else if (job < JW + JA + JD) {
            const int d = job - JW - JA;                          // 1 KB = 1024/(4 BM) sub-blocks' scales
            const int sb = (256 / BM) * d + lane / (BM / 4), r = 4 * (lane % (BM / 4));
            p_dst[k] = D_OFF + 1024 * d;
            p_kind[k] = 2;
            p_go0[k] = p_go1[k] = (uint32_t)((sb * Mp + r) * 4);
        } else {
            p_dst[k] = C::DUMP;
            p_kind[k] = 3;
            p_go0[k] = p_go1[k] = OOB;
        }
    }
    // tile t -> (activation block, weight block), the weight block fastest;
    // unit half j: super-block j/2, sub-blocks 4*(j%2) .. 4*(j%2)+3
    auto issue = [&](const Chunk &c, auto bc) __attribute__((always_inline)) {
        char *buf = lds_area<decltype(bc)::value, BUFQ>();
        const int mb = c.t / wblocks, wb = c.t - mb * wblocks, js = c.j0 >> 1, hf = c.j0 & 1;
        const bool live = c.cl > 0;
        const uint32_t wbase = (uint32_t)wb * BN * row_bytes + (uint32_t)js * sblk_bytes(C::F);
        const int sb0 = js * SUBS + HALF * hf;
        const uint32_t abase = (uint32_t)((sb0 * Mp + mb * BM) * SB);
        const uint32_t dbase = (uint32_t)(dp_at + (sb0 * Mp + mb * BM) * 4);
#pragma unroll
        for (int k = 0; k < SLOTS; k++) {
            const uint32_t base = p_kind[k] == 0 ? wbase : p_kind[k] == 1 ? abase : dbase;
            const bool ok = live && p_kind[k] != 3;
            load_lds16(p_kind[k] == 0 ? wr : xr, buf + p_dst[k], ok ? (hf ? p_go1[k] : p_go0[k]) + base : OOB);
        }
    };

    float acc[GQ][16];
#pragma unroll
    for (int i = 0; i < GQ; i++)
#pragma unroll
        for (int r = 0; r < 16; r++)
            acc[i][r] = 0.0f;
    // result register r of lane (col, h) holds activation row 8*(r/4) + 4*h + r%4
    auto flush = [&](int t, bool owned) __attribute__((always_inline)) {
        if (owned) {
            const int mb = t / wblocks, wb = t - mb * wblocks;
            const int n = wb * BN + nt * TILE + col;
#pragma unroll
            for (int i = 0; i < GQ; i++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int m = mb * BM + (GQ * mq + i) * TILE + 8 * (r / 4) + 4 * h + (r % 4);
                    if (m < M && n < N)
                        Y[(int64_t)m * N + n] = acc[i][r];
                }
        } else if (add_into_y) {                              // (uniform) two owners at most
            const int mb = t / wblocks, wb = t - mb * wblocks;
            const int n = wb * BN + nt * TILE + col;
#pragma unroll
            for (int i = 0; i < GQ; i++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    const int m = mb * BM + (GQ * mq + i) * TILE + 8 * (r / 4) + 4 * h + (r % 4);
                    if (m < M && n < N)
                        atomicAdd(Y + (int64_t)m * N + n, acc[i][r]);
                }
        } else {
            float4 *slot = slot_at<GQ>(ws, g, t == t_first ? 0 : 1);
#pragma unroll
            for (int i = 0; i < GQ; i++)
#pragma unroll
                for (int q = 0; q < 4; q++)
                    slot[(4 * i + q) * NTQ + tid] =
                        make_float4(acc[i][4 * q], acc[i][4 * q + 1], acc[i][4 * q + 2], acc[i][4 * q + 3]);
        }
#pragma unroll
        for (int i = 0; i < GQ; i++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                acc[i][r] = 0.0f;
    };
    auto compute = [&](const Chunk &c, auto bc) __attribute__((always_inline)) {
        const char *B = lds_area<decltype(bc)::value, BUFQ>();
        const char *wrow = B + (nt * TILE + col) * WROWQ;
        const int hf = c.j0 & 1;
        // (IQ4_XS: the header; the other formats read each block's d)
        uint2 hdr = make_uint2(0u, 0u);
        if constexpr (C::F == FMT_IQ4_XS)
            hdr = *reinterpret_cast<const uint2 *>(wrow);
        const char *unit = wrow - 64 * hf;                    // where the 144-byte unit would start
        // U sub-blocks at a time (two with G = 2, one with G = 4): all their
        // LDS reads first, then all U*G products (each into registers of its
        // own), then the epilogues, so that reads, lookups, matrix-core work
        // and rescaling overlap.
#pragma unroll
        for (int s0 = 0; s0 < HALF; s0 += UQ) {
            uint2 q[UQ];
            v4i ax[UQ][GQ];
            float4 dx[UQ][GQ][4];
            // this lane's activation scales of subtile i, sub-block s: rows
            // 8*qd + 4*h .. +3
            auto load_dx = [&](int u, int i) __attribute__((always_inline)) {
#pragma unroll
                for (int qd = 0; qd < 4; qd++)
                    dx[u][i][qd] = *reinterpret_cast<const float4 *>(
                        B + D_OFF + ((s0 + u) * BM + (GQ * mq + i) * TILE + 4 * h + 8 * qd) * 4);
            };
#pragma unroll
            for (int u = 0; u < UQ; u++) {
                const int s = s0 + u;
                if constexpr (C::F == FMT_IQ4_XS)
                    q[u] = *reinterpret_cast<const uint2 *>(wrow + 16 + 16 * s + 8 * h);
                else
                    q[u] = unit_qs<C::F>(unit, HALF * hf + s, h);
#pragma unroll
                for (int i = 0; i < GQ; i++) {
                    const int mt = GQ * mq + i;
                    ax[u][i] = *reinterpret_cast<const v4i *>(B + A_OFF + (s * BM + mt * TILE + col) * SB + 16 * h);
                    if constexpr (GQ == 2)
                        load_dx(u, i);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            v16i D[UQ][GQ];
            float sw[UQ];
            if constexpr (UQ == 2) {
                // (the two halves of the wavefront, same rows, each decode one
                // of the two sub-blocks' scales and swap them)
                const float sc = C::F == FMT_IQ4_XS ? sub_scale(hdr.x, hdr.y, HALF * hf + s0 + h)
                                                    : unit_scale<C::F>(unit, HALF * hf + s0 + h, true);
                const uint32_t own = __builtin_bit_cast(uint32_t, sc);
                const auto both = __builtin_amdgcn_permlane32_swap(own, own, false, false);
                sw[0] = __builtin_bit_cast(float, (uint32_t)both[0]);
                sw[1] = __builtin_bit_cast(float, (uint32_t)both[1]);
            } else {
                sw[0] = C::F == FMT_IQ4_XS ? sub_scale(hdr.x, hdr.y, HALF * hf + s0)
                                           : unit_scale<C::F>(unit, HALF * hf + s0, true);
            }
#pragma unroll
            for (int u = 0; u < UQ; u++) {
                uint32_t wf[4];
                expand8<C::F>(q[u].x, q[u].y, wf);
                const v4i bf = {(int)wf[0], (int)wf[1], (int)wf[2], (int)wf[3]};
#pragma unroll
                for (int i = 0; i < GQ; i++) {
                    const v16i zero = {0};
                    D[u][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(ax[u][i], bf, zero, 0, 0, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int u = 0; u < UQ; u++)
#pragma unroll
                for (int i = 0; i < GQ; i++) {
                    if constexpr (GQ == 4) {
                        // (scales loaded per subtile: sixteen registers live, not 64)
                        load_dx(u, i);
                        __builtin_amdgcn_sched_barrier(0);
                    }
#pragma unroll
                    for (int r = 0; r < 16; r++) {
                        const float d = (r % 4 == 0) ? dx[u][i][r / 4].x : (r % 4 == 1) ? dx[u][i][r / 4].y
                                      : (r % 4 == 2) ? dx[u][i][r / 4].z : dx[u][i][r / 4].w;
                        acc[i][r] += (sw[u] * d) * (float)D[u][i][r];
                    }
                }
#pragma unroll
            for (int u = 0; u < UQ; u++)
#pragma unroll
                for (int i = 0; i < GQ; i++)
                    keep_live(D[u][i]);
        }
        if (c.flags & 1)
            flush(c.t, (c.flags & 2) != 0);
    };

    UnitCursor cur;
    cur.ua = ua;
    cur.ub = ub;
    cur.nh = 2 * nb;
    cur.u = ua;
    cur.t = t_first;
    cur.j = ua - cur.t * 2 * nb;
    Chunk info[NB];
    static_for(std::make_integer_sequence<int, NB - 1>(), [&](auto bc) {
        info[decltype(bc)::value] = cur.next();
        issue(info[decltype(bc)::value], bc);
    });
    // Step on buffer b: wait for this wavefront's loads of the unit (those of
    // the NB-2 units issued after it stay in flight), meet the others (all
    // loads landed; the buffer computed last is free), load the unit NB-1
    // ahead into that buffer, compute.
    auto step = [&](auto bc) __attribute__((always_inline)) {
        constexpr int b = decltype(bc)::value, nxt = (b + NB - 1) % NB;
        if (info[b].cl == 0)
            return false;
        __builtin_amdgcn_s_waitcnt(wait_vm_lds(SLOTS * (NB - 2)));
        raw_barrier();
        info[nxt] = cur.next();
        issue(info[nxt], std::integral_constant<int, nxt>());
        compute(info[b], bc);
        return true;
    };
    bool go = true;
    do
        static_for(std::make_integer_sequence<int, NB>(), [&](auto bc) __attribute__((always_inline)) {
            if (go)
                go = step(bc);
        });
    while (go);
    __builtin_amdgcn_s_waitcnt(wait_vm_lds(0));
}

// The shared tiles: workgroup (i, e) takes run k = fix.k[i], which starts
// inside its first tile and reaches that tile's end (each shared tile is the
// first tile of exactly one such run, the last of its owners), and adds
// float4 e of every thread's slot over the owners k', k'+1, .., k in that
// order.
template <class C>
__global__ void __launch_bounds__(NTQ, 1)
k_mmqt_fix(const float *__restrict__ ws, float *__restrict__ Y, int M, int N, int nh, int wblocks, Runs runs,
           FixRuns fix)
{
    constexpr int BM = C::BM, BN = C::BN;
    const int k = fix.k[blockIdx.x], e = blockIdx.y, tid = threadIdx.x;
    const int t = runs.t[k];
    const int t0 = t * nh;
    int g0 = k - 1;
    while (runs.u[g0] > t0)                                    // runs.u[0] == 0 <= t0
        g0--;
    // owners in groups of eight: all loads of a group in flight together,
    // then the adds in owner order (an owner with an empty run adds zero)
    float4 sum = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    for (int gg0 = g0; gg0 <= k; gg0 += 8) {
        float4 v[8];
#pragma unroll
        for (int q = 0; q < 8; q++) {
            const int gg = gg0 + q;
            v[q] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (gg <= k && runs.u[gg] != runs.u[gg + 1])          // (uniform)
                v[q] = (reinterpret_cast<const float4 *>(ws) +
                        (size_t)(2 * gg + (runs.t[gg] == t ? 0 : 1)) * slot_f4(C::G))[e * NTQ + tid];
        }
#pragma unroll
        for (int q = 0; q < 8; q++) {
            sum.x += v[q].x;
            sum.y += v[q].y;
            sum.z += v[q].z;
            sum.w += v[q].w;
        }
    }
    const int lane = tid & 63, wave = tid >> 6;
    const int nt = wave % C::NTW, mq = wave / C::NTW, col = lane & 31, h = lane >> 5;
    const int mb = t / wblocks, wb = t - mb * wblocks;
    const int n = wb * BN + nt * TILE + col;
    const float v4[4] = {sum.x, sum.y, sum.z, sum.w};
#pragma unroll
    for (int c = 0; c < 4; c++) {
        const int i = e / 4, r = 4 * (e % 4) + c;
        const int m = mb * BM + (C::G * mq + i) * TILE + 8 * (r / 4) + 4 * h + (r % 4);
        if (m < M && n < N)
            Y[(int64_t)m * N + n] = v4[c];
    }
}

template <class C>
hipError_t launch_cfg(const void *W, const XPlanes &x, float *Y, float *ws, int64_t N, const MmqtPlan &p,
                      const Runs &runs, hipStream_t s)
{
    const int nb = (int)(x.K / QK);
    hipLaunchKernelGGL((k_mmqt<C>), dim3((unsigned)p.grid), dim3(NTQ), 0, s, (const uint8_t *)W, x.qp, Y, ws,
                       (int)x.M, (int)N, (int)x.K, (int)x.Mp, nb, p.wblocks, p.grid, p.zero_y ? 1 : 0, runs);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.workspace_bytes == 0)
        return e;
    // one group of 4*G workgroups per shared tile: the runs that start inside
    // their first tile and reach its end
    FixRuns fix;
    int nfix = 0;
    const int nh = 2 * nb;
    for (int k = 0; k < p.grid; k++) {
        const int t0 = runs.t[k] * nh;
        if (runs.u[k] != runs.u[k + 1] && runs.u[k] != t0 && runs.u[k + 1] >= t0 + nh)
            fix.k[nfix++] = k;
    }
    if (nfix == 0)
        return hipSuccess;
    hipLaunchKernelGGL((k_mmqt_fix<C>), dim3((unsigned)nfix, 4 * C::G), dim3(NTQ), 0, s, (const float *)ws, Y,
                       (int)x.M, (int)N, nh, p.wblocks, runs, fix);
    return hipGetLastError();
}

}  // namespace

namespace {

// The plan for tiles of BM x BN (not ok: offsets past 32 bits).
MmqtPlan plan_tiles(int64_t M, int64_t N, int64_t K, int cus, int fmt, int64_t BM, int64_t BN)
{
    MmqtPlan p;
    const int64_t nb = K / QK, row_bytes = nb * sblk_bytes(fmt);
    const int64_t Mp = round_up(M, MPAD);
    const int64_t mblocks = (M + BM - 1) / BM, wblocks = (N + BN - 1) / BN;
    const int64_t T = mblocks * wblocks, U = T * 2 * nb;
    // 32-bit offsets
    if (M <= TILE || nb >= (1 << 15) || N * row_bytes >= (1LL << 31) ||
        Mp * K + Mp * K / 8 + BM * 288 >= (1LL << 31) || U >= (1LL << 31))
        return p;
    // Runs of at least 8 units (writing and re-reading a partial tile, 64 KB,
    // stays small against a run's work) while that keeps at least half of
    // the compute units busy, else of 4, else of 2 (measured on MI355X: 8 is
    // best at M=64, 10240 x 5120 (44 vs 50 us with 4); 4 at M=64, 5120 x
    // 5120 (37 vs 40 us); 2 at M=64, 5120 x 1024 (26 vs 28 us)).
    const int64_t cap = std::min<int64_t>(cus, MAXG);
    int64_t G = U / 8;
    if (G < cap / 2)
        G = U / 4 >= cap / 4 ? U / 4 : U / 2;
    G = std::min<int64_t>(G, cap);
    p.grid = (int)std::max<int64_t>(G, 1);
    p.mblocks = (int)mblocks;
    p.wblocks = (int)wblocks;
    p.bm = (int)BM;
    p.bn = (int)BN;
    p.tiles = T;
    // With at least one tile's units per run a tile has two owners at most:
    // they add into a zeroed Y (0 + a + b == 0 + b + a), which costs less
    // than writing and summing partial tiles (M=512, 10240 x 5120: the
    // summing kernel took 10 of 150 us).  With shorter runs the partial
    // tiles go to the workspace.
    p.zero_y = false;
    if (G <= T) {
        for (int64_t g = 1; g < p.grid; g++)
            if (U * g / p.grid % (2 * nb) != 0) {
                p.zero_y = true;
                break;
            }
        p.workspace_bytes = 0;
    } else {
        p.workspace_bytes = (size_t)p.grid * 2 * slot_f4((int)((BM / TILE) * (BN / TILE) / NWQ)) * sizeof(float4);
    }
    p.fmt = fmt;
    p.ok = true;
    return p;
}

}  // namespace

ZeroTiles mmqt_zero_tiles(const MmqtPlan &p, int64_t M, int64_t N, int64_t K, float *Y)
{
    static_assert(MAXZT == MAXG, "one shared tile per run boundary at most");
    ZeroTiles zt;
    if (!p.ok || !p.zero_y)
        return zt;
    zt.y = Y;
    zt.M = M;
    zt.N = N;
    zt.bm = p.bm;
    zt.bn = p.bn;
    zt.wblocks = p.wblocks;
    // the run bounds of launch_mmqt: a bound inside a tile makes it shared
    // (runs of at least a tile: one bound per shared tile)
    const int64_t nh = 2 * (K / QK), U = p.tiles * nh;
    for (int g = 1; g < p.grid; g++) {
        const int64_t u = U * g / p.grid;
        if (u % nh != 0)
            zt.t[zt.count++] = (int)(u / nh);
    }
    return zt;
}

// The tiles with four activation subtiles per wavefront (128 x 256 from
// M = 128, 256 x 128 from 256), else 64 x 256 up to M = 64 and 128 x 128
// above.  The larger tiles lose only where they need partial tiles summed
// from a workspace, the smaller ones do not, and the runs are shorter than
// a super-block (8 units): the summing then outweighs the lookups saved.
// (Measured: 512 x 10240 x 5120, 25 units per run, 137 against 157 us;
// 512 x 5120 x 1024, 4 units per run, 37.5 against 29.7 us; 512 x 17408 x
// 5120 without a workspace, almost every tile with two owners, 206 against
// 235 us; 256 x 17408 x 5120 with one, 118 against 136 us.)
MmqtPlan mmqt_plan(int64_t M, int64_t N, int64_t K, int cus, int fmt)
{
    const MmqtPlan small =
        M <= 2 * TILE ? plan_tiles(M, N, K, cus, fmt, 64, 256) : plan_tiles(M, N, K, cus, fmt, 128, 128);
    if (M >= 128) {
        const int64_t BM = M >= 256 ? 256 : 128, BN = 32768 / BM;
        const MmqtPlan big = plan_tiles(M, N, K, cus, fmt, BM, BN);
        const int64_t units_per_run = big.tiles * 2 * (K / QK) / std::max(big.grid, 1);
        if (big.ok && (big.workspace_bytes == 0 || !small.ok || small.workspace_bytes != 0 || units_per_run >= 8))
            return big;
    }
    return small;
}

hipError_t launch_mmqt(const void *W, const XPlanes &x, float *Y, int64_t N, const MmqtPlan &p, void *workspace,
                       hipStream_t s)
{
    const int cfg = p.bm == 64 ? 0 : p.bm == 128 && p.bn == 128 ? 1 : p.bm == 256 ? 2 : 3;
    if (!p.ok || p.grid < 1 || p.grid > MAXG || (p.workspace_bytes && workspace == nullptr))
        return hipErrorInvalidValue;
    if ((const char *)x.dp != (const char *)x.qp + x.Mp * x.K)
        return hipErrorInvalidValue;
    const int nb = (int)(x.K / QK), nh = 2 * nb;
    const int64_t BN = p.bn;
    const int64_t U = (int64_t)p.mblocks * ((N + BN - 1) / BN) * nh;
    Runs runs;
    for (int g = 0; g <= p.grid; g++) {
        runs.u[g] = (int)(U * g / p.grid);
        if (g < p.grid)
            runs.t[g] = runs.u[g] / nh;
    }
    float *ws = (float *)workspace;
    switch (p.fmt * 4 + cfg) {
    case 4 * FMT_IQ4_XS: return launch_cfg<QCfg<64, 256, FMT_IQ4_XS>>(W, x, Y, ws, N, p, runs, s);
    case 4 * FMT_IQ4_XS + 1: return launch_cfg<QCfg<128, 128, FMT_IQ4_XS>>(W, x, Y, ws, N, p, runs, s);
    case 4 * FMT_IQ4_XS + 2: return launch_cfg<QCfg<256, 128, FMT_IQ4_XS>>(W, x, Y, ws, N, p, runs, s);
    case 4 * FMT_IQ4_XS + 3: return launch_cfg<QCfg<128, 256, FMT_IQ4_XS>>(W, x, Y, ws, N, p, runs, s);
    case 4 * FMT_IQ4_NL: return launch_cfg<QCfg<64, 256, FMT_IQ4_NL>>(W, x, Y, ws, N, p, runs, s);
    case 4 * FMT_IQ4_NL + 1: return launch_cfg<QCfg<128, 128, FMT_IQ4_NL>>(W, x, Y, ws, N, p, runs, s);
    case 4 * FMT_IQ4_NL + 2: return launch_cfg<QCfg<256, 128, FMT_IQ4_NL>>(W, x, Y, ws, N, p, runs, s);
    case 4 * FMT_IQ4_NL + 3: return launch_cfg<QCfg<128, 256, FMT_IQ4_NL>>(W, x, Y, ws, N, p, runs, s);
    case 4 * FMT_Q4_0: return launch_cfg<QCfg<64, 256, FMT_Q4_0>>(W, x, Y, ws, N, p, runs, s);
    case 4 * FMT_Q4_0 + 1: return launch_cfg<QCfg<128, 128, FMT_Q4_0>>(W, x, Y, ws, N, p, runs, s);
    case 4 * FMT_Q4_0 + 2: return launch_cfg<QCfg<256, 128, FMT_Q4_0>>(W, x, Y, ws, N, p, runs, s);
    case 4 * FMT_Q4_0 + 3: return launch_cfg<QCfg<128, 256, FMT_Q4_0>>(W, x, Y, ws, N, p, runs, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace iq4xs
