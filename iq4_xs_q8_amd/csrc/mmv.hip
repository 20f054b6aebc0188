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
//    length (the run bounds are computed on the host and passed in).  The grid never has more workgroups than tiles, so a run covers at
//    least one tile's worth of units and a tile is shared by at most two
//    workgroups: every compute unit gets the same work whatever the shape.
//  * A run is walked in chunks of up to CH super-blocks of one tile, chunk
//    windows starting at even super-blocks (with K/256 even, every window is
//    16-byte aligned and ends inside its row).  Every wavefront walks the
//    chunk sequence itself with a scalar cursor.
//  * A chunk's weights (32 rows x up to CH*136 contiguous bytes per row) and
//    the activations of its sub-blocks (one contiguous range of the
//    sub-block-major planes) go straight from memory into one of NBUF LDS
//    buffers with 16-byte buffer loads that write LDS (no register staging):
//    each load instruction fills 1 KB of the buffer, its lanes reading the
//    global pieces that belong there, so every HBM access is a long run of
//    whole rows.  The loads of a chunk are issued NBUF-1 chunks ahead of its
//    use; a step waits for its own loads of the chunk to land, meets the other
//    wavefronts at one barrier, issues the loads of the chunk NBUF-1 ahead into
//    the buffer freed by the barrier, then computes.
//  * Sixteen wavefronts compute: wavefront w takes sub-block w%8 of the
//    chunk's super-blocks w/8, w/8+2, ... from LDS (the 8 index bytes and
//    header of its lane's row, the 16 activation bytes of its lane's row;
//    rows past M read a zero row).  The two halves of a wavefront hold the
//    same 32 rows, so each decodes the scales of one of two super-blocks and
//    they swap them with one cross-half lane permute.
//  * When a tile's units end, the wavefronts' partial tiles are summed in LDS
//    in wavefront order.  A tile owned by one workgroup is stored; a tile
//    shared by two is added into Y with one atomic add per element, Y having
//    been zeroed beforehand: 0 + a + b == 0 + b + a in floating point, so the
//    result does not depend on which workgroup comes first.
#include "common.hpp"
#include "stream.hpp"

#include <type_traits>
#include <utility>

namespace iq4xs {
namespace {

using namespace stream;

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int TILE = 32;
constexpr int NW = 16;                     // wavefronts per workgroup
constexpr int NT = 64 * NW;                // threads per workgroup
constexpr int PAR = NW / SUBS;             // wavefronts per sub-block
// LDS row stride of a weight chunk: CH units of UB bytes (136 or 144) rounded
// up to an odd number of 16-byte units, so that the 32 rows of an MFMA operand
// read spread over the banks.
constexpr int wrow_bytes(int ch, int ub)
{
    const int u = (ch * ub + 15) / 16;
    return 16 * (u % 2 ? u : u + 1);
}

// LIVE result registers, activation rows padded to MPC (>= Mp) in LDS, CH
// super-blocks per chunk, NBUF chunk buffers.  SPLIT (M <= 4): the
// activation rows go to MFMA rows 0..LIVE-1 and 4..4+LIVE-1, so that both
// halves of a wavefront hold real rows in their LIVE result registers (row
// h*LIVE + r in register r of half h): half the rescale work of putting all
// rows in the first half.  F: the weight format; a "super-block" below is
// its 256-weight unit of UB bytes.
template <int LIVE_, int MPC_, int CH_, int NBUF_, bool SPLIT_ = false, int F_ = FMT_IQ4_XS>
struct Cfg {
    static constexpr int LIVE = LIVE_, MPC = MPC_, CH = CH_, NBUF = NBUF_;
    static constexpr bool SPLIT = SPLIT_;
    static constexpr int F = F_, UB = sblk_bytes(F_);
    static constexpr int WROW = wrow_bytes(CH, UB);
    static constexpr int W_PR = CH * UB / 16;                                 // pieces per row
    // one chunk buffer: weights [32][WROW] (padded to whole KB), activations
    // [CH*8][MA][32], scales [CH*8][Mp] (padded to whole KB), a 32-byte zero
    // row (the operand of rows >= M) and slack for the scales a lane reads
    // past the last sub-block's rows (activations: MA rows per sub-block in
    // LDS, MA >= M); besides the buffers, one 1 KB area that load slots
    // without a job fill (shared: nothing reads it)
    static constexpr int MA = SPLIT ? 2 * LIVE : LIVE < 4 ? LIVE : MPC;
    static constexpr int W_BYTES = round_up_c(TILE * WROW, 1024);
    static constexpr int A_OFF = W_BYTES, A_BYTES = CH * SUBS * MA * SB;
    static constexpr int D_OFF = A_OFF + A_BYTES, D_BYTES = round_up_c(CH * SUBS * MPC * 4, 1024);
    static constexpr int Z_OFF = D_OFF + D_BYTES;
    static constexpr int BUF = Z_OFF + 32 + 128;
    static constexpr int RED = LIVE * 64 * (NW + 1) * 4;                      // partial tiles
    static constexpr int TOTAL = NBUF * BUF + RED + 1024;
    template <int B>
    static __device__ __forceinline__ char *buf() { return lds_area<B, BUF>(); }
    static __device__ __forceinline__ float *red() { return reinterpret_cast<float *>(lds_area<-1, RED>()); }
    static __device__ __forceinline__ char *dump() { return lds_area<-2, 1024>(); }
    // A chunk is copied by load jobs of 1 KB of a buffer each: JW of weights,
    // JQ of activations, JD of scales.  Every wavefront issues SLOTS loads
    // per chunk: wavefronts 0..WA-1 take the weight jobs, the others the
    // activation jobs and then the scale jobs; slots left over load nothing
    // into the dump area.
    static constexpr int JW = W_BYTES / 1024, JQ = A_BYTES / 1024, JD = D_BYTES / 1024;
    static constexpr int SLOTS = (JW + JQ + JD + NW - 1) / NW;
    static constexpr int WA = (JW + SLOTS - 1) / SLOTS;
    static_assert(NW == 16, "the flush sums 16 partials per output in a row of 16 lanes");
    static_assert(A_BYTES % 1024 == 0 && BUF % 16 == 0, "whole 1 KB load jobs, aligned buffers");
    static_assert(WA + (JQ + JD + SLOTS - 1) / SLOTS <= NW, "load jobs fit the wavefronts");
    static_assert(CH % PAR == 0 && CH % 2 == 0, "every wavefront gets the same super-blocks");
    static_assert(NBUF >= 2 && TOTAL <= 160 * 1024, "LDS budget");
    static_assert(!SPLIT || (LIVE <= 2 && MPC == 4), "split rows: M <= 4");
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
// 16 (M <= 32).  MPC: a bound on the padded activation rows Mp.  GRP: grp
// holds several matrices (else only matrix 0 is read, at fixed offsets).
template <class C, bool GRP>
__global__ void __launch_bounds__(NT, 1)
k_mmv(MmvGroup grp, const int8_t *__restrict__ qp, int M, int K, int Mp, int nb, Runs runs)
{
    constexpr int LIVE = C::LIVE, CH = C::CH, NBUF = C::NBUF, SLOTS = C::SLOTS;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int s = wave % SUBS, par = wave / SUBS;             // sub-block, first super-block
    const int col = lane & 31, h = lane >> 5;
    // this workgroup's run of units
    const int g = blockIdx.x;
    const int ua = runs.u[g], ub = runs.u[g + 1];
    constexpr int UB = C::UB;
    const uint32_t row_bytes = (uint32_t)nb * UB;

    // ---- chunk copy: fixed per-lane geometry ------------------------------
    // descriptors over the whole weight matrix and over both activation planes
    // (contiguous: scales at qp + Mp*K); offsets are per lane, so rows past N
    // and pieces past a plane read as zero
    const int dp_at = Mp * K;
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc((void *)qp, (short)0, dp_at + Mp * (K / SB) * 4, BUFFER_FLAGS);
    const bool w_group = wave < C::WA;                        // (uniform)
    // per slot: the LDS offset its load fills inside a buffer and whether it
    // holds scales (both uniform), this lane's global offset relative to the
    // chunk's base, and the key that decides whether the lane's piece belongs
    // to the chunk
    int p_dst[SLOTS];
    bool p_scale[SLOTS];
    uint32_t p_go[SLOTS];
    int p_key[SLOTS];
    // (geometry in 16-byte pieces: piece i of a 1 KB job is lane i's)
    constexpr uint32_t LIM = 64 * NW * SLOTS;                 // bound on the piece indices
#pragma unroll
    for (int k = 0; k < SLOTS; k++) {
        if (w_group) {
            const int job = wave * SLOTS + k;
            const uint32_t pi = 64 * job + lane;               // piece of the weight area
            const uint32_t r = div_small<C::WROW / 16, LIM>(pi);
            const uint32_t c = pi - (uint32_t)__umul24(r, C::WROW / 16);
            const bool ok = job < C::JW && r < TILE && c < C::W_PR;
            p_dst[k] = job < C::JW ? 1024 * job : -1;          // (-1: the dump area)
            p_scale[k] = false;
            p_go[k] = ok ? r * row_bytes + 16 * c : OOB;
            p_key[k] = ok ? (int)(16 * c + 15) : -(1 << 30);   // piece bytes [16c, 16c+16)
        } else {
            const int job = (wave - C::WA) * SLOTS + k;       // activation jobs, then scales
            const bool isq = job < C::JQ, isd = !isq && job < C::JQ + C::JD;
            const uint32_t pi = 64 * (isq ? job : job - C::JQ) + lane;
            // activation piece: half `hf` of row m of sub-block sb, whose plane
            // holds Mp rows per sub-block
            const uint32_t sb2 = div_small<2 * C::MA, LIM>(pi);
            const uint32_t m = (pi - 2 * C::MA * sb2) >> 1, hf = pi & 1;
            const int qo = (int)(((uint32_t)__umul24(sb2, (uint32_t)Mp) + m) * SB + 16 * hf);
            const int at = (int)(16 * pi);
            p_dst[k] = isq ? C::A_OFF + 1024 * job : isd ? C::D_OFF + 1024 * (job - C::JQ) : -1;
            p_scale[k] = isd;
            p_go[k] = isq ? (uint32_t)qo : isd ? (uint32_t)at : OOB;
            p_key[k] = isq ? qo : isd ? at : 1 << 30;
        }
    }
    // Issue the loads of chunk c into buffer B: weight pieces holding none of
    // the chunk's super-blocks (the window starts at j0 & ~1), and activation
    // or scale pieces past the chunk, read nothing and fill zeros.  Every
    // wavefront issues SLOTS loads per chunk, also for chunks past the run,
    // so the wait counts are the same on every path.
    auto issue = [&](const Chunk &c, auto bc) __attribute__((always_inline)) {
        char *buf = C::template buf<decltype(bc)::value>();
        if (w_group) {
            // the chunk's matrix (tiles are numbered across the matrices)
            const int gi = GRP ? grp.matrix_of(c.t) : 0;
            const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
                (void *)grp.w[gi], (short)0, (int)((uint32_t)grp.n[gi] * row_bytes), BUFFER_FLAGS);
            const int lo = (c.j0 & 1) * UB, hi = lo + c.cl * UB;
            const uint32_t base = (uint32_t)(c.t - grp.t0[gi]) * TILE * row_bytes + (c.j0 & ~1) * UB;
#pragma unroll
            for (int k = 0; k < SLOTS; k++) {
                const bool need = (uint32_t)(p_key[k] - lo) < (uint32_t)(hi - lo + 15);
                load_lds16(wr, p_dst[k] < 0 ? C::dump() : buf + p_dst[k], need ? p_go[k] + base : OOB);
            }
        } else {
            const int qn = c.cl * SUBS * Mp * SB, dn = c.cl * SUBS * Mp * 4;
            const uint32_t qbase = (uint32_t)c.j0 * SUBS * Mp * SB, dbase = (uint32_t)dp_at + c.j0 * SUBS * Mp * 4;
#pragma unroll
            for (int k = 0; k < SLOTS; k++) {
                const bool need = p_key[k] < (p_scale[k] ? dn : qn);
                load_lds16(xr, p_dst[k] < 0 ? C::dump() : buf + p_dst[k],
                           need ? p_go[k] + (p_scale[k] ? dbase : qbase) : OOB);
            }
        }
    };

    float acc[LIVE];
#pragma unroll
    for (int r = 0; r < LIVE; r++)
        acc[r] = 0.0f;
    float *red = C::red();
    // Sum the wavefronts' partial tiles: output o (LIVE*64 of them) gathers
    // its 16 partials at red[o*17 + wave] and adds them in one fixed balanced
    // tree over the wavefront index, whatever LIVE is (so a row's result does
    // not depend on how many rows are computed with it).  After the barrier GS
    // consecutive lanes take one output: each adds 16/GS partials (the lower
    // levels of the tree), row shifts add the lanes' sums (the upper levels;
    // the total lands in the group's last lane).  The reads are done before
    // this wavefront reaches the next step's barrier, which every later
    // flush's writes follow.
    auto flush = [&](int t, bool owned) __attribute__((always_inline)) {
#pragma unroll
        for (int r = 0; r < LIVE; r++) {
            red[(r * 64 + lane) * (NW + 1) + wave] = acc[r];
            acc[r] = 0.0f;
        }
        __builtin_amdgcn_s_waitcnt(WAIT_LDS);
        raw_barrier();
        constexpr int GS = LIVE == 1 ? 16 : LIVE == 2 ? 8 : LIVE <= 4 ? 4 : LIVE == 8 ? 2 : 1;
        constexpr int PER = NW / GS;
        const int o = tid / GS, part = tid % GS;
        if (o < LIVE * 64) {
            // (the in-lane part continues the same balanced tree)
            float a[PER];
#pragma unroll
            for (int q = 0; q < PER; q++)
                a[q] = red[o * (NW + 1) + part * PER + q];
#pragma unroll
            for (int d = 1; d < PER; d *= 2)
#pragma unroll
                for (int q = 0; q < PER; q += 2 * d)
                    a[q] += a[q + d];
            float v = a[0];
            if constexpr (GS >= 2)
                v += shr_row(v, std::integral_constant<int, 1>());
            if constexpr (GS >= 4)
                v += shr_row(v, std::integral_constant<int, 2>());
            if constexpr (GS >= 8)
                v += shr_row(v, std::integral_constant<int, 4>());
            if constexpr (GS >= 16)
                v += shr_row(v, std::integral_constant<int, 8>());
            const int gi = GRP ? grp.matrix_of(t) : 0;
            const int N = grp.n[gi];
            float *const Y = grp.y[gi];
            const int r = o >> 6, l2 = o & 63;
            const int m = C::SPLIT ? (l2 >> 5) * LIVE + r : 8 * (r / 4) + 4 * (l2 >> 5) + (r % 4);
            const int n = (t - grp.t0[gi]) * TILE + (l2 & 31);
            if (part == GS - 1 && m < M && n < N) {
                if (owned)
                    Y[(int64_t)m * N + n] = v;
                else
                    atomicAdd(Y + (int64_t)m * N + n, v);
            }
        }
    };

    // per-lane LDS read offsets inside a chunk buffer (rows >= M: the zero row)
    const int w_lane = col * C::WROW;
    // the activation row feeding this lane's MFMA row (M or more: the zero row)
    const int arow = C::SPLIT ? ((col < 8 && (col & 3) < LIVE) ? ((col >> 2) & 1) * LIVE + (col & 3) : M) : col;
    const int a_step = arow < M ? C::MA * SB : 0;
    // (offsets for the wavefronts that take the chunk's even super-blocks; the
    // others add one super-block's worth, see compute)
    int a_off[CH / PAR], d_off[CH / PAR];
#pragma unroll
    for (int i = 0; i < CH / PAR; i++) {
        const int sb = (PAR * i) * SUBS + s;                  // sub-block within the chunk
        a_off[i] = (arow < M ? C::A_OFF + arow * SB : C::Z_OFF) + 16 * h + sb * a_step;
        d_off[i] = C::D_OFF + (C::SPLIT ? 4 * LIVE * h : 16 * h) + 4 * sb * Mp;
    }
    auto compute = [&](const Chunk &c, auto bc) __attribute__((always_inline)) {
        const char *B = C::template buf<decltype(bc)::value>();
        const char *wchunk = B + w_lane + (c.j0 & 1) * UB;    // the window starts at j0 & ~1
        // Wavefront pair `par` takes the super-blocks whose absolute index j
        // has j % 2 == par, in increasing order, whatever the chunk length
        // (which depends on M) and wherever the chunk starts: every output
        // then sums the same products in the same order for every M.
        const int pc = par ^ (c.j0 & 1);                      // first one within the chunk (uniform)
        const int a_pc = pc * SUBS * a_step, d_pc = pc * SUBS * 4 * Mp;
        // The I = CH/PAR super-blocks go in groups of GI whose LDS reads are
        // issued together, so that reads, lookups and MFMAs of different
        // super-blocks overlap; groups past the chunk's end are skipped, and
        // a super-block past it inside a group is computed with a zero scale
        // (its LDS reads stay inside the buffer).
        constexpr int I = CH / PAR, DQ = LIVE >= 4 ? LIVE / 4 : 1;
        constexpr int GI = I < 2 ? I : 2;
#pragma unroll
        for (int g = 0; g < I; g += GI) {
            if (pc + PAR * g >= c.cl)                        // (uniform)
                break;
            uint2 hdr[GI], q[GI];
            v4i ax[GI];
            float4 dx[GI][DQ];
            // With two super-blocks in the group, the two halves of the
            // wavefront (same rows) each decode one of the two scales and
            // swap them.
            if constexpr (GI == 2)
                hdr[0] = unit_scale_raw<C::F>(wchunk + (pc + PAR * (g + h)) * UB, s);
#pragma unroll
            for (int k = 0; k < GI; k++) {
                const char *wrow = wchunk + (pc + PAR * (g + k)) * UB;
                if constexpr (GI != 2)
                    hdr[k] = unit_scale_raw<C::F>(wrow, s);
                q[k] = unit_qs<C::F>(wrow, s, h);
                ax[k] = *reinterpret_cast<const v4i *>(B + a_off[g + k] + a_pc);
#pragma unroll
                for (int qd = 0; qd < DQ; qd++)
                    if constexpr (!C::SPLIT)
                        dx[k][qd] = *reinterpret_cast<const float4 *>(B + d_off[g + k] + d_pc + 32 * qd);
                    else if constexpr (LIVE == 1)
                        dx[k][qd] = make_float4(*reinterpret_cast<const float *>(B + d_off[g + k] + d_pc), 0.f, 0.f, 0.f);
                    else {
                        const float2 d2 = *reinterpret_cast<const float2 *>(B + d_off[g + k] + d_pc);
                        dx[k][qd] = make_float4(d2.x, d2.y, 0.f, 0.f);
                    }
            }
            // (all of the group's reads are issued before any of them is used)
            __builtin_amdgcn_sched_barrier(0);
            float sw[GI];
            if constexpr (GI == 2) {
                // (a super-block past the chunk gets a zero scale)
                const float own = unit_scale_dec<C::F>(hdr[0], s, pc + PAR * (g + h) < c.cl);
                const uint32_t ob = __builtin_bit_cast(uint32_t, own);
                // (lanes 0-31 of the first result: their own scale; lanes
                // 32-63: that of lanes 0-31; the second result the converse)
                const auto both = __builtin_amdgcn_permlane32_swap(ob, ob, false, false);
                sw[0] = __builtin_bit_cast(float, (uint32_t)both[0]);
                sw[1] = __builtin_bit_cast(float, (uint32_t)both[1]);
            } else {
#pragma unroll
                for (int k = 0; k < GI; k++)
                    sw[k] = unit_scale_dec<C::F>(hdr[k], s, pc + PAR * (g + k) < c.cl);
            }
            v16i D[GI];
#pragma unroll
            for (int k = 0; k < GI; k++) {
                uint32_t wa[4], wb[4];
                expand8_split<C::F>(q[k].x, q[k].y, wa, wb);
                const v4i ba = {(int)wa[0], (int)wa[1], (int)wa[2], (int)wa[3]};
                const v4i bb = {(int)wb[0], (int)wb[1], (int)wb[2], (int)wb[3]};
                const v16i zero = {0};
                D[k] = __builtin_amdgcn_mfma_i32_32x32x32_i8(
                    ax[k], bb, __builtin_amdgcn_mfma_i32_32x32x32_i8(ax[k], ba, zero, 0, 0, 0), 0, 0, 0);
            }
            // (the group's products are all issued before the first is read,
            // each into registers of its own)
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < GI; k++)
                epilogue<LIVE>(D[k], sw[k], dx[k], acc);
#pragma unroll
            for (int k = 0; k < GI; k++)
                keep_live(D[k]);
        }
        if (c.flags & 1)                                      // the tile's units end here
            flush(c.t, (c.flags & 2) != 0);
    };

    // the zero rows of the buffers (published by the first step's barrier)
    if (tid < 8)
        static_for(std::make_integer_sequence<int, NBUF>(), [&](auto bc) {
            reinterpret_cast<uint32_t *>(C::template buf<decltype(bc)::value>() + C::Z_OFF)[tid] = 0u;
        });

    Cursor cur;
    cur.ua = ua;
    cur.ub = ub;
    cur.nb = nb;
    cur.u = ua;
    cur.t = runs.t[g];
    cur.j = ua - cur.t * nb;
    // (every chunk is CH super-blocks long where the run allows: a short first
    // chunk, to start computing earlier, measured slower on every shape)
    Chunk info[NBUF];
    static_for(std::make_integer_sequence<int, NBUF - 1>(), [&](auto bc) {
        constexpr int b = decltype(bc)::value;
        info[b] = cur.next(CH);
        issue(info[b], bc);
    });
    // Step on buffer b: wait for this wavefront's loads of its chunk (the
    // loads of the NBUF-2 chunks issued after it stay in flight), meet the
    // other wavefronts (all loads of the chunk have landed, and the buffer
    // computed last is free), refill that buffer NBUF-1 chunks ahead, compute.
    auto step = [&](auto bc) __attribute__((always_inline)) {
        constexpr int b = decltype(bc)::value, nxt = (b + NBUF - 1) % NBUF;
        if (info[b].cl == 0)
            return false;                                     // (uniform) the run is done
        __builtin_amdgcn_s_waitcnt(wait_vm_lds(SLOTS * (NBUF - 2)));
        raw_barrier();
        info[nxt] = cur.next(CH);
        issue(info[nxt], std::integral_constant<int, nxt>());
        compute(info[b], bc);
        return true;
    };
    bool go = true;
    do
        static_for(std::make_integer_sequence<int, NBUF>(), [&](auto bc) __attribute__((always_inline)) {
            if (go)
                go = step(bc);
        });
    while (go);
    // no load may still write this workgroup's LDS when it ends
    __builtin_amdgcn_s_waitcnt(wait_vm_lds(0));
}

template <class C>
hipError_t launch_c(const MmvGroup &grp, const XPlanes &x, const MmvPlan &p, hipStream_t s)
{
    const int nb = (int)(x.K / QK);
    const int64_t T = grp.t0[grp.count];
    // (the kernel reads both planes through one descriptor)
    if ((const char *)x.dp != (const char *)x.qp + x.Mp * x.K || x.Mp > C::MPC || x.M > C::MA)
        return hipErrorInvalidValue;
    const int64_t U = T * nb;
    if (p.grid < 1 || p.grid > MAXG)
        return hipErrorInvalidValue;
    Runs runs;
    for (int g = 0; g <= p.grid; g++) {
        runs.u[g] = (int)(U * g / p.grid);
        if (g < p.grid)
            runs.t[g] = runs.u[g] / nb;
    }
    if (grp.count > 1)
        hipLaunchKernelGGL((k_mmv<C, true>), dim3((unsigned)p.grid), dim3(NT), 0, s, grp, x.qp, (int)x.M,
                           (int)x.K, (int)x.Mp, nb, runs);
    else
        hipLaunchKernelGGL((k_mmv<C, false>), dim3((unsigned)p.grid), dim3(NT), 0, s, grp, x.qp, (int)x.M,
                           (int)x.K, (int)x.Mp, nb, runs);
    return hipGetLastError();
}

}  // namespace

MmvPlan mmv_plan_group(int64_t M, const int64_t *N, int count, int64_t K, int cus, int fmt)
{
    MmvPlan p;
    const int64_t nb = K / QK, row_bytes = nb * sblk_bytes(fmt);
    const int64_t Mp = round_up(M, MPAD);
    if (count < 1 || count > MAXGRP)
        return p;
    // K/256 even (16-byte aligned chunk windows) and below 2^16; 32-bit
    // buffer offsets and unit counts: each weight matrix, the activation
    // planes and (all tiles)*K/256 stay below 2^31
    int64_t T = 0;
    for (int g = 0; g < count; g++) {
        if (N[g] < 1 || N[g] * row_bytes >= (1LL << 31))
            return p;
        T += (N[g] + TILE - 1) / TILE;
    }
    // (144-byte units are 16-byte aligned wherever a window starts)
    if (M < 1 || M > TILE || (fmt == FMT_IQ4_XS && nb % 2 != 0) || nb >= (1 << 16) ||
        Mp * K + Mp * K / 8 >= (1LL << 31) || T * nb >= (1LL << 31))
        return p;
    const int64_t U = T * nb;
    p.grid = (int)(T < cus ? T : cus);
    if (p.grid > MAXG)
        p.grid = MAXG;
    p.live = M <= 4 ? (int)M : M <= 8 ? 4 : M <= 16 ? 8 : 16;
    p.zero_y = false;
    for (int64_t g = 1; g < p.grid; g++)
        if (U * g / p.grid % nb != 0) {
            p.zero_y = true;                                // some tile has two owners
            break;
        }
    p.fmt = fmt;
    p.ok = true;
    return p;
}

MmvPlan mmv_plan(int64_t M, int64_t N, int64_t K, int cus, int fmt) { return mmv_plan_group(M, &N, 1, K, cus, fmt); }

MmvGroup mmv_group(const void *const *W, float *const *Y, const int64_t *N, int count)
{
    MmvGroup g{};
    g.count = count;
    g.t0[0] = 0;
    for (int i = 0; i < count; i++) {
        g.w[i] = (const uint8_t *)W[i];
        g.y[i] = Y[i];
        g.n[i] = (int)N[i];
        g.t0[i + 1] = g.t0[i] + (int)((N[i] + TILE - 1) / TILE);
    }
    for (int i = count; i < MAXGRP; i++)
        g.t0[i + 1] = g.t0[count];
    return g;
}

template <int F>
hipError_t launch_fmt(const MmvGroup &grp, const XPlanes &x, const MmvPlan &p, hipStream_t s)
{
    switch (p.live) {
    // (M = 2..4: rows split over both halves of the MFMA tile; measured 2-4%
    // faster than all rows in the first half)
    case 1: return launch_c<Cfg<1, 4, 8, 3, false, F>>(grp, x, p, s);
    case 2: return launch_c<Cfg<1, 4, 8, 3, true, F>>(grp, x, p, s);
    case 3: return launch_c<Cfg<2, 4, 8, 3, true, F>>(grp, x, p, s);
    case 4:
        return x.Mp <= 4 ? launch_c<Cfg<2, 4, 8, 3, true, F>>(grp, x, p, s)
                         : launch_c<Cfg<4, 8, 4, 3, false, F>>(grp, x, p, s);
    case 8: return launch_c<Cfg<8, 16, 4, 3, false, F>>(grp, x, p, s);
    case 16: return launch_c<Cfg<16, 32, 2, 3, false, F>>(grp, x, p, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_mmv_group(const MmvGroup &grp, const XPlanes &x, const MmvPlan &p, hipStream_t s)
{
    if (!p.ok || grp.count < 1 || grp.count > MAXGRP)
        return hipErrorInvalidValue;
    switch (p.fmt) {
    case FMT_IQ4_XS: return launch_fmt<FMT_IQ4_XS>(grp, x, p, s);
    case FMT_IQ4_NL: return launch_fmt<FMT_IQ4_NL>(grp, x, p, s);
    case FMT_Q4_0: return launch_fmt<FMT_Q4_0>(grp, x, p, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_mmv(const void *W, const XPlanes &x, float *Y, int64_t N, const MmvPlan &p, hipStream_t s)
{
    return launch_mmv_group(mmv_group(&W, &Y, &N, 1), x, p, s);
}

}  // namespace iq4xs
