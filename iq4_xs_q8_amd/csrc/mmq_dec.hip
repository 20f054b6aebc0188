// mmq_dec.hip -- IQ4_XS x Q8_1 on the int8 matrix cores for decode-sized M
// (M <= 32: one 32-row activation tile).
//
// Same arithmetic as mmq.hip (one v_mfma_i32_32x32x32_i8 per 32-element
// sub-block, fp32 rescale by d_w*(ls-32)*d_x; "V100TPS engine log",
// agent-report.daedalus.work/V100TPS/engine.html, batched IQ4_XS kernel
// section), organised so the weight stream runs near HBM speed:
//
//  * A workgroup owns NW*32 output columns (NW wavefronts, 32 columns each)
//    and a slice of KR super-blocks along K.  Its activations for the slice
//    (at most 32 rows x KR*256 int8 values, plus their block scales) are
//    copied to LDS once.  Rows M..31 of the MFMA tile read an all-zero row.
//  * Weights are loaded coalesced: two consecutive super-blocks of a row are
//    272 contiguous bytes, and the 64 lanes of a wavefront read them as
//    consecutive 8-byte pieces (32 rows x 34 pieces = 17 loads per lane).  The
//    pieces go to a per-wavefront LDS tile (rows padded to 280 bytes, which
//    spreads the MFMA-layout reads over all banks) and each lane then reads
//    the index bytes of its own row and half sub-block from there.  The next
//    stage's loads are in flight while the current stage is computed.
//  * K is split over KS workgroups when the columns alone do not fill the
//    chip; each writes its partial tile to a workspace and a separate kernel
//    adds the KS partials in order 0..KS-1 (deterministic, no atomics).
#include "common.hpp"

namespace iq4xs {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int TILE = 32;
constexpr int BUFFER_FLAGS = 0x00020000;   // raw buffer resource, gfx9 family
constexpr int SJ = 2;                      // super-blocks per weight stage
constexpr int WPIECES = SJ * WBLK / 8;     // 8-byte pieces per row per stage (34)
constexpr int WSTRIDE = SJ * WBLK + 8;     // LDS bytes per weight row (280)
constexpr int WLOADS = TILE * WPIECES / 64;  // loads per lane per stage (17)
static_assert(TILE * WPIECES % 64 == 0, "a stage is a whole number of wave loads");
constexpr int XROW_PAD = 16;               // bytes added to each LDS activation row
constexpr int XGRAN = 8;                   // activation granules staged per thread per round
constexpr size_t LDS_BUDGET = 76 * 1024;   // two workgroups per CU

// Rescale one sub-block's MFMA result into acc.
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

// LIVE: result registers that can hold a real row: 1,2,3,4 (M <= LIVE, lanes
// 0-31 only; LIVE = 4 also serves M <= 8 through lanes 32-63), 8 (M <= 16),
// 16 (M <= 32).
template <int LIVE, int NW>
__global__ void __launch_bounds__(64 * NW)
k_mmq_dec(const uint8_t *__restrict__ W, const int8_t *__restrict__ qp, const float *__restrict__ dp,
          float *__restrict__ out, int64_t M, int64_t N, int64_t K, int64_t Mp)
{
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: descriptors stay scalar
    const int col = lane & 31, h = lane >> 5;
    const int64_t nb = K / QK;
    const int ks = gridDim.y, z = blockIdx.y;
    const int64_t j0 = nb * z / ks, j1 = nb * (z + 1) / ks;
    const int kr = (int)(j1 - j0);
    const int rows = M < TILE ? (int)M : TILE;
    const int xstride = kr * QK + XROW_PAD;
    int8_t *xs = reinterpret_cast<int8_t *>(lds);                        // [rows+1][xstride]
    float *ds = reinterpret_cast<float *>(lds + (rows + 1) * xstride);   // [kr*8][32]
    char *wt = reinterpret_cast<char *>(ds + kr * SUBS * TILE) + wave * (TILE * WSTRIDE);
    char *sink = reinterpret_cast<char *>(ds + kr * SUBS * TILE) + NW * (TILE * WSTRIDE);   // 16 bytes

    // weights of this wave's 32 rows; rows past N and bytes past the matrix read as 0
    const int64_t n0 = ((int64_t)blockIdx.x * NW + wave) * TILE;
    const uint32_t row_bytes = (uint32_t)(nb * WBLK);
    const int64_t n_rows = N - n0 < TILE ? (N - n0 > 0 ? N - n0 : 0) : TILE;
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(W + (n0 < N ? n0 : 0) * (int64_t)row_bytes), (short)0, (int)(n_rows * row_bytes),
        BUFFER_FLAGS);
    // the piece each lane loads in load k of a stage: row r, piece c
    uint32_t goff[WLOADS];
    int loff[WLOADS];
#pragma unroll
    for (int k = 0; k < WLOADS; k++) {
        const int idx = lane + 64 * k;
        const int r = idx / WPIECES, c = idx - r * WPIECES;
        goff[k] = (uint32_t)r * row_bytes + (uint32_t)j0 * WBLK + 8 * c;
        loff[k] = r * WSTRIDE + 8 * c;
    }
    uint2 wreg[WLOADS];
    auto load_stage = [&](int st) {
#pragma unroll
        for (int k = 0; k < WLOADS; k++)
            wreg[k] = __builtin_bit_cast(
                uint2, __builtin_amdgcn_raw_buffer_load_b64(wr, goff[k] + (uint32_t)(st * SJ * WBLK), 0, 0));
    };
    auto store_stage = [&]() {
#pragma unroll
        for (int k = 0; k < WLOADS; k++)
            *reinterpret_cast<uint2 *>(wt + loff[k]) = wreg[k];
    };
    load_stage(0);

    // activations and their scales -> LDS, XGRAN granules of 16 bytes per
    // thread per round, loads branch-free (clamped, zeroed) so they overlap
    const int gran_row = kr * 16;
    const int gran_x = (rows + 1) * gran_row;
    for (int g0 = 0; g0 < gran_x; g0 += 64 * NW * XGRAN) {
        v4i v[XGRAN];
#pragma unroll
        for (int i = 0; i < XGRAN; i++) {
            const int g = g0 + tid + 64 * NW * i;
            const int r = g / gran_row, c = g - r * gran_row;
            const bool real = g < gran_x && r < rows;
            const v4i t = *reinterpret_cast<const v4i *>(qp + (real ? r : 0) * K + j0 * QK + 16 * (real ? c : 0));
            const v4i zero = {0, 0, 0, 0};
            v[i] = real ? t : zero;
        }
#pragma unroll
        for (int i = 0; i < XGRAN; i++) {   // unconditional: granules past the end go to the sink
            const int g = g0 + tid + 64 * NW * i;
            const int r = g / gran_row, c = g - r * gran_row;
            char *dst = g < gran_x ? reinterpret_cast<char *>(xs + r * xstride + 16 * c) : sink;
            *reinterpret_cast<v4i *>(dst) = v[i];
        }
    }
    const int gran_d = kr * SUBS * (TILE / 4);          // float4 granules of scales
    for (int g = tid; g < gran_d; g += 64 * NW) {
        const int sb = g / (TILE / 4), c = g - sb * (TILE / 4);
        *reinterpret_cast<float4 *>(ds + 4 * g) =
            *reinterpret_cast<const float4 *>(dp + (SUBS * j0 + sb) * Mp + 4 * c);
    }
    store_stage();
    __syncthreads();

    float acc[LIVE];
#pragma unroll
    for (int r = 0; r < LIVE; r++)
        acc[r] = 0.0f;
    const int8_t *xrow = xs + (col < rows ? col : rows) * xstride;
    const char *wrow = wt + col * WSTRIDE;
    const int nstages = (kr + SJ - 1) / SJ;
    for (int st = 0; st < nstages; st++) {
        load_stage(st + 1 < nstages ? st + 1 : st);     // next stage in flight meanwhile
#pragma unroll
        for (int jj = 0; jj < SJ; jj++) {
            const int jl = st * SJ + jj;                // super-block within the slice
            if (jl < kr) {
                const uint2 hdr = *reinterpret_cast<const uint2 *>(wrow + jj * WBLK);
#pragma unroll
                for (int s = 0; s < SUBS; s++) {
                    const uint2 q = *reinterpret_cast<const uint2 *>(wrow + jj * WBLK + QS_OFF + 16 * s + 8 * h);
                    const v4i ax = *reinterpret_cast<const v4i *>(xrow + jl * QK + 32 * s + 16 * h);
                    float4 dx[LIVE >= 4 ? LIVE / 4 : 1];
#pragma unroll
                    for (int qd = 0; qd < (LIVE >= 4 ? LIVE / 4 : 1); qd++)
                        dx[qd] = *reinterpret_cast<const float4 *>(ds + (jl * SUBS + s) * TILE + 4 * h + 8 * qd);
                    uint32_t wv[4];
                    expand8(q.x, q.y, wv);
                    const v4i bw = {(int)wv[0], (int)wv[1], (int)wv[2], (int)wv[3]};
                    const v16i zero = {0};
                    const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(ax, bw, zero, 0, 0, 0);
                    epilogue<LIVE>(D, sub_scale(hdr.x, hdr.y, s), dx, acc);
                }
            }
        }
        store_stage();                                  // same wave: after this stage's reads
    }

    // rows m = 8*(r/4) + 4*h + r%4 of columns n0 + col; with a K split, out is
    // this split's slice of the [KS][M][N] workspace
    const int64_t n = n0 + col;
    if (n >= N)
        return;
    float *o = out + (int64_t)z * M * N;
#pragma unroll
    for (int r = 0; r < LIVE; r++) {
        const int64_t m = 8 * (r / 4) + 4 * h + (r % 4);
        if (m < M)
            o[m * N + n] = acc[r];
    }
}

__global__ void __launch_bounds__(256)
k_sum_splits_dec(const float *__restrict__ P, float *__restrict__ Y, int64_t MN, int ks)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= MN)
        return;
    float s = P[i];
    for (int z = 1; z < ks; z++)
        s += P[z * MN + i];
    Y[i] = s;
}

size_t lds_bytes(int rows, int kr, int nw)
{
    return (size_t)(rows + 1) * (kr * QK + XROW_PAD) + (size_t)kr * SUBS * TILE * 4 +
           (size_t)nw * TILE * WSTRIDE + 16;
}

template <int LIVE, int NW>
void launch_lnw(const uint8_t *W, const XPlanes &x, float *out, int64_t N, int ks, hipStream_t s)
{
    const int64_t nb = x.K / QK;
    const int kr_max = (int)((nb + ks - 1) / ks);
    const int rows = x.M < TILE ? (int)x.M : TILE;
    const dim3 grid((unsigned)((N + TILE * NW - 1) / (TILE * NW)), (unsigned)ks);
    hipLaunchKernelGGL((k_mmq_dec<LIVE, NW>), grid, dim3(64 * NW), lds_bytes(rows, kr_max, NW), s, W,
                       x.qp, x.dp, out, x.M, N, x.K, x.Mp);
}

template <int NW>
void launch_nw(const uint8_t *W, const XPlanes &x, float *out, int64_t N, int ks, hipStream_t s)
{
    switch (x.M) {
    case 1: launch_lnw<1, NW>(W, x, out, N, ks, s); break;
    case 2: launch_lnw<2, NW>(W, x, out, N, ks, s); break;
    case 3: launch_lnw<3, NW>(W, x, out, N, ks, s); break;
    case 4: launch_lnw<4, NW>(W, x, out, N, ks, s); break;
    default:
        if (x.M <= 8)
            launch_lnw<4, NW>(W, x, out, N, ks, s);
        else if (x.M <= 16)
            launch_lnw<8, NW>(W, x, out, N, ks, s);
        else
            launch_lnw<16, NW>(W, x, out, N, ks, s);
    }
}

}  // namespace

DecPlan mmq_dec_plan(int64_t M, int64_t N, int64_t K)
{
    DecPlan p;
    const int64_t nb = K / QK;
    const TuneOverride &t = tune_override();
    p.nw = t.dec_nw == 2 ? 2 : 4;
    const int rows = M < TILE ? (int)M : TILE;
    const int64_t nblk = (N + TILE * p.nw - 1) / (TILE * p.nw);
    int64_t ks = t.dec_ks > 0 ? t.dec_ks : (512 + nblk - 1) / nblk;   // ~two workgroups per CU
    if (ks > nb)
        ks = nb;
    // the activation slice must fit the LDS budget
    while (ks < nb && lds_bytes(rows, (int)((nb + ks - 1) / ks), p.nw) > LDS_BUDGET)
        ks++;
    p.ks = (int)ks;
    p.workspace_bytes = p.ks > 1 ? (size_t)(p.ks * M * N) * sizeof(float) : 0;
    p.ok = M <= TILE && lds_bytes(rows, (int)((nb + ks - 1) / ks), p.nw) <= 160 * 1024;
    return p;
}

hipError_t launch_mmq_dec(const void *Wv, const XPlanes &x, float *Y, int64_t N, void *workspace,
                          const DecPlan &p, hipStream_t s)
{
    const uint8_t *W = (const uint8_t *)Wv;
    if (!p.ok || (p.ks > 1 && workspace == nullptr))
        return hipErrorInvalidValue;
    float *out = p.ks > 1 ? (float *)workspace : Y;
    if (p.nw == 2)
        launch_nw<2>(W, x, out, N, p.ks, s);
    else
        launch_nw<4>(W, x, out, N, p.ks, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.ks == 1)
        return e;
    const int64_t MN = x.M * N;
    hipLaunchKernelGGL(k_sum_splits_dec, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, s,
                       (const float *)workspace, Y, MN, p.ks);
    return hipGetLastError();
}

}  // namespace iq4xs
