// mmq.hip -- IQ4_XS x Q8_1 tile kernel on the int8 matrix cores of gfx950.
//
// Prior art: the batched IQ4_XS MMQ kernel of the "V100TPS engine log"
// (agent-report.daedalus.work/V100TPS/engine.html, section on the batched
// IQ4_XS kernel and the new-kernel vs dispatcher table): one weight read is
// shared by all M activation rows; the 32-element sub-block keeps the Q4_0
// tile geometry with two changes, the per-sub-block scale d*(ls-32) and the
// kvalues_iq4nl lookup in place of q-8.
//
// gfx950 design.  v_mfma_i32_32x32x32_i8 contracts exactly K = 32, one
// IQ4_XS sub-block, so every MFMA result is the exact integer dot
// D[m,n] = sum_t kv[n,32b+t] * q[m,32b+t] of one sub-block, which is then
// scaled in fp32 by d_w*(ls-32) (per lane: the lane's column n) times d_x
// (per register: the register's row m) and accumulated.
//   A operand = activations: lane l supplies row m0 + l%32, chunk h = l/32
//     (16 bytes of the chunk-ordered activation plane);
//   B operand = weights: lane l supplies row n0 + l%32, chunk h: the 8 index
//     bytes qs[16b+8h .. 16b+8h+7] expanded in registers to 16 int8 kvalues
//     in the same element order (low nibbles then high nibbles).
// The two operands use the same per-lane element order, so the hardware's
// pairing of k positions inside the instruction is irrelevant.
// Result layout (16 int32 per lane): column n = l%32, register r holds row
// 8*(r/4) + 4*(l/32) + r%4.
//
// The weights go straight from HBM to registers (each byte is needed by one
// lane only).  A wavefront walks whole super-blocks: the next super-block's
// header and index bytes are loaded before the current one is computed, and
// the activation operands of a group of G sub-blocks are loaded before their
// MFMAs.  Work split: KW wavefronts of a workgroup share 32 columns x 32*TM
// rows and split the workgroup's super-blocks; their partial sums meet in LDS
// and are added in wave order.  For long K and small N the super-blocks are
// further split over KS workgroups (grid z); each writes its partial tile to
// a workspace and a second kernel adds the KS partials in order.  Everything
// is deterministic: no atomics, fixed summation order.
#include "common.hpp"

namespace iq4xs {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int TILE = 32;   // MFMA tile edge (rows and columns)
// Buffer-resource flags word for raw (stride 0) buffers on the gfx9 family.
constexpr int BUFFER_FLAGS = 0x00020000;

// TM   : 32-row activation subtiles per wavefront (weights reused TM times)
// LIVE : result registers per subtile that can hold a real row (4: M<=8,
//        8: M<=16, 16: M<=32); the rest are skipped in the epilogue
// KW   : wavefronts per workgroup splitting the super-blocks
// G    : sub-blocks whose activation operands are loaded together (1,2,4,8)
template <int TM, int LIVE, int KW, int G>
__global__ void __launch_bounds__(64 * KW)
k_mmq(const uint8_t *__restrict__ W, const int8_t *__restrict__ qp, const float *__restrict__ dp,
      float *__restrict__ Y, int64_t M, int64_t N, int64_t K, int64_t Mp)
{
    static_assert(LIVE == 4 || LIVE == 8 || LIVE == 16, "live register count");
    static_assert(TM >= 1 && TM <= 4 && KW >= 1 && KW <= 8, "tile shape");
    static_assert(G == 1 || G == 2 || G == 4 || G == 8, "activation group");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 31, h = lane >> 5;
    const int64_t n0 = (int64_t)blockIdx.y * TILE;
    const int64_t m0 = (int64_t)blockIdx.x * TILE * TM;
    const int64_t nb = K / QK;
    const uint32_t row_bytes = (uint32_t)(nb * WBLK);
    const int ks = gridDim.z;                     // workgroups splitting K
    const int64_t jw0 = nb * blockIdx.z / ks, jw1 = nb * (blockIdx.z + 1) / ks;
    const int64_t j_begin = jw0 + (jw1 - jw0) * wave / KW;
    const int64_t j_end = jw0 + (jw1 - jw0) * (wave + 1) / KW;
    int tm_live = (int)((M - m0 + TILE - 1) / TILE);   // 32-row subtiles holding real rows
    if (tm_live > TM)
        tm_live = TM;

    // Buffer descriptors: rows past N (weights) and everything past the
    // activation planes lie beyond num_records, so their loads return zeros
    // without a memory access.  Activation rows M..m0+32*TM-1 of a block read
    // pad rows or the next block's rows: they only feed result rows >= M,
    // which are not stored.
    const int64_t n_rows = (N - n0) < TILE ? (N - n0) : TILE;
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(W + n0 * (int64_t)row_bytes), (short)0, (int)(n_rows * row_bytes), BUFFER_FLAGS);
    const __amdgpu_buffer_rsrc_t xr =
        __builtin_amdgcn_make_buffer_rsrc((void *)qp, (short)0, (int)(Mp * K), BUFFER_FLAGS);
    const __amdgpu_buffer_rsrc_t dr =
        __builtin_amdgcn_make_buffer_rsrc((void *)dp, (short)0, (int)(Mp * (K / SB) * 4), BUFFER_FLAGS);
    const uint32_t w_lane = (uint32_t)col * row_bytes;

    float acc[TM][LIVE];
#pragma unroll
    for (int t = 0; t < TM; t++)
#pragma unroll
        for (int r = 0; r < LIVE; r++)
            acc[t][r] = 0.0f;

    uint2 hdr_c = make_uint2(0, 0), qs_c[SUBS];
    uint2 hdr_n = make_uint2(0, 0), qs_n[SUBS];
#pragma unroll
    for (int s = 0; s < SUBS; s++)
        qs_c[s] = qs_n[s] = make_uint2(0, 0);
    auto load_w = [&](int64_t j, uint2 &hdr, uint2 *qs) {
        const uint32_t o = w_lane + (uint32_t)j * WBLK;
        hdr = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(wr, o, 0, 0));
#pragma unroll
        for (int s = 0; s < SUBS; s++)
            qs[s] = __builtin_bit_cast(
                uint2, __builtin_amdgcn_raw_buffer_load_b64(wr, o + QS_OFF + 16 * s + 8 * h, 0, 0));
    };
    if (j_begin < j_end)
        load_w(j_begin, hdr_c, qs_c);

    for (int64_t j = j_begin; j < j_end; j++) {
#pragma unroll
        for (int g = 0; g < SUBS; g += G) {
            // activation operands of sub-blocks g..g+G-1 of super-block j ...
            v4i ax[TM][G];
            float4 dx[TM][G][LIVE / 4];
#pragma unroll
            for (int t = 0; t < TM; t++) {
                if (t < tm_live) {
                    const int64_t mt = m0 + TILE * t;
#pragma unroll
                    for (int s = 0; s < G; s++) {
                        const int64_t sb = SUBS * j + g + s;
                        ax[t][s] = __builtin_amdgcn_raw_buffer_load_b128(
                            xr, (uint32_t)((sb * Mp + mt + col) * SB + 16 * h), 0, 0);
#pragma unroll
                        for (int q = 0; q < LIVE / 4; q++)
                            dx[t][s][q] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                dr, (uint32_t)((sb * Mp + mt + 4 * h + 8 * q) * 4), 0, 0));
                    }
                }
            }
            // ... then, once the last group's activations are in flight, the
            // next super-block's weights: loads retire in order, so waiting for
            // the activations above never waits for this prefetch
            if (g + G == SUBS && j + 1 < j_end)
                load_w(j + 1, hdr_n, qs_n);
#pragma unroll
            for (int s = 0; s < G; s++) {
                uint32_t wv[4];
                expand8(qs_c[g + s].x, qs_c[g + s].y, wv);
                const v4i bw = {(int)wv[0], (int)wv[1], (int)wv[2], (int)wv[3]};
                const float sw = sub_scale(hdr_c.x, hdr_c.y, g + s);
#pragma unroll
                for (int t = 0; t < TM; t++) {
                    if (t < tm_live) {
                        const v16i zero = {0};
                        const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(ax[t][s], bw, zero, 0, 0, 0);
#pragma unroll
                        for (int q = 0; q < LIVE / 4; q++) {
                            acc[t][4 * q + 0] += (sw * dx[t][s][q].x) * (float)D[4 * q + 0];
                            acc[t][4 * q + 1] += (sw * dx[t][s][q].y) * (float)D[4 * q + 1];
                            acc[t][4 * q + 2] += (sw * dx[t][s][q].z) * (float)D[4 * q + 2];
                            acc[t][4 * q + 3] += (sw * dx[t][s][q].w) * (float)D[4 * q + 3];
                        }
                    }
                }
            }
        }
        hdr_c = hdr_n;
#pragma unroll
        for (int s = 0; s < SUBS; s++)
            qs_c[s] = qs_n[s];
    }

    if constexpr (KW > 1) {
        __shared__ float red[KW - 1][TM * LIVE][64];
        if (wave > 0) {
#pragma unroll
            for (int t = 0; t < TM; t++)
#pragma unroll
                for (int r = 0; r < LIVE; r++)
                    red[wave - 1][t * LIVE + r][lane] = acc[t][r];
        }
        __syncthreads();
        if (wave != 0)
            return;
#pragma unroll
        for (int w = 0; w < KW - 1; w++)
#pragma unroll
            for (int t = 0; t < TM; t++)
#pragma unroll
                for (int r = 0; r < LIVE; r++)
                    acc[t][r] += red[w][t * LIVE + r][lane];
    }

    const int64_t n = n0 + col;
    if (n >= N)
        return;
    // with a K split, Y points at this split's slice of the [KS][M][N] workspace
    float *out = Y + (int64_t)blockIdx.z * M * N;
#pragma unroll
    for (int t = 0; t < TM; t++)
#pragma unroll
        for (int r = 0; r < LIVE; r++) {
            const int64_t m = m0 + TILE * t + 8 * (r / 4) + 4 * h + (r % 4);
            if (m < M)
                out[m * N + n] = acc[t][r];
        }
}

// Y[m,n] = sum_{z<KS} P[z][m][n], in order of z.
__global__ void __launch_bounds__(256)
k_sum_splits(const float *__restrict__ P, float *__restrict__ Y, int64_t MN, int ks)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= MN)
        return;
    float s = P[i];
    for (int z = 1; z < ks; z++)
        s += P[z * MN + i];
    Y[i] = s;
}

template <int TM, int LIVE, int G>
void launch_tm(const uint8_t *W, const XPlanes &x, float *out, int64_t N, int kw, int ks, hipStream_t s)
{
    const dim3 grid((unsigned)((x.Mp + TILE * TM - 1) / (TILE * TM)), (unsigned)((N + TILE - 1) / TILE),
                    (unsigned)ks);
    switch (kw) {
    case 1: hipLaunchKernelGGL((k_mmq<TM, LIVE, 1, G>), grid, dim3(64), 0, s, W, x.qp, x.dp, out, x.M, N, x.K, x.Mp); break;
    case 2: hipLaunchKernelGGL((k_mmq<TM, LIVE, 2, G>), grid, dim3(128), 0, s, W, x.qp, x.dp, out, x.M, N, x.K, x.Mp); break;
    case 4: hipLaunchKernelGGL((k_mmq<TM, LIVE, 4, G>), grid, dim3(256), 0, s, W, x.qp, x.dp, out, x.M, N, x.K, x.Mp); break;
    default:
        if constexpr (TM == 1)
            hipLaunchKernelGGL((k_mmq<TM, LIVE, 8, G>), grid, dim3(512), 0, s, W, x.qp, x.dp, out, x.M, N, x.K, x.Mp);
        break;
    }
}

}  // namespace

MmqPlan mmq_plan(int64_t M, int64_t N, int64_t K, int fmt)
{
    MmqPlan p;
    if (M <= TILE && tune_override().mmv != 0) {
        p.vp = mmv_plan(M, N, K, device_cus(), fmt);
        if (p.vp.ok) {
            p.mmv = true;
            p.zero_y = p.vp.zero_y;
            return p;
        }
    }
    if (M > TILE && tune_override().tile != 0) {
        p.tp = mmqt_plan(M, N, K, device_cus(), fmt);
        if (p.tp.ok) {
            p.tile = true;
            p.zero_y = p.tp.zero_y;
            p.workspace_bytes = p.tp.workspace_bytes;
            return p;
        }
    }
    if (fmt != FMT_IQ4_XS) {
        p.ok = false;
        return p;
    }
    const int64_t Mp = round_up(M, MPAD);
    const int tm = M <= 32 ? 1 : (M <= 64 ? 2 : 4);
    const int64_t nb = K / QK;
    const int64_t tiles = ((N + TILE - 1) / TILE) * ((Mp + TILE * tm - 1) / (TILE * tm));
    // enough workgroups to cover the 256 CUs twice, then enough wavefronts
    // per workgroup for latency hiding; every wave keeps >= 2 super-blocks
    int ks = 1;
    while (ks < 8 && tiles * ks < 512 && nb / (ks * 2) >= 4)
        ks *= 2;
    // (8 wavefronts per workgroup only for single-subtile tiles: a 512-thread
    // workgroup caps a lane at 256 registers, too few for TM >= 2)
    const int kw_max = tm == 1 ? 8 : 4;
    int kw = 1;
    while (kw < kw_max && tiles * ks * kw < 4096 && nb / (ks * kw * 2) >= 2)
        kw *= 2;
    p.tm = tm;
    p.kw = kw;
    p.ks = ks;
    p.workspace_bytes = ks > 1 ? (size_t)(ks * M * N) * sizeof(float) : 0;
    return p;
}

hipError_t launch_mmq(const void *Wv, const XPlanes &x, float *Y, int64_t N, void *workspace,
                      bool y_zeroed, hipStream_t s, int fmt)
{
    const uint8_t *W = (const uint8_t *)Wv;
    const MmqPlan p = mmq_plan(x.M, N, x.K, fmt);
    if (!p.ok)
        return hipErrorInvalidValue;
    if (p.mmv) {
        if (p.vp.zero_y && !y_zeroed) {
            const hipError_t e = launch_zero(Y, x.M * N, s);
            if (e != hipSuccess)
                return e;
        }
        return launch_mmv(Wv, x, Y, N, p.vp, s);
    }
    if (p.tile) {
        if (p.tp.workspace_bytes && workspace == nullptr)
            return hipErrorInvalidValue;
        if (p.tp.zero_y && !y_zeroed) {
            const hipError_t e = launch_zero_tiles(mmqt_zero_tiles(p.tp, x.M, N, x.K, Y), s);
            if (e != hipSuccess)
                return e;
        }
        return launch_mmqt(Wv, x, Y, N, p.tp, workspace, s);
    }
    if (p.ks > 1 && workspace == nullptr)
        return hipErrorInvalidValue;
    float *out = p.ks > 1 ? (float *)workspace : Y;
    if (x.M <= 8)
        launch_tm<1, 4, 8>(W, x, out, N, p.kw, p.ks, s);
    else if (x.M <= 16)
        launch_tm<1, 8, 8>(W, x, out, N, p.kw, p.ks, s);
    else if (x.M <= 32)
        launch_tm<1, 16, 4>(W, x, out, N, p.kw, p.ks, s);
    else if (x.M <= 64)
        launch_tm<2, 16, 2>(W, x, out, N, p.kw, p.ks, s);
    else
        launch_tm<4, 16, 1>(W, x, out, N, p.kw, p.ks, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.ks == 1)
        return e;
    const int64_t MN = x.M * N;
    hipLaunchKernelGGL(k_sum_splits, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, s,
                       (const float *)workspace, Y, MN, p.ks);
    return hipGetLastError();
}

}  // namespace iq4xs
