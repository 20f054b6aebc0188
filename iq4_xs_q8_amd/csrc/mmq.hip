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
// The weights go straight from HBM to registers (no LDS round trip): each
// byte is needed by exactly one lane.  A workgroup is KW wavefronts over the
// same 32 columns and 32*TM rows, each taking 1/KW of the sub-blocks; their
// partial sums meet in LDS and are added in wave order (deterministic).
#include "common.hpp"

namespace iq4xs {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int TILE = 32;   // MFMA tile edge (rows and columns)

// TM   : 32-row activation subtiles per wavefront (weights reused TM times)
// LIVE : result registers per subtile that can hold a real row (4: M<=8,
//        8: M<=16, 16: M<=32) -- the rest are skipped in the epilogue
// KW   : wavefronts per workgroup, splitting the sub-blocks
template <int TM, int LIVE, int KW>
__global__ void __launch_bounds__(64 * KW)
k_mmq(const uint8_t *__restrict__ W, const int8_t *__restrict__ qp, const float *__restrict__ dp,
      float *__restrict__ Y, int64_t M, int64_t N, int64_t K, int64_t Mp)
{
    static_assert(LIVE == 4 || LIVE == 8 || LIVE == 16, "live register count");
    static_assert(TM >= 1 && TM <= 4 && KW >= 1 && KW <= 8, "tile shape");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int col = lane & 31, h = lane >> 5;
    const int64_t n0 = (int64_t)blockIdx.y * TILE;
    const int64_t m0 = (int64_t)blockIdx.x * TILE * TM;
    const int64_t n_ld = (n0 + col < N) ? n0 + col : N - 1;   // clamp loads, mask stores
    const int64_t nb = K / QK, nsub = K / SB;
    const uint8_t *row = W + n_ld * nb * WBLK;

    const int64_t per = nsub / KW;                // nsub is a multiple of 8, KW divides 8
    const int64_t b_begin = wave * per, b_end = b_begin + per;

    float acc[TM][LIVE];
#pragma unroll
    for (int t = 0; t < TM; t++)
#pragma unroll
        for (int r = 0; r < LIVE; r++)
            acc[t][r] = 0.0f;

    for (int64_t b = b_begin; b < b_end; b++) {
        const uint8_t *blk = row + (b >> 3) * WBLK;
        const uint2 hdr = *reinterpret_cast<const uint2 *>(blk);
        const uint2 qs = *reinterpret_cast<const uint2 *>(blk + QS_OFF + 16 * (b & 7) + 8 * h);
        uint32_t wv[4];
        expand8(qs.x, qs.y, wv);
        const v4i bw = {(int)wv[0], (int)wv[1], (int)wv[2], (int)wv[3]};
        const float sw = sub_scale(hdr.x, hdr.y, (int)(b & 7));
#pragma unroll
        for (int t = 0; t < TM; t++) {
            const int64_t mt = m0 + TILE * t;
            if (mt >= Mp)
                break;                            // uniform: whole subtile past the padding
            const v4i ax = *reinterpret_cast<const v4i *>(qp + (mt + col) * K + 32 * b + 16 * h);
            const v16i zero = {0};
            const v16i D = __builtin_amdgcn_mfma_i32_32x32x32_i8(ax, bw, zero, 0, 0, 0);
            const float *dxp = dp + b * Mp + mt + 4 * h;
#pragma unroll
            for (int j = 0; j < LIVE / 4; j++) {
                const float4 dx = *reinterpret_cast<const float4 *>(dxp + 8 * j);
                acc[t][4 * j + 0] += (sw * dx.x) * (float)D[4 * j + 0];
                acc[t][4 * j + 1] += (sw * dx.y) * (float)D[4 * j + 1];
                acc[t][4 * j + 2] += (sw * dx.z) * (float)D[4 * j + 2];
                acc[t][4 * j + 3] += (sw * dx.w) * (float)D[4 * j + 3];
            }
        }
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
#pragma unroll
    for (int t = 0; t < TM; t++)
#pragma unroll
        for (int r = 0; r < LIVE; r++) {
            const int64_t m = m0 + TILE * t + 8 * (r / 4) + 4 * h + (r % 4);
            if (m < M)
                Y[m * N + n] = acc[t][r];
        }
}

template <int TM, int LIVE>
hipError_t launch_tm(const uint8_t *W, const XPlanes &x, float *Y, int64_t N, int kw,
                     hipStream_t s)
{
    const dim3 grid((unsigned)((x.Mp + TILE * TM - 1) / (TILE * TM)), (unsigned)((N + TILE - 1) / TILE));
    switch (kw) {
    case 1: hipLaunchKernelGGL((k_mmq<TM, LIVE, 1>), grid, dim3(64), 0, s, W, x.qp, x.dp, Y, x.M, N, x.K, x.Mp); break;
    case 2: hipLaunchKernelGGL((k_mmq<TM, LIVE, 2>), grid, dim3(128), 0, s, W, x.qp, x.dp, Y, x.M, N, x.K, x.Mp); break;
    case 4: hipLaunchKernelGGL((k_mmq<TM, LIVE, 4>), grid, dim3(256), 0, s, W, x.qp, x.dp, Y, x.M, N, x.K, x.Mp); break;
    case 8: hipLaunchKernelGGL((k_mmq<TM, LIVE, 8>), grid, dim3(512), 0, s, W, x.qp, x.dp, Y, x.M, N, x.K, x.Mp); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mmq(const void *Wv, const XPlanes &x, float *Y, int64_t N, hipStream_t s)
{
    const uint8_t *W = (const uint8_t *)Wv;
    const int64_t ntile = (N + TILE - 1) / TILE;
    int tm = x.M <= 32 ? 1 : (x.M <= 64 ? 2 : 4);
    const int64_t wg = ntile * ((x.Mp + TILE * tm - 1) / (TILE * tm));
    // enough wavefronts to cover the chip several times; nsub is a multiple of 8
    int kw = 1;
    while (kw < 8 && wg * kw < 2048)
        kw *= 2;
    if (x.M <= 8)
        return launch_tm<1, 4>(W, x, Y, N, kw, s);
    if (x.M <= 16)
        return launch_tm<1, 8>(W, x, Y, N, kw, s);
    if (x.M <= 32)
        return launch_tm<1, 16>(W, x, Y, N, kw, s);
    if (x.M <= 64)
        return launch_tm<2, 16>(W, x, Y, N, kw, s);
    return launch_tm<4, 16>(W, x, Y, N, kw, s);
}

}  // namespace iq4xs
