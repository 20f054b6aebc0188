// gemv.hip -- IQ4_XS x Q8_1 for a handful of activation rows (M <= 4).
//
// Prior art: the mmvq kernel of the "V100TPS engine log"
// (agent-report.daedalus.work/V100TPS/engine.html, mmvq vs dequant+GEMM table),
// a dp4a vector dot whose cost grows linearly with M.  Here one wavefront owns
// one output row n and streams its K/256 super-blocks once for all M rows.
//
// Work unit = half a sub-block: 8 index bytes = 16 weights (elements
// 8h..8h+7 and 16+8h..16+8h+7 of sub-block b).  Lane u of the wave takes units
// u, u+64, ...; per unit it
//   1. loads the 8 index bytes and the 8-byte block header (d, scales),
//   2. expands the nibbles to int8 kvalues with byte permutes,
//   3. forms the exact integer dot with the matching 16 activation bytes
//      (v_dot4_i32_i8 x4) for each row m,
//   4. adds (d*(ls-32) * d_x) * D to a per-row fp32 accumulator;
// then the wave sums its 64 partial accumulators in a fixed butterfly order
// (deterministic, no atomics) and lane 0 writes Y[m, n].
#include "common.hpp"

namespace iq4xs {
namespace {

constexpr int GEMV_WAVES = 4;   // rows per workgroup

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

template <int M>
__global__ void __launch_bounds__(64 * GEMV_WAVES)
k_gemv(const uint8_t *__restrict__ W, const int8_t *__restrict__ qp, const float *__restrict__ dp,
       float *__restrict__ Y, int64_t N, int64_t K, int64_t Mp)
{
    static_assert(M >= 1 && M <= GEMV_MAX_M, "GEMV handles 1..4 rows");
    const int lane = threadIdx.x & 63;
    const int64_t n = (int64_t)blockIdx.x * GEMV_WAVES + (threadIdx.x >> 6);
    if (n >= N)
        return;                                    // uniform per wave
    const int64_t nb = K / QK;
    const uint8_t *row = W + n * nb * WBLK;
    const int units = (int)(K / 16);

    float acc[M];
#pragma unroll
    for (int m = 0; m < M; m++)
        acc[m] = 0.0f;

    for (int u = lane; u < units; u += 64) {
        const int b = u >> 1, h = u & 1;           // sub-block, half
        const uint8_t *blk = row + (int64_t)(b >> 3) * WBLK;
        const uint2 hdr = *reinterpret_cast<const uint2 *>(blk);
        const uint2 qs = *reinterpret_cast<const uint2 *>(blk + QS_OFF + 16 * (b & 7) + 8 * h);
        uint32_t wv[4];
        expand8(qs.x, qs.y, wv);
        const float sw = sub_scale(hdr.x, hdr.y, b & 7);
        const float4 dx4 = *reinterpret_cast<const float4 *>(dp + (int64_t)b * Mp);
        const float dx[4] = {dx4.x, dx4.y, dx4.z, dx4.w};
#pragma unroll
        for (int m = 0; m < M; m++) {
            const int4 xv = *reinterpret_cast<const int4 *>(qp + m * K + 32 * (int64_t)b + 16 * h);
            int D = __builtin_amdgcn_sdot4((int)wv[0], xv.x, 0, false);
            D = __builtin_amdgcn_sdot4((int)wv[1], xv.y, D, false);
            D = __builtin_amdgcn_sdot4((int)wv[2], xv.z, D, false);
            D = __builtin_amdgcn_sdot4((int)wv[3], xv.w, D, false);
            acc[m] += (sw * dx[m]) * (float)D;
        }
    }
#pragma unroll
    for (int m = 0; m < M; m++) {
        const float s = wave_sum(acc[m]);
        if (lane == 0)
            Y[m * N + n] = s;
    }
}

}  // namespace

hipError_t launch_gemv(const void *W, const XPlanes &x, float *Y, int64_t N, hipStream_t s)
{
    const dim3 grid((unsigned)((N + GEMV_WAVES - 1) / GEMV_WAVES)), block(64 * GEMV_WAVES);
    const uint8_t *w = (const uint8_t *)W;
    switch (x.M) {
    case 1: hipLaunchKernelGGL(k_gemv<1>, grid, block, 0, s, w, x.qp, x.dp, Y, N, x.K, x.Mp); break;
    case 2: hipLaunchKernelGGL(k_gemv<2>, grid, block, 0, s, w, x.qp, x.dp, Y, N, x.K, x.Mp); break;
    case 3: hipLaunchKernelGGL(k_gemv<3>, grid, block, 0, s, w, x.qp, x.dp, Y, N, x.K, x.Mp); break;
    case 4: hipLaunchKernelGGL(k_gemv<4>, grid, block, 0, s, w, x.qp, x.dp, Y, N, x.K, x.Mp); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace iq4xs
