// gemv.hip -- IQ4_XS x Q8_1 for a handful of activation rows (M <= 4).
//
// Prior art: the mmvq kernel of the "V100TPS engine log"
// (agent-report.daedalus.work/V100TPS/engine.html, mmvq vs dequant+GEMM table),
// a dp4a vector dot whose cost grows linearly with M.  Here a wavefront owns
// R output rows and streams their K/256 super-blocks once for all M rows.
//
// Work unit = half a sub-block: 8 index bytes = 16 weights (elements
// 8h..8h+7 and 16+8h..16+8h+7 of sub-block b).  Lane l takes units
// l, l+64, ... in chunks of U; for a chunk it first issues every load (the
// R rows' block headers and index bytes, the matching 16 activation bytes of
// each of the M rows and their block scales), then for each unit and row
//   1. expands the nibbles to int8 kvalues with byte permutes,
//   2. forms the exact integer dot with the activations (v_dot4_i32_i8 x4),
//   3. adds (d*(ls-32) * d_x) * D to a per-(row, m) fp32 accumulator.
// The activations of a unit are loaded once and reused for all R rows.  At
// the end the wave sums its 64 partial accumulators in a fixed butterfly
// order (deterministic, no atomics) and lane 0 writes Y.
#include "common.hpp"

namespace iq4xs {
namespace {

constexpr int GEMV_WAVES = 4;   // wavefronts per workgroup

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

// F: the weight format (its 256-weight unit is 136 or 144 bytes; the scale
// and index bytes of sub-block b are read through unit_scale_raw / unit_qs).
template <int M, int R, int U, int F>
__global__ void __launch_bounds__(64 * GEMV_WAVES)
k_gemv(const uint8_t *__restrict__ W, const int8_t *__restrict__ qp, const float *__restrict__ dp,
       float *__restrict__ Y, int64_t N, int64_t K, int64_t Mp)
{
    constexpr int UB = sblk_bytes(F);
    static_assert(M >= 1 && M <= GEMV_MAX_M, "GEMV handles 1..4 rows");
    const int lane = threadIdx.x & 63;
    const int64_t n0 = ((int64_t)blockIdx.x * GEMV_WAVES + (threadIdx.x >> 6)) * R;
    if (n0 >= N)
        return;                                    // uniform per wave
    const int64_t nb = K / QK;
    const int units = (int)(K / 16);
    const uint8_t *row[R];
#pragma unroll
    for (int r = 0; r < R; r++)
        row[r] = W + (n0 + r < N ? n0 + r : N - 1) * nb * UB;     // clamp loads, mask stores

    float acc[R][M];
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int m = 0; m < M; m++)
            acc[r][m] = 0.0f;

    for (int base = 0; base < units; base += 64 * U) {
        // all loads of the chunk first, with no branch around them (a lane past
        // the last unit re-reads the last unit and discards it), so they are
        // all in flight together
        uint2 hdr[U][R], qs[U][R];
        int4 xv[U][M];
        float4 dx[U];
#pragma unroll
        for (int i = 0; i < U; i++) {
            const int u0 = base + lane + 64 * i;
            const int u = u0 < units ? u0 : units - 1;
            const int b = u >> 1, h = u & 1;
            const uint32_t off_blk = (uint32_t)(b >> 3) * UB;
#pragma unroll
            for (int r = 0; r < R; r++) {
                const char *unit = reinterpret_cast<const char *>(row[r] + off_blk);
                hdr[i][r] = unit_scale_raw<F>(unit, b & 7);
                qs[i][r] = unit_qs<F>(unit, b & 7, h);
            }
            dx[i] = *reinterpret_cast<const float4 *>(dp + (uint32_t)b * (uint32_t)Mp);
#pragma unroll
            for (int m = 0; m < M; m++)
                xv[i][m] = *reinterpret_cast<const int4 *>(qp + ((uint32_t)(b * Mp + m) * SB + 16 * h));
        }
#pragma unroll
        for (int i = 0; i < U; i++) {
            const int u = base + lane + 64 * i;
            if (u < units) {
                const int b = u >> 1;
                const float dxm[4] = {dx[i].x, dx[i].y, dx[i].z, dx[i].w};
#pragma unroll
                for (int r = 0; r < R; r++) {
                    uint32_t wv[4];
                    expand8<F>(qs[i][r].x, qs[i][r].y, wv);
                    const float sw = unit_scale_dec<F>(hdr[i][r], b & 7, true);
#pragma unroll
                    for (int m = 0; m < M; m++) {
                        int D = __builtin_amdgcn_sdot4((int)wv[0], xv[i][m].x, 0, false);
                        D = __builtin_amdgcn_sdot4((int)wv[1], xv[i][m].y, D, false);
                        D = __builtin_amdgcn_sdot4((int)wv[2], xv[i][m].z, D, false);
                        D = __builtin_amdgcn_sdot4((int)wv[3], xv[i][m].w, D, false);
                        acc[r][m] += (sw * dxm[m]) * (float)D;
                    }
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; r++)
#pragma unroll
        for (int m = 0; m < M; m++) {
            const float s = wave_sum(acc[r][m]);
            if (lane == 0 && n0 + r < N)
                Y[m * N + n0 + r] = s;
        }
}

template <int M, int R, int U, int F>
void launch_mru(const uint8_t *w, const XPlanes &x, float *Y, int64_t N, hipStream_t s)
{
    const int64_t rows_per_block = (int64_t)GEMV_WAVES * R;
    const dim3 grid((unsigned)((N + rows_per_block - 1) / rows_per_block)), block(64 * GEMV_WAVES);
    hipLaunchKernelGGL((k_gemv<M, R, U, F>), grid, block, 0, s, w, x.qp, x.dp, Y, N, x.K, x.Mp);
}

// Chunk size: the units each lane owns (K/16/64), split into equal chunks
// of at most UMAX so every load of a chunk is in flight at once.
template <int M, int R, int UMAX, int F>
void launch_m(const uint8_t *w, const XPlanes &x, float *Y, int64_t N, hipStream_t s)
{
    const int64_t per_lane = (x.K / 16 + 63) / 64;
    const int64_t chunks = (per_lane + UMAX - 1) / UMAX;
    const int u = (int)((per_lane + chunks - 1) / chunks);
    switch (u) {
    case 1: launch_mru<M, R, 1, F>(w, x, Y, N, s); break;
    case 2: launch_mru<M, R, 2, F>(w, x, Y, N, s); break;
    case 3: launch_mru<M, R, 3, F>(w, x, Y, N, s); break;
    case 4: launch_mru<M, R, 4, F>(w, x, Y, N, s); break;
    case 5: if constexpr (UMAX >= 5) launch_mru<M, R, 5, F>(w, x, Y, N, s); break;
    default: if constexpr (UMAX >= 6) launch_mru<M, R, 6, F>(w, x, Y, N, s); break;
    }
}

template <int F>
hipError_t launch_gemv_fmt(const uint8_t *w, const XPlanes &x, float *Y, int64_t N, hipStream_t s)
{
    switch (x.M) {
    // two rows per wavefront (measured on MI355X, M=1, 10240 x 5120: 11.6 us
    // against 12.8 with four rows and 13.1 with one)
    case 1: launch_m<1, 2, 6, F>(w, x, Y, N, s); break;
    case 2: launch_m<2, 2, 6, F>(w, x, Y, N, s); break;
    case 3: launch_m<3, 2, 4, F>(w, x, Y, N, s); break;
    case 4: launch_m<4, 2, 4, F>(w, x, Y, N, s); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv(const void *W, const XPlanes &x, float *Y, int64_t N, hipStream_t s, int fmt)
{
    const uint8_t *w = (const uint8_t *)W;
    switch (fmt) {
    case FMT_IQ4_XS: return launch_gemv_fmt<FMT_IQ4_XS>(w, x, Y, N, s);
    case FMT_IQ4_NL: return launch_gemv_fmt<FMT_IQ4_NL>(w, x, Y, N, s);
    case FMT_Q4_0: return launch_gemv_fmt<FMT_Q4_0>(w, x, Y, N, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace iq4xs
