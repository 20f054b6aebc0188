// quantize.hip -- fp32 activations -> Q8_1 ("V100TPS engine log",
// agent-report.daedalus.work/V100TPS/engine.html, M=64 kernel-launch table:
// quantize_q8_1 runs before every integer matmul).
//
// Per 32-element block: amax = max|x|; d = amax/127 (IEEE fp32 division);
// q = round-half-away-from-zero(x/d) (IEEE fp32 division, q = 0 when d == 0),
// clamped to [-127, 127]; stored d16 = fp16(d) (nearest even); stored
// s16 = fp16(d16 * sum q) -- d16 * sum q is exact in fp32 (11 + 12 bits), so
// it is rounded once.  The pages give only "Q8_1"; the rounding rule is the
// reading stated in the ABI header.
//
// Layout: eight consecutive lanes own one block, four elements each, so
// the block reductions are three butterfly steps inside an 8-lane group.
#include "common.hpp"

#include <algorithm>

namespace iq4xs {
namespace {

__device__ __forceinline__ uint32_t pack_q(int q0, int q1, int q2, int q3)
{
    return (uint32_t)(uint8_t)q0 | ((uint32_t)(uint8_t)q1 << 8) | ((uint32_t)(uint8_t)q2 << 16) |
           ((uint32_t)(uint8_t)q3 << 24);
}

// Position (in bytes) of the 4-byte group holding elements 4t..4t+3 of a
// sub-block inside the chunk-ordered plane layout: element e of 8-group
// g = e/8 moves by +0, +8, -8, +0 for g = 0..3.
__device__ __forceinline__ int plane_pos(int t)
{
    const int g = t >> 1;
    const int delta = (g == 1) ? 8 : (g == 2) ? -8 : 0;
    return 4 * t + delta;
}

// yz[0..nz) = 0 over a grid of `stride` threads (yz 16-byte aligned).
__device__ __forceinline__ void zero_range(float *yz, int64_t nz, int64_t tid, int64_t stride)
{
    if (yz == nullptr)
        return;
    const int64_t n4 = nz >> 2;
    for (int64_t i = tid; i < n4; i += stride)
        reinterpret_cast<float4 *>(yz)[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (tid < (nz & 3))
        yz[4 * n4 + tid] = 0.0f;
}

// The listed tiles of zt.y = 0 over a grid of `stride` threads (elements
// past M or N skipped; fewer than 2^31 elements in all).  Four consecutive
// columns of a tile row per step: one 16-byte store where the row is 16-byte
// aligned (N a multiple of 4) and the four columns lie inside N, else up to
// four single stores.
__device__ __forceinline__ void zero_tiles(const ZeroTiles &zt, int64_t tid, int64_t stride)
{
    if (zt.count == 0)
        return;
    const int per4 = zt.bm * zt.bn / 4;                   // (bn a multiple of 4)
    const bool vec = (zt.N & 3) == 0;
    for (int e = (int)tid; e < zt.count * per4; e += (int)stride) {
        const int i = e / per4, w = 4 * (e - i * per4);
        const int t = zt.t[i], row = w / zt.bn, col = w - row * zt.bn;
        const int64_t m = (int64_t)(t / zt.wblocks) * zt.bm + row;
        const int64_t n = (int64_t)(t % zt.wblocks) * zt.bn + col;
        if (m >= zt.M)
            continue;
        float *y = zt.y + m * zt.N + n;
        if (vec && n + 4 <= zt.N) {
            *reinterpret_cast<float4 *>(y) = make_float4(0.f, 0.f, 0.f, 0.f);
        } else {
#pragma unroll
            for (int c = 0; c < 4; c++)
                if (n + c < zt.N)
                    y[c] = 0.0f;
        }
    }
}

__device__ __forceinline__ void zero_list(const ZeroList &zl, int64_t tid, int64_t stride)
{
#pragma unroll
    for (int i = 0; i < MAXGRP; i++)
        if (i < zl.count)
            zero_range(zl.p[i], zl.n[i], tid, stride);
    zero_tiles(zl.tiles, tid, stride);
}

__global__ void __launch_bounds__(256) k_zero(float *__restrict__ y, int64_t n)
{
    zero_range(y, n, (int64_t)blockIdx.x * blockDim.x + threadIdx.x, (int64_t)gridDim.x * blockDim.x);
}

__global__ void __launch_bounds__(256) k_zero_tiles(ZeroTiles zt)
{
    zero_tiles(zt, (int64_t)blockIdx.x * blockDim.x + threadIdx.x, (int64_t)gridDim.x * blockDim.x);
}

// Elements 4t..4t+3 of block b of row m into the compensated bf16 planes
// (rows past M carry q = 0, so zeros).  d*q is exact in fp32.
__device__ __forceinline__ void write_split(const XSplit &xs, int64_t m, int64_t b, int t, float d, int q0,
                                            int q1, int q2, int q3)
{
    if (xs.p == nullptr || m >= xs.Ms)
        return;
    uint32_t h01, l01, h23, l23;
    bf16x2_split(d * (float)q0, d * (float)q1, h01, l01);
    bf16x2_split(d * (float)q2, d * (float)q3, h23, l23);
    uint16_t *o = xs.p + (b * xs.Ms + m) * 64 + 4 * t;
    *reinterpret_cast<uint2 *>(o) = make_uint2(h01, h23);
    *reinterpret_cast<uint2 *>(o + 32) = make_uint2(l01, l23);
}

__device__ __forceinline__ int quant1(float x, float d)
{
    if (d == 0.0f)
        return 0;
    int q = (int)roundf(x / d);   // correctly rounded fp32 division (no fast-math)
    return q > 127 ? 127 : (q < -127 ? -127 : q);
}

// Grid: one thread per 4 activations over Mrows x K (Mrows = M, or the
// padded row count of the compensated bf16 planes when those are written:
// their rows past M get zeros).  The plane rows M..Mp-1 are never written:
// the matmul kernels either skip them or read them through buffer
// descriptors that stop at row M.
__global__ void __launch_bounds__(256)
k_quantize(const float *__restrict__ X, uint8_t *__restrict__ Xq, int8_t *__restrict__ qp,
           float *__restrict__ dp, ZeroList zl, XSplit xs,
           int64_t M, int64_t Mrows, int64_t Mp, int64_t K)
{
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    zero_list(zl, tid, (int64_t)gridDim.x * blockDim.x);
    const int64_t nblk_row = K / SB;
    const int64_t blk = tid >> 3;                 // global Q8_1 block index
    const int t = (int)(tid & 7);                 // lane within the block
    if (blk >= Mrows * nblk_row)
        return;                                   // whole 8-lane groups exit together
    const int64_t m = blk / nblk_row, b = blk - m * nblk_row;

    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (m < M)
        v = *reinterpret_cast<const float4 *>(X + m * K + b * SB + 4 * t);

    float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    amax = fmaxf(amax, __shfl_xor(amax, 1, 8));
    amax = fmaxf(amax, __shfl_xor(amax, 2, 8));
    amax = fmaxf(amax, __shfl_xor(amax, 4, 8));
    const float d = amax / 127.0f;                // correctly rounded fp32 division

    const int q0 = quant1(v.x, d), q1 = quant1(v.y, d), q2 = quant1(v.z, d), q3 = quant1(v.w, d);
    int sum = q0 + q1 + q2 + q3;
    sum += __shfl_xor(sum, 1, 8);
    sum += __shfl_xor(sum, 2, 8);
    sum += __shfl_xor(sum, 4, 8);

    const _Float16 d16 = (_Float16)d;             // v_cvt_f16_f32, round to nearest even
    const float dst = (float)d16;
    const uint32_t qword = pack_q(q0, q1, q2, q3);

    if (Xq != nullptr && m < M) {
        uint8_t *o = Xq + blk * XBLK;
        const _Float16 s16 = (_Float16)(dst * (float)sum);   // exact product, one rounding
        *reinterpret_cast<uint32_t *>(o + 4 + 4 * t) = qword;
        if (t == 0)
            *reinterpret_cast<uint32_t *>(o) = (uint32_t)__builtin_bit_cast(uint16_t, d16) |
                                               ((uint32_t)__builtin_bit_cast(uint16_t, s16) << 16);
    }
    if (qp != nullptr && m < Mp) {
        *reinterpret_cast<uint32_t *>(qp + (b * Mp + m) * SB + plane_pos(t)) = qword;
        if (t == 0)
            dp[b * Mp + m] = dst;
    }
    write_split(xs, m, b, t, dst, q0, q1, q2, q3);
}

// ABI Q8_1 blocks -> internal planes and/or the compensated bf16 planes.
// Same grid shape as k_quantize.
__global__ void __launch_bounds__(256)
k_q8_1_convert(const uint8_t *__restrict__ Xq, int8_t *__restrict__ qp, float *__restrict__ dp,
               ZeroList zl, XSplit xs, int64_t M, int64_t Mrows,
               int64_t Mp, int64_t K)
{
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    zero_list(zl, tid, (int64_t)gridDim.x * blockDim.x);
    const int64_t nblk_row = K / SB;
    const int64_t blk = tid >> 3;
    const int t = (int)(tid & 7);
    if (blk >= Mrows * nblk_row)
        return;
    const int64_t m = blk / nblk_row, b = blk - m * nblk_row;
    uint32_t qword = 0, head = 0;
    if (m < M) {
        const uint8_t *src = Xq + blk * XBLK;
        qword = *reinterpret_cast<const uint32_t *>(src + 4 + 4 * t);
        head = *reinterpret_cast<const uint32_t *>(src);
    }
    const float dst = half_bits_to_float(head & 0xFFFFu);
    if (qp != nullptr && m < Mp) {
        *reinterpret_cast<uint32_t *>(qp + (b * Mp + m) * SB + plane_pos(t)) = qword;
        if (t == 0)
            dp[b * Mp + m] = dst;
    }
    write_split(xs, m, b, t, dst, (int8_t)(qword & 0xFF), (int8_t)((qword >> 8) & 0xFF),
                (int8_t)((qword >> 16) & 0xFF), (int8_t)(qword >> 24));
}

}  // namespace

hipError_t launch_zero(float *y, int64_t n, hipStream_t s)
{
    if (n <= 0)
        return hipSuccess;
    const int64_t n4 = (n + 3) / 4;
    const int64_t grid = std::min<int64_t>((n4 + 255) / 256, 2048);
    hipLaunchKernelGGL(k_zero, dim3((unsigned)grid), dim3(256), 0, s, y, n);
    return hipGetLastError();
}

hipError_t launch_quantize(const float *X, void *Xq, const XPlanes *planes, int64_t M, int64_t K, hipStream_t s,
                           const ZeroList &zl, const XSplit *xs)
{
    const int64_t Mrows = xs ? xs->Ms : M;
    const int64_t threads = Mrows * (K / 4);
    const int64_t grid = (threads + 255) / 256;
    hipLaunchKernelGGL(k_quantize, dim3((unsigned)grid), dim3(256), 0, s, X, (uint8_t *)Xq,
                       planes ? planes->qp : nullptr, planes ? planes->dp : nullptr,
                       zl, xs ? *xs : XSplit(), M, Mrows,
                       planes ? planes->Mp : M, K);
    return hipGetLastError();
}

hipError_t launch_quantize(const float *X, void *Xq, const XPlanes *planes, int64_t M, int64_t K, hipStream_t s,
                           float *yz, int64_t nz, const XSplit *xs)
{
    ZeroList zl;
    if (yz != nullptr && nz > 0) {
        zl.p[0] = yz;
        zl.n[0] = nz;
        zl.count = 1;
    }
    return launch_quantize(X, Xq, planes, M, K, s, zl, xs);
}

hipError_t launch_zero_tiles(const ZeroTiles &zt, hipStream_t s)
{
    if (zt.count == 0)
        return hipSuccess;
    const int64_t n = (int64_t)zt.count * zt.bm * zt.bn / 4;
    const int64_t grid = std::min<int64_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(k_zero_tiles, dim3((unsigned)grid), dim3(256), 0, s, zt);
    return hipGetLastError();
}

hipError_t launch_q8_1_convert(const void *Xq, const XPlanes *planes, int64_t M, int64_t K, hipStream_t s,
                              float *yz, int64_t nz, const XSplit *xs)
{
    ZeroList zl;
    if (yz != nullptr && nz > 0) {
        zl.p[0] = yz;
        zl.n[0] = nz;
        zl.count = 1;
    }
    return launch_q8_1_convert(Xq, planes, M, K, s, zl, xs);
}

hipError_t launch_q8_1_convert(const void *Xq, const XPlanes *planes, int64_t M, int64_t K, hipStream_t s,
                              const ZeroList &zl, const XSplit *xs)
{
    const int64_t Mrows = xs ? xs->Ms : M;
    const int64_t threads = Mrows * (K / 4);
    const int64_t grid = (threads + 255) / 256;
    hipLaunchKernelGGL(k_q8_1_convert, dim3((unsigned)grid), dim3(256), 0, s, (const uint8_t *)Xq,
                       planes ? planes->qp : nullptr, planes ? planes->dp : nullptr,
                       zl, xs ? *xs : XSplit(), M, Mrows,
                       planes ? planes->Mp : M, K);
    return hipGetLastError();
}

}  // namespace iq4xs
