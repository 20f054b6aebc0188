// probe.hip -- measurement kernels (include/iq4xs_probe.h): what this device
// sustains for a plain stream read, a plain stream write, back-to-back
// int8 and bf16 matrix-core instructions, and matrix-core beside vector-ALU
// work on the same SIMDs.  The matmul's rooflines are quoted
// against the published peaks; these give the achievable figures beside them
// ("V100TPS engine log", opening section: a bytes-moved / time check against
// the card's peak exposes a kernel that did not run).  They also calibrate
// the HBM traffic counters: a read of known bytes and a write of known bytes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "iq4xs_probe.h"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int PT = 256;            // threads per workgroup

// Every thread reads 16-byte pieces i = tid, tid + stride, ... of src (plain
// loads, as the matmul kernels' reads) and
// folds them into one value; one value per workgroup is stored (so the loads
// cannot be dropped).  n16 = number of 16-byte pieces.
__global__ void __launch_bounds__(PT) k_probe_read(const u4 *__restrict__ src, uint64_t n16,
                                                   uint32_t *__restrict__ sink)
{
    const uint64_t stride = (uint64_t)gridDim.x * PT;
    uint64_t i = (uint64_t)blockIdx.x * PT + threadIdx.x;
    uint32_t a = 0, b = 0, c = 0, d = 0;
    // four pieces in flight per thread
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const u4 v0 = src[i];
        const u4 v1 = src[i + stride];
        const u4 v2 = src[i + 2 * stride];
        const u4 v3 = src[i + 3 * stride];
        a ^= v0.x ^ v1.y ^ v2.z ^ v3.w;
        b ^= v0.y ^ v1.z ^ v2.w ^ v3.x;
        c ^= v0.z ^ v1.w ^ v2.x ^ v3.y;
        d ^= v0.w ^ v1.x ^ v2.y ^ v3.z;
    }
    for (; i < n16; i += stride) {
        const u4 v = src[i];
        a ^= v.x;
        b ^= v.y;
        c ^= v.z;
        d ^= v.w;
    }
    uint32_t r = a ^ b ^ c ^ d;
    for (int off = 32; off >= 1; off >>= 1)
        r ^= __shfl_xor(r, off, 64);
    __shared__ uint32_t part[PT / 64];
    if ((threadIdx.x & 63) == 0)
        part[threadIdx.x >> 6] = r;
    __syncthreads();
    if (threadIdx.x == 0)
        sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

// dst[i] = value for every 16-byte piece, grid-strided (plain stores, as the
// matmul kernels' writes).
__global__ void __launch_bounds__(PT) k_probe_write(u4 *__restrict__ dst, uint64_t n16, uint32_t value)
{
    const uint64_t stride = (uint64_t)gridDim.x * PT;
    const u4 v = {value, value, value, value};
    for (uint64_t i = (uint64_t)blockIdx.x * PT + threadIdx.x; i < n16; i += stride)
        dst[i] = v;
}

// Each wavefront issues `iters` rounds of four independent
// v_mfma_i32_32x32x32_i8 (or v_mfma_f32_32x32x16_bf16) chains, so the
// matrix core never waits on a result; the accumulators are stored so that
// nothing is dropped.  Operands are lane-dependent constants.
__global__ void __launch_bounds__(PT) k_probe_mfma_i8(int iters, int *__restrict__ out)
{
    const int lane = threadIdx.x & 63;
    const v4i a = {lane, lane + 1, lane * 3, 7};
    const v4i b = {1, lane, 2, lane ^ 5};
    v16i c0 = {0}, c1 = {0}, c2 = {0}, c3 = {0};
    for (int i = 0; i < iters; i++) {
        c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, b, c3, 0, 0, 0);
    }
    int s = 0;
#pragma unroll
    for (int r = 0; r < 16; r++)
        s += c0[r] ^ c1[r] ^ c2[r] ^ c3[r];
    out[(size_t)blockIdx.x * PT + threadIdx.x] = s;
}

__global__ void __launch_bounds__(PT) k_probe_mfma_bf16(int iters, float *__restrict__ out)
{
    const int lane = threadIdx.x & 63;
    v8bf a, b;
#pragma unroll
    for (int k = 0; k < 8; k++) {
        a[k] = (__bf16)(float)((lane + k) & 7);
        b[k] = (__bf16)(float)((lane * 3 + k) & 5);
    }
    v16f c0 = {0}, c1 = {0}, c2 = {0}, c3 = {0};
    for (int i = 0; i < iters; i++) {
        c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, c1, 0, 0, 0);
        c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, c2, 0, 0, 0);
        c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, c3, 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; r++)
        s += c0[r] + c1[r] + c2[r] + c3[r];
    out[(size_t)blockIdx.x * PT + threadIdx.x] = s;
}

// MODE: 0 MFMAs only, 1 FMAs only, 2 both in every wavefront, 3 split
// between the two wavefronts of a SIMD (waves w and w+4 of the workgroup,
// which the compute unit places on the same SIMD).
template <int MODE>
__global__ void __launch_bounds__(512) k_probe_mix(int iters, int *__restrict__ out)
{
    constexpr int NV = 96;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool dm = MODE == 0 || MODE == 2 || (MODE == 3 && ((wave >> 2) & 1) == 0);
    const bool dv = MODE == 1 || MODE == 2 || (MODE == 3 && ((wave >> 2) & 1) == 1);
    const v4i a = {lane, lane + 1, lane * 3, 7};
    const v4i b = {1, lane, 2, lane ^ 5};
    v16i c0 = {0}, c1 = {0};
    float f[NV];
#pragma unroll
    for (int j = 0; j < NV; j++)
        f[j] = 1.0f + 0.001f * (float)(lane + j);
    const float x = 0.999f + 1e-6f * (float)lane, y = 1e-3f;
    for (int i = 0; i < iters; i++) {
        if (dm) {                                              // (uniform)
            c0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(b, a, c1, 0, 0, 0);
        }
        if (dv) {
#pragma unroll
            for (int j = 0; j < NV; j++)
                f[j] = __builtin_fmaf(f[j], x, y);
        }
    }
    int s = 0;
#pragma unroll
    for (int r = 0; r < 16; r++)
        s += c0[r] ^ c1[r];
    // 96 KB of LDS (never used: iters >= 1) so that one workgroup runs per
    // compute unit, two wavefronts per SIMD
    __shared__ int hold[96 * 256];
    if (iters < 0) {
        hold[tid] = s;
        __syncthreads();
        s += hold[(tid + 1) & 511];
    }
    float t = 0.0f;
#pragma unroll
    for (int j = 0; j < NV; j++)
        t += f[j];
    out[(size_t)blockIdx.x * 512 + tid] = s + (int)t;
}

int launch_status(void)
{
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? 0 : -5;
}

}  // namespace

extern "C" {

int iq4xs_probe_read(const void *src, size_t nbytes, void *sink, int grid, void *stream)
{
    if (!src || !sink || nbytes == 0 || nbytes % 16 || grid < 1 || grid > 65536 || ((uintptr_t)src % 16) ||
        ((uintptr_t)sink % 4))
        return -1;
    hipLaunchKernelGGL(k_probe_read, dim3((unsigned)grid), dim3(PT), 0, (hipStream_t)stream,
                       (const u4 *)src, (uint64_t)(nbytes / 16), (uint32_t *)sink);
    return launch_status();
}

int iq4xs_probe_write(void *dst, size_t nbytes, uint32_t value, int grid, void *stream)
{
    if (!dst || nbytes == 0 || nbytes % 16 || grid < 1 || grid > 65536 || ((uintptr_t)dst % 16))
        return -1;
    hipLaunchKernelGGL(k_probe_write, dim3((unsigned)grid), dim3(PT), 0, (hipStream_t)stream, (u4 *)dst,
                       (uint64_t)(nbytes / 16), value);
    return launch_status();
}

int iq4xs_probe_mfma(int kind, int iters, void *out, int grid, void *stream)
{
    if (!out || iters < 1 || grid < 1 || grid > 65536 || ((uintptr_t)out % 4))
        return -1;
    if (kind == IQ4XS_PROBE_MFMA_I8)
        hipLaunchKernelGGL(k_probe_mfma_i8, dim3((unsigned)grid), dim3(PT), 0, (hipStream_t)stream, iters,
                           (int *)out);
    else if (kind == IQ4XS_PROBE_MFMA_BF16)
        hipLaunchKernelGGL(k_probe_mfma_bf16, dim3((unsigned)grid), dim3(PT), 0, (hipStream_t)stream, iters,
                           (float *)out);
    else
        return -1;
    return launch_status();
}

int iq4xs_probe_mix(int mode, int iters, void *out, int grid, void *stream)
{
    if (!out || iters < 1 || grid < 1 || grid > 65536 || ((uintptr_t)out % 4) || mode < IQ4XS_PROBE_MIX_MFMA ||
        mode > IQ4XS_PROBE_MIX_SPLIT)
        return -1;
    const hipStream_t s = (hipStream_t)stream;
    int *o = (int *)out;
    switch (mode) {
    case IQ4XS_PROBE_MIX_MFMA: hipLaunchKernelGGL(k_probe_mix<0>, dim3((unsigned)grid), dim3(512), 0, s, iters, o); break;
    case IQ4XS_PROBE_MIX_VALU: hipLaunchKernelGGL(k_probe_mix<1>, dim3((unsigned)grid), dim3(512), 0, s, iters, o); break;
    case IQ4XS_PROBE_MIX_SAME: hipLaunchKernelGGL(k_probe_mix<2>, dim3((unsigned)grid), dim3(512), 0, s, iters, o); break;
    default: hipLaunchKernelGGL(k_probe_mix<3>, dim3((unsigned)grid), dim3(512), 0, s, iters, o); break;
    }
    return launch_status();
}

}  // extern "C"
