// deq.hip -- IQ4_XS weights dequantized to bf16 (iq4xs_dequantize_bf16).
//
// Prior art: "V100TPS engine log" (agent-report.daedalus.work/V100TPS/engine.html,
// M=64 kernel-launch table): dequantize_block_iq4_xs writes the whole weight in
// fp16 before a dense tensor-core GEMM.  Here every weight d*(ls-32)*kv is
// exact in fp32 and rounded once to bf16 (nearest even).  The matmul paths do
// not materialise this copy: DEQ_BF16 and BF16X3 dequantize inside the GEMM
// (fused.hip); this kernel serves callers that want the bf16 weights
// themselves, and the tests that pin the rounding.
#include "common.hpp"

namespace iq4xs {
namespace {

__device__ __forceinline__ uint32_t bf16_rne(float f)
{
    const uint32_t u = __builtin_bit_cast(uint32_t, f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    return bf16_rne(lo) | (bf16_rne(hi) << 16);
}

// One thread per half sub-block (16 weights).
__global__ void __launch_bounds__(256)
k_dequant_bf16(const uint8_t *__restrict__ W, uint16_t *__restrict__ Wb, int64_t N, int64_t K)
{
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t units = K / 16;
    if (tid >= N * units)
        return;
    const int64_t n = tid / units, u = tid - n * units;
    const int64_t b = u >> 1;
    const int h = (int)(u & 1);
    const uint8_t *blk = W + (n * (K / QK) + (b >> 3)) * WBLK;
    const uint2 hdr = *reinterpret_cast<const uint2 *>(blk);
    const uint2 qs = *reinterpret_cast<const uint2 *>(blk + QS_OFF + 16 * (b & 7) + 8 * h);
    uint32_t wv[4];
    expand8(qs.x, qs.y, wv);
    const float sw = sub_scale(hdr.x, hdr.y, (int)(b & 7));
    uint32_t o[8];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint32_t v = wv[i];
        o[2 * i] = pack_bf16x2(sw * (float)(int8_t)(v & 0xFF), sw * (float)(int8_t)((v >> 8) & 0xFF));
        o[2 * i + 1] = pack_bf16x2(sw * (float)(int8_t)((v >> 16) & 0xFF), sw * (float)(int8_t)(v >> 24));
    }
    // wv[0..1] -> elements 8h..8h+7, wv[2..3] -> elements 16+8h..16+8h+7
    uint16_t *dst = Wb + n * K + 32 * b + 8 * h;
    *reinterpret_cast<uint4 *>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<uint4 *>(dst + 16) = make_uint4(o[4], o[5], o[6], o[7]);
}

}  // namespace

hipError_t launch_dequant_bf16(const void *W, uint16_t *Wb, int64_t N, int64_t K, hipStream_t s)
{
    const int64_t threads = N * (K / 16);
    hipLaunchKernelGGL(k_dequant_bf16, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                       (const uint8_t *)W, Wb, N, K);
    return hipGetLastError();
}

}  // namespace iq4xs
