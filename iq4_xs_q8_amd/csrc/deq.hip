// deq.hip -- the dequantize-then-dense-GEMM path.
//
// Prior art: "V100TPS engine log" (agent-report.daedalus.work/V100TPS/engine.html,
// M=64 kernel-launch table): dequantize_block_iq4_xs writes the whole weight in
// fp16 and a dense tensor-core GEMM follows; its cost is flat in M, so it wins
// only at prefill-sized M.  Here: W -> bf16 (every weight d*(ls-32)*kv is
// exact in fp32, then rounded once to bf16), X~ = bf16(d_x*q) from the same
// Q8_1 activations, and a bf16 MFMA GEMM with fp32 accumulation.  bf16 keeps
// 8 significant bits, so this path is an approximation of the integer-dot
// result; it exists for the prefill crossover and is never chosen by the
// default dispatch table.
#include "common.hpp"

namespace iq4xs {
namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

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

// ---------------------------------------------------------------- GEMM
// C[M,N] = A[M,K] * B[N,K]^T, A and B bf16 row-major (K contiguous), C fp32.
// Workgroup tile 128x128, K step 64, 4 wavefronts in a 2x2 grid of 64x64,
// each a 2x2 grid of v_mfma_f32_32x32x16_bf16 tiles.  LDS rows are padded by
// 8 bf16 to spread the 16-byte fragment reads over the banks.
constexpr int BM = 128, BN = 128, BK = 64, LDS_STRIDE = BK + 8;

__global__ void __launch_bounds__(256)
k_gemm_bf16(const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, float *__restrict__ C,
            int64_t M, int64_t N, int64_t K)
{
    __shared__ __attribute__((aligned(16))) uint16_t As[BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[BN * LDS_STRIDE];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)blockIdx.x * BM, n0 = (int64_t)blockIdx.y * BN;
    const int col = lane & 31, h = lane >> 5;

    v16f acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                acc[i][j][r] = 0.0f;

    for (int64_t k0 = 0; k0 < K; k0 += BK) {
        // global -> LDS: 128 rows x 8 chunks of 16 bytes per operand, 4 chunks per thread
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int c = tid + 256 * i;
            const int r = c >> 3, kc = c & 7;
            uint4 va = make_uint4(0, 0, 0, 0), vb = make_uint4(0, 0, 0, 0);
            if (m0 + r < M)
                va = *reinterpret_cast<const uint4 *>(A + (m0 + r) * K + k0 + 8 * kc);
            if (n0 + r < N)
                vb = *reinterpret_cast<const uint4 *>(B + (n0 + r) * K + k0 + 8 * kc);
            *reinterpret_cast<uint4 *>(As + r * LDS_STRIDE + 8 * kc) = va;
            *reinterpret_cast<uint4 *>(Bs + r * LDS_STRIDE + 8 * kc) = vb;
        }
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < BK / 16; ks++) {
            v8bf a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; i++) {
                const uint4 ra = *reinterpret_cast<const uint4 *>(
                    As + (64 * wm + 32 * i + col) * LDS_STRIDE + 16 * ks + 8 * h);
                a[i] = __builtin_bit_cast(v8bf, ra);
                const uint4 rb = *reinterpret_cast<const uint4 *>(
                    Bs + (64 * wn + 32 * i + col) * LDS_STRIDE + 16 * ks + 8 * h);
                b[i] = __builtin_bit_cast(v8bf, rb);
            }
#pragma unroll
            for (int i = 0; i < 2; i++)
#pragma unroll
                for (int j = 0; j < 2; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++) {
            const int64_t n = n0 + 64 * wn + 32 * j + col;
            if (n >= N)
                continue;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int64_t m = m0 + 64 * wm + 32 * i + 8 * (r / 4) + 4 * h + (r % 4);
                if (m < M)
                    C[m * N + n] = acc[i][j][r];
            }
        }
}

}  // namespace

hipError_t launch_dequant_bf16(const void *W, uint16_t *Wb, int64_t N, int64_t K, hipStream_t s)
{
    const int64_t threads = N * (K / 16);
    hipLaunchKernelGGL(k_dequant_bf16, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                       (const uint8_t *)W, Wb, N, K);
    return hipGetLastError();
}

hipError_t launch_gemm_bf16(const uint16_t *Xb, const uint16_t *Wb, float *Y, int64_t M, int64_t N,
                            int64_t K, hipStream_t s)
{
    const dim3 grid((unsigned)((M + BM - 1) / BM), (unsigned)((N + BN - 1) / BN));
    hipLaunchKernelGGL(k_gemm_bf16, grid, dim3(256), 0, s, Xb, Wb, Y, M, N, K);
    return hipGetLastError();
}

}  // namespace iq4xs
