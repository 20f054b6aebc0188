/*
 * iq4xs_probe.h -- measurement kernels of libiq4xs.so: what one MI355X
 * sustains beside its published peaks.  Not part of the matmul; the
 * benchmark quotes them next to the matmul kernels' rooflines and uses the
 * read and write probes (known bytes) to calibrate the HBM traffic counters.
 * Source: "V100TPS engine log", opening section (the correctness gate pairs
 * every throughput figure with bytes-moved / time against the card's peak:
 * a figure above it means the kernel did not run).
 *
 * All pointers are device pointers owned by the caller; `stream` is a
 * hipStream_t passed as void*; calls are asynchronous.  Each returns 0, -1
 * for a bad argument (nothing launched) or -5 when the launch failed.
 */
#ifndef IQ4XS_PROBE_H
#define IQ4XS_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Read nbytes (a multiple of 16, src 16-byte aligned) with plain 16-byte
 * loads over `grid` workgroups of 256 threads, grid-strided;
 * one 32-bit value per workgroup is written to sink[0..grid). */
int iq4xs_probe_read(const void *src, size_t nbytes, void *sink, int grid, void *stream);

/* Write `value` to every 32-bit word of dst[0..nbytes) with plain 16-byte
 * stores (nbytes a multiple of 16, dst 16-byte aligned). */
int iq4xs_probe_write(void *dst, size_t nbytes, uint32_t value, int grid, void *stream);

/* Back-to-back matrix-core instructions: every wavefront of `grid`
 * workgroups of 256 threads issues 4*iters v_mfma_i32_32x32x32_i8
 * (kind IQ4XS_PROBE_MFMA_I8, 65536 int8 ops each) or
 * v_mfma_f32_32x32x16_bf16 (IQ4XS_PROBE_MFMA_BF16, 32768 flops each) in four
 * independent chains, then writes one value per thread to out[0..grid*256). */
#define IQ4XS_PROBE_MFMA_I8 0
#define IQ4XS_PROBE_MFMA_BF16 1
int iq4xs_probe_mfma(int kind, int iters, void *out, int grid, void *stream);

/* Matrix-core and vector-ALU work on the same SIMDs: `grid` workgroups of
 * 512 threads (eight wavefronts, two per SIMD when one workgroup runs per
 * compute unit).  Each iteration of `iters` holds 2 independent
 * v_mfma_i32_32x32x32_i8 and 96 independent v_fma_f32: 48 VALU operations
 * per MFMA, the mix of the int8 tile kernel's rescale (16 outputs of a
 * lane per MFMA, three VALU operations each).  mode IQ4XS_PROBE_MIX_MFMA: every wavefront issues only the
 * MFMAs; _VALU: only the FMAs; _SAME: both, in every wavefront; _SPLIT: the
 * two wavefronts of a SIMD split them (one the MFMAs, the other the FMAs), so
 * that each SIMD gets half of _SAME's work.  One value per thread is written
 * to out[0..grid*512) (int32).  The ratio of _SAME to _MFMA + _VALU says
 * whether the two kinds of work overlap on a SIMD. */
#define IQ4XS_PROBE_MIX_MFMA 0
#define IQ4XS_PROBE_MIX_VALU 1
#define IQ4XS_PROBE_MIX_SAME 2
#define IQ4XS_PROBE_MIX_SPLIT 3
int iq4xs_probe_mix(int mode, int iters, void *out, int grid, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* IQ4XS_PROBE_H */
