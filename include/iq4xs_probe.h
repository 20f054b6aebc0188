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

#ifdef __cplusplus
}
#endif

#endif /* IQ4XS_PROBE_H */
