/*
 * iq4xs.h -- C ABI of libiq4xs.so: the IQ4_XS x Q8_1 quantized matmul
 *            Y[M,N] = X[M,K] * W[N,K]^T on AMD Instinct MI355X (gfx950).
 *
 * Sources.  "V100TPS engine log" (agent-report.daedalus.work/V100TPS/engine.html):
 *   - section on the batched IQ4_XS kernel: the IQ4_XS sub-block (32 weights
 *     in four 32-bit words, low nibbles = elements 0-15, high nibbles =
 *     16-31), the per-sub-block scale d*(ls-32), the kvalues_iq4nl lookup in
 *     place of q-8, and the Q8_1-quantized activations;
 *   - the M=64 kernel-launch table: quantize_q8_1 followed by the matmul; the
 *     dequantize-then-dense-GEMM path;
 *   - the mmvq vs dequant+GEMM table and the new-kernel vs dispatcher table:
 *     one path per range of M, chosen by a dispatcher.
 * "SGLang MoE port thread" (lcz.me/post/31556), section on the torch bridge:
 *   the stream crosses the boundary as a plain integer handle and the shim
 *   includes no framework header.
 *
 * Formats (GGUF; the pages name them but print no byte layout):
 *   IQ4_XS super-block, 136 bytes, 256 weights along K:
 *     bytes 0-1   fp16 d
 *     bytes 2-3   u16 scales_h: bits 2b..2b+1 = high 2 bits of ls_b
 *     bytes 4-7   u8 scales_l[4]: nibble b%2 of scales_l[b/2] = low 4 bits of ls_b
 *     bytes 8-135 u8 qs[128]: sub-block b (elements 32b..32b+31) owns
 *                 qs[16b..16b+15]; element 32b+t is the low nibble of
 *                 qs[16b+t] for t < 16 and the high nibble of qs[16b+t-16]
 *                 otherwise.
 *     weight = d * (ls_b - 32) * kvalues_iq4nl[index].
 *   W is [N][K/256] super-blocks: row n's blocks are contiguous.
 *   Q8_1 block, 36 bytes, 32 activations: fp16 d, fp16 s, int8 q[32].
 *     d = fp16(amax/127), q = round-half-away(x / (amax/127)) computed in
 *     IEEE fp32 (q = 0 if the fp32 scale is 0), s = fp16(d * sum q).
 *   Xq is [M][K/32] blocks, row-major.
 *   X and Y are dense row-major fp32, [M][K] and [M][N].
 *
 * Conventions for every entry point:
 *   - returns IQ4XS_OK (0) or a negative IQ4XS_E* code and never throws; the
 *     message of the last error on the calling thread is iq4xs_last_error();
 *   - arguments are validated on the host before any HIP call;
 *   - device pointers are caller-owned (the library never frees them);
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream);
 *     work is enqueued asynchronously and stream-ordered, there is no host
 *     synchronisation; errors raised while kernels execute surface at the
 *     caller's next synchronisation, as in HIP;
 *   - the library is thread-safe; environment variables are read once, at
 *     the first call.
 */
#ifndef IQ4XS_H
#define IQ4XS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ---- */
#define IQ4XS_OK 0
#define IQ4XS_EINVAL (-1)  /* null pointer, M/N < 1, K not a multiple of 256, size overflow
                              (for the matmul entry points also M*K >= 1.9e9: the
                              activations' internal copy must stay below 2 GiB),
                              Y overlapping an input, unknown path                         */
#define IQ4XS_EALIGN (-2)  /* W, X or Y not 16-byte aligned, Xq not 4-byte aligned          */
#define IQ4XS_EDEVICE (-3) /* no HIP device, or the current device is not gfx950            */
#define IQ4XS_ETABLE (-4)  /* dispatch table unreadable, malformed, or for another device   */
#define IQ4XS_ELAUNCH (-5) /* a HIP runtime call or a kernel launch failed                  */
#define IQ4XS_ENOMEM (-6)  /* stream-ordered scratch allocation failed                      */
#define IQ4XS_EPATH (-7)   /* the requested path cannot run this shape                     */

/* ---- paths ---- */
#define IQ4XS_PATH_AUTO 0     /* the dispatcher picks from its measured table            */
#define IQ4XS_PATH_GEMV 1     /* wavefront-per-row integer-dot kernel, 1 <= M <= 4        */
#define IQ4XS_PATH_MMQ 2      /* int8-MFMA tile kernel, any M                             */
#define IQ4XS_PATH_DEQ_BF16 3 /* W~ and X~ rounded to bf16, bf16-MFMA GEMM, W dequantized
                                 inside the GEMM (inexact: 8 significant bits per operand) */
#define IQ4XS_PATH_BF16X3 4   /* W dequantized inside the GEMM into LDS, W~ and X~ each as
                                 bf16 hi + lo, three bf16-MFMA products per term (within
                                 the per-row bound; see iq4xs_gemm_path)                 */
#define IQ4XS_NUM_PATHS 5

/* ---- weight formats (the iq4xs_*_fmt entry points) ----
 * "V100TPS engine log", batched IQ4_XS kernel section: an IQ4_XS sub-block of
 * 32 weights has the geometry of a whole Q4_0 block (16 bytes of nibbles, low
 * nibbles elements 0-15, high nibbles 16-31); Q4_0 keeps one scale d per block
 * and the value q-8, IQ4_XS stores d*(ls-32) per sub-block and looks the value
 * up in kvalues_iq4nl.  "SGLang MoE port thread", the passage that retracts a
 * TP block-alignment conclusion: an IQ4_NL block is 32 values in 18 bytes.
 * Byte order (GGUF; convention): IQ4_NL and Q4_0 blocks are {fp16 d, u8 qs[16]}
 * with the IQ4_XS sub-block's nibble placement; a row of K weights is K/32
 * consecutive blocks.  The kernels work in units of 256 weights, so K must be
 * a multiple of 256 for every format. */
#define IQ4XS_FMT_IQ4_XS 0 /* 136-byte super-blocks of 256 weights (above)            */
#define IQ4XS_FMT_IQ4_NL 1 /* 18-byte blocks of 32 weights, weight d*kvalues_iq4nl[q] */
#define IQ4XS_FMT_Q4_0 2   /* 18-byte blocks of 32 weights, weight d*(q-8)             */

/* Sizes in bytes of an IQ4_XS matrix [N][K] and of a Q8_1 matrix [M][K]:
 * N*(K/256)*136 and M*(K/32)*36.  The "V100TPS engine log", section on the
 * batched IQ4_XS kernel, names both formats and the 32-weight sub-block with
 * its own scale d*(ls-32); the byte counts per block are the GGUF formats'
 * (the pages print none).  *out is written only on success.  EINVAL for a
 * null `out`, non-positive sizes, K % 256 != 0 (K % 32 for Q8_1), overflow.
 * Host-only: no HIP call. */
int iq4xs_weight_bytes(int64_t N, int64_t K, size_t *out);
int iq4xs_q8_1_bytes(int64_t M, int64_t K, size_t *out);

/* Optional explicit initialisation: reads IQ4XS_DISPATCH_TABLE, IQ4XS_LOG and
 * IQ4XS_ALLOW_BF16 and loads the dispatch table.  Every other entry point calls
 * it on first use.  Does not touch the GPU. */
int iq4xs_init(void);

/* Quantize fp32 X [M][K] to Q8_1 Xq [M][K/32] (36-byte blocks), bit-exactly as
 * described above ("V100TPS engine log", M=64 kernel-launch table:
 * quantize_q8_1).  K % 32 == 0.  X 16-byte aligned, Xq 4-byte aligned. */
int iq4xs_quantize_q8_1(const float *X, void *Xq, int64_t M, int64_t K, void *stream);

/* Y = X * W^T with X quantized to Q8_1 on the device ("V100TPS engine log",
 * batched IQ4_XS kernel section).  Quantization, the dispatcher's choice of
 * path and the matmul are all enqueued on `stream`.  Y is overwritten.
 * Stream-ordered scratch (about 1.2*M*K bytes; 4*K*M' for the bf16 paths,
 * M' = M rounded up to 256) is allocated from the device's default memory
 * pool and released on `stream`. */
int iq4xs_gemm(const void *W, const float *X, float *Y, int64_t M, int64_t N, int64_t K,
               void *stream);

/* As iq4xs_gemm with the path forced (IQ4XS_PATH_*; AUTO = dispatcher).
 * BF16X3 ("V100TPS engine log", M=64 kernel-launch table: dequantize, then a
 * dense tensor-core GEMM; "V100TPS MTP investigation", crossover passage:
 * the dense path wins at larger M): each weight d*(ls-32)*kv and each
 * d_x*q is split into hi = bf16(v) and lo = bf16(v - hi) (nearest even),
 * and Wh*Xh + Wh*Xl + Wl*Xh is summed in fp32 on the matrix cores, the
 * weights dequantized per 32-weight sub-block into LDS (no bf16 copy of W in
 * HBM).  Each product is within 3.02*2^-16 of the exact one, so the result
 * meets the same per-row bound as GEMV and MMQ (measured per-row ratio near
 * 1e-5) and the table may route to it without an opt-in.  IQ4_XS weights
 * only; EPATH when the activation planes would reach 2 GiB. */
int iq4xs_gemm_path(const void *W, const float *X, float *Y, int64_t M, int64_t N, int64_t K,
                    int path, void *stream);

/* Caller-provided scratch: iq4xs_gemm_ws is iq4xs_gemm_path with the
 * scratch supplied by the caller (`workspace`, at least
 * iq4xs_gemm_workspace_bytes(M, N, K, path) bytes, 256-byte aligned, not
 * overlapping W, X or Y: IQ4XS_EINVAL).  It allocates nothing, so it can be recorded into a
 * HIP graph; calls that share one workspace must be ordered on one stream.
 * The size query resolves AUTO with the dispatch table in force. */
int iq4xs_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int path, size_t *out);
int iq4xs_gemm_ws(const void *W, const float *X, float *Y, int64_t M, int64_t N, int64_t K, int path,
                  void *workspace, size_t workspace_bytes, void *stream);

/* For callers that cannot allocate -- code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc: iq4xs_gemm_path with its
 * scratch taken from a static device array of the library, of
 * IQ4XS_STATIC_SCRATCH_BYTES per device, instead of the stream-ordered
 * allocation.  Nothing is allocated: no hipMalloc/hipFree, no pool call.
 * Arguments, result and errors are iq4xs_gemm_path's; in addition EINVAL
 * when the shape and path need more scratch than the array holds (the need
 * is iq4xs_gemm_workspace_bytes(M, N, K, path)).  Each device has its own
 * array, held from the first call on that device until the process ends.
 * Every call on one device uses that device's array and leaves its contents
 * behind: calls that overlap in time on one device (two streams, two threads)
 * race and give undefined results, so order them on one stream. */
#define IQ4XS_STATIC_SCRATCH_BYTES (128u << 20)
int iq4xs_gemm_noalloc(const void *W, const float *X, float *Y, int64_t M, int64_t N, int64_t K,
                       int path, void *stream);

/* The matmul for weights in any of the three formats: W is [N] rows of
 * iq4xs_weight_bytes_fmt(fmt, 1, K) bytes (caller-owned, 16-byte aligned),
 * X fp32 [M][K], Y fp32 [M][N] (overwritten).  Arithmetic as iq4xs_gemm:
 * X quantized to Q8_1, per 32-weight block the exact integer dot of the
 * block's values with the Q8_1 values, scaled in fp32 by d (or d*(ls-32))
 * and d_x; the result is within the same per-row bound of the oracle.
 * `path`: AUTO (the measured table's GEMV / MMQ bands; its bf16 bands
 * apply to IQ4_XS only), GEMV (M <= 4) or MMQ; DEQ_BF16 and BF16X3 are EPATH for IQ4_NL
 * and Q4_0, and so is MMQ for a matrix of 2 GiB or more in those formats
 * (the fallback kernel for such sizes reads IQ4_XS only).  `workspace` as in
 * iq4xs_gemm_ws (at least iq4xs_gemm_fmt_workspace_bytes bytes, 256-byte
 * aligned; then nothing is allocated), or NULL for stream-ordered scratch.
 * EINVAL for an unknown `fmt` and as iq4xs_gemm_path otherwise.
 * iq4xs_weight_bytes_fmt: N*(K/256)*136 (IQ4_XS) or N*(K/32)*18. */
int iq4xs_weight_bytes_fmt(int fmt, int64_t N, int64_t K, size_t *out);
int iq4xs_gemm_fmt_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K, int path, size_t *out);
int iq4xs_gemm_fmt(int fmt, const void *W, const float *X, float *Y, int64_t M, int64_t N, int64_t K,
                   int path, void *workspace, size_t workspace_bytes, void *stream);

/* Y = X * W^T from activations already quantized to Q8_1 (Xq [M][K/32]
 * blocks of 36 bytes, layout above; caller-owned, 4-byte aligned, read only).
 * The "V100TPS engine log", M=64 kernel-launch table, shows quantize_q8_1 as
 * a launch of its own ahead of the matmul: this entry point is that matmul
 * on its own, on the same path choice as iq4xs_gemm_path.  Y is overwritten;
 * the result equals iq4xs_gemm_path's on the X that Xq quantizes.  Errors as
 * iq4xs_gemm_path (EALIGN for Xq not 4-byte aligned). */
int iq4xs_gemm_q8_1(const void *W, const void *Xq, float *Y, int64_t M, int64_t N, int64_t K,
                    int path, void *stream);

/* Prepared activations: X quantized once (bit-identical to
 * iq4xs_quantize_q8_1) into the layout the GEMV and MMQ kernels read, so one
 * quantization can feed several weight matrices and the matmul kernel can be
 * launched on its own.  `act` is a caller-owned device buffer of
 * iq4xs_act_bytes(M, K) bytes, 256-byte aligned; its contents are private to
 * the library (int8 values reordered per 32-block plus one fp32 scale per
 * block, rows padded to a multiple of 4).  K % 256 == 0. */
int iq4xs_act_bytes(int64_t M, int64_t K, size_t *out);
int iq4xs_prepare_act(const float *X, void *act, int64_t M, int64_t K, void *stream);
/* Y = X * W^T from prepared activations; path AUTO, GEMV or MMQ (DEQ_BF16 and
 * BF16X3 are EPATH here; AUTO takes MMQ where the table names BF16X3).  Launches the matmul kernel only -- plus, where output tiles
 * are shared by more than two workgroups (MMQ tile kernel with few tiles,
 * K-split fallback), a second kernel that adds their partial results in a
 * fixed order from a stream-ordered workspace; and, where the MMQ kernels
 * share output tiles between two workgroups (which add into Y), a kernel
 * that zeroes Y first.  OR IQ4XS_Y_ZEROED into `path` when Y already holds
 * zeros (e.g. cleared together with other buffers): that zeroing kernel is
 * then skipped and the result is the same; with any other Y contents the
 * result of such shared tiles is undefined.  Shapes without such tiles
 * overwrite Y and ignore the flag. */
#define IQ4XS_Y_ZEROED 0x100
int iq4xs_gemm_act(const void *W, const void *act, float *Y, int64_t M, int64_t N, int64_t K,
                   int path, void *stream);
/* iq4xs_gemm_act with the partial-result scratch supplied by the caller, so
 * that the launch allocates nothing and can be recorded into a HIP graph.
 * iq4xs_gemm_act_workspace_bytes gives the bytes that the shape and path need
 * (AUTO resolved with the dispatch table in force, IQ4XS_Y_ZEROED ignored);
 * most shapes need 0, and then `workspace` may be NULL.  Otherwise
 * `workspace` holds at least that many bytes, is 256-byte aligned and does
 * not overlap W, act or Y (EINVAL for NULL, too small or overlapping; EALIGN
 * when misaligned).  Its contents on entry do not matter and are left
 * undefined; calls that share one workspace must be ordered on one stream.
 * Result and other errors as iq4xs_gemm_act. */
int iq4xs_gemm_act_workspace_bytes(int64_t M, int64_t N, int64_t K, int path, size_t *out);
int iq4xs_gemm_act_ws(const void *W, const void *act, float *Y, int64_t M, int64_t N, int64_t K, int path,
                      void *workspace, size_t workspace_bytes, void *stream);

/* Several weight matrices that share one X ("SGLang MoE port thread",
 * decode measurements of the grouped expert call: one call per layer,
 * because a single small call is dominated by launch cost and a grouped one
 * adds little per extra unit): Y[g] = X * W[g]^T for g < G, with X quantized
 * once and, when the shapes allow (M <= 32, K/256 even), one launch of the
 * streaming matmul kernel over the tiles of all G matrices, numbered one
 * matrix after the other.  W, Y and N are host arrays of G entries:
 * W[g] [N[g]][K/256] IQ4_XS super-blocks, Y[g] fp32 [M][N[g]] (overwritten);
 * 1 <= G <= IQ4XS_MAX_GROUP; pointers 16-byte aligned; no Y[g] may overlap X,
 * any W[h] or another Y[h].  Other shapes run one iq4xs_gemm per matrix.
 * Every output is within the same bound of the oracle as iq4xs_gemm; where a
 * tile's K range is split between workgroups at other points than in a
 * single-matrix call, the last bits can differ from that call's.  Scratch:
 * `workspace` (256-byte aligned, at least iq4xs_gemm_group_workspace_bytes
 * bytes, overlapping no input or output; then nothing is allocated and the
 * call can be captured in a graph), or NULL for stream-ordered scratch from
 * the device's default pool. */
#define IQ4XS_MAX_GROUP 4
int iq4xs_gemm_group_workspace_bytes(const int64_t *N, int G, int64_t M, int64_t K, size_t *out);
int iq4xs_gemm_group(const void *const *W, float *const *Y, const int64_t *N, int G, const float *X,
                     int64_t M, int64_t K, void *workspace, size_t workspace_bytes, void *stream);

/* Dequantize W [N][K] to bf16 Wb [N][K] (row-major): each weight
 * d*(ls-32)*kvalues[index], computed exactly in fp32, rounded to the nearest
 * bf16 (ties to even).  ("V100TPS engine log", M=64 kernel-launch table:
 * dequantize_block_iq4_xs before the dense GEMM.)  Wb 16-byte aligned. */
int iq4xs_dequantize_bf16(const void *W, void *Wb, int64_t N, int64_t K, void *stream);

/* Host-only query: the path IQ4XS_PATH_AUTO resolves to for (M, N, K) under the
 * loaded table ("V100TPS engine log", mmvq vs dequant+GEMM table: the band
 * boundaries are measured, not hard-coded). */
int iq4xs_dispatch(int64_t M, int64_t N, int64_t K, int *path_out);

/* Replace the dispatch table with the one in `path` (NULL: the built-in
 * default).  "V100TPS engine log", mmvq vs dequant+GEMM table: the measured
 * crossover sat near M = 15 while the dispatcher's hard-coded threshold was 8;
 * here the bands are data measured on the device they name, and a table that
 * cannot be read or parsed is refused as a whole (ETABLE; the previous table
 * stays in force).  `path` is a host file path, read once during the call.
 * Format: text lines
 *   arch <gfx name>
 *   cus <compute units>        (optional: the device the bands were measured on)
 *   band <GEMV|MMQ|BF16X3|DEQ_BF16> <M_lo> <M_hi> <N> <K>
 * where N and K are "*" (any), a value, or an inclusive range "lo-hi";
 * '#' starts a comment; the first band that matches (M, N, K) wins; DEQ_BF16
 * bands are skipped unless IQ4XS_ALLOW_BF16=1 was set at initialisation.
 * With a `cus` line, a call that asks for IQ4XS_PATH_AUTO on a device with
 * another number of compute units (e.g. a partitioned one) fails with ETABLE;
 * explicit paths and the host-only iq4xs_dispatch query are unaffected. */
int iq4xs_load_dispatch_table(const char *path);

/* Name of a path ("AUTO", "GEMV", "MMQ", "DEQ_BF16", "BF16X3") or "?" */
const char *iq4xs_path_name(int path);

/* Message for the last error on this thread ("" if none); the pointer stays
 * valid until the thread's next failing call.  Convention of this C ABI (no
 * passage): status codes are returned, never thrown across the boundary, and
 * the text is kept per thread. */
const char *iq4xs_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* IQ4XS_H */
