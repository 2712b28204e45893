/*
 * seedlm_bench.h -- measurement-only entry points of libseedlm.  They are not
 * part of the method's interface (seedlm.h): a kernel-variant selector for A/B
 * timing of the batch-1 paths, and the two same-chip baselines a benchmark
 * reports beside the fused decode-GEMV (an fp16 GEMV, and a plain streaming
 * read that measures the device's HBM read ceiling).  Conventions, status codes
 * and dtype codes are those of seedlm.h.
 */
#ifndef SEEDLM_BENCH_H
#define SEEDLM_BENCH_H

#include "seedlm.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * seedlm_gemv_variant -- seedlm_gemv with the kernel chosen by the caller.
 * SEEDLM_VARIANT_AUTO is exactly seedlm_gemv (for the pages' two formats: LUT
 * at batch 1, DIRECT for small batch-1 calls, MFMA for every other fp16-x/
 * fp16-y call; DIRECT otherwise, where fp32 x or fp32 y needs fp32 weights for
 * the 1e-5 bar, and for the other packed formats).  The others:
 *   SEEDLM_VARIANT_LUT     batch 1, both formats: basis bits from GF(2) byte
 *                          tables in LDS, dot with x through activation byte
 *                          tables in LDS
 *   SEEDLM_VARIANT_TABLE   batch 1, 4-bit: as LUT, basis bits from the device's
 *                          2^16-entry table in L2 (built by the first
 *                          seedlm_pack on the device), the alternative the
 *                          LDS tables are measured against
 *   SEEDLM_VARIANT_SIMPLE  any shape: one wave per row, per-lane LFSR stepping,
 *                          fp32 weights
 *   SEEDLM_VARIANT_MFMA    fp16 x and y, any batch: each block decoded once to
 *                          fp16 (weights x 2^10) in MFMA operand registers
 *   SEEDLM_VARIANT_DIRECT  any format, batch and dtypes: exact per-lane decode
 *                          of one block per lane, whole rows per workgroup, one
 *                          launch (what seedlm_gemv runs for the other packed
 *                          formats, for fp32 calls at batch > 1 and for small
 *                          batch-1 calls)
 * Scratch, streams and errors as for seedlm_gemv; SEEDLM_E_UNSUPPORTED when
 * the variant does not take the format, batch or dtypes.
 */
#define SEEDLM_VARIANT_AUTO 0
#define SEEDLM_VARIANT_LUT 1
#define SEEDLM_VARIANT_TABLE 2
#define SEEDLM_VARIANT_SIMPLE 3
#define SEEDLM_VARIANT_MFMA 4
#define SEEDLM_VARIANT_DIRECT 5
SEEDLM_API int seedlm_gemv_variant(seedlm_handle h, const void* x, void* y, int batch,
                                   int x_dtype, int y_dtype, int variant, void* stream);

/*
 * seedlm_bench_time_next_call -- the next gemv call of this host thread
 * (seedlm_gemv, seedlm_gemv_variant, seedlm_gemv_many or _begin) times its main
 * decode-GEMV kernels: `start` is recorded when the first of them starts and
 * `stop` when the last one ends (hipEvent_t values created by the caller, taken
 * by hipExtLaunchKernel from the kernels' own dispatch, so the interval holds
 * no launch gap before the first kernel and no reduction launch after the
 * last).  Read them with hipEventElapsedTime after the call.  NULL, NULL
 * cancels a pending request; a call that fails its argument checks still
 * consumes it, and _end calls leave it pending.  Events recorded inside graph
 * capture are not supported.
 * Errors: SEEDLM_E_INVALID (only one of the two is NULL).
 */
SEEDLM_API int seedlm_bench_time_next_call(void* start_event, void* stop_event);

/*
 * seedlm_fp16_gemv -- measurement baseline, not part of the method: a plain
 * fp16 GEMV y[batch][rows] = W[rows][cols] x[batch][cols] with fp16 W, x, y
 * and fp32 accumulation, used as the speed-up denominator (the pages compare
 * against an FP16 design: atlas.scime.ai "Key results").
 * All pointers are device memory; cols must be a multiple of 8.
 */
SEEDLM_API int seedlm_fp16_gemv(const void* W, const void* x, void* y, int64_t rows,
                                int64_t cols, int batch, void* stream);

/*
 * seedlm_stream_read -- measurement baseline, not part of the method: reads
 * `bytes` of device memory at `buf` once with 16-byte loads (a plain streaming
 * read; on a buffer larger than the last-level cache its rate is the HBM read
 * ceiling a bandwidth-bound kernel can approach on this device) and folds the
 * data into per-workgroup XOR checksums.
 *   buf   device memory, 16-byte aligned; bytes > 0 and a multiple of 16
 *   sink  device uint32[SEEDLM_STREAM_READ_SINK], caller-owned; the launch
 *         writes one checksum per workgroup into its leading entries (at most
 *         all of them) and leaves the rest untouched, so the XOR of a sink that
 *         started at zero equals the XOR of the buffer's 32-bit words
 * Asynchronous on `stream`.  Errors: SEEDLM_E_INVALID (null pointer, size or
 * alignment), SEEDLM_E_DEVICE (launch failure).
 */
#define SEEDLM_STREAM_READ_SINK 8192
SEEDLM_API int seedlm_stream_read(const void* buf, int64_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SEEDLM_BENCH_H */
