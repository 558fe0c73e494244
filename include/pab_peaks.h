/*
 * pab_peaks.h -- measurement helpers of libpab.so: microbenchmarks that give
 * the roofline denominators this MI355X actually sustains, reported beside
 * the datasheet peaks (HBM 8 TB/s, dense bf16 MFMA 2516.6 TFLOP/s).  They
 * are not part of the PAB method and no attention call uses them.
 *
 * Conventions as in pab.h (status codes, pab_last_error, validation before
 * any HIP call, caller-owned device memory, enqueue on `stream` without
 * waiting).  The caller times each launch (HIP events on `stream`) and
 * divides the figure below by the time.
 */
#ifndef PAB_PEAKS_H_
#define PAB_PEAKS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Device bytes every `sink` below must hold (16-byte aligned). */
size_t pab_peak_sink_bytes(void);

/*
 * Plain copy dst[0..bytes) = src[0..bytes): 16-byte non-temporal loads and
 * stores over a fixed grid.  Moves 2*bytes through HBM when neither buffer
 * is cache resident (rotate over buffers larger than the 256 MB Infinity
 * Cache to measure HBM).  bytes: positive multiple of 16; src, dst 16-byte
 * aligned and disjoint (else PAB_ERR_INVALID_ARG).
 */
int pab_peak_copy(const void* src, void* dst, size_t bytes, void* stream);

/*
 * Read-only pass over src[0..bytes) (16-byte non-temporal loads, folded
 * into one word per block written to sink).  Reads `bytes`.
 */
int pab_peak_read(const void* src, size_t bytes, void* sink, size_t sink_bytes, void* stream);

/*
 * Independent chains of v_mfma_f32_32x32x16_bf16 on register operands, eight
 * waves per CU.  *flops (host) receives the launch's multiply-add flops
 * (2 per multiply-add); iters >= 1.
 */
int pab_peak_mfma_bf16(int32_t iters, void* sink, size_t sink_bytes, double* flops, void* stream);

/*
 * Independent chains of v_exp_f32 (eight per lane).  *exps (host) receives
 * the number of exponentials of the launch; iters >= 1.
 */
int pab_peak_exp(int32_t iters, void* sink, size_t sink_bytes, double* exps, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAB_PEAKS_H_ */
