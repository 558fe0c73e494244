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
 * HBM streaming microbenchmark: one pass over n_src source and n_dst
 * destination buffers of `bytes` each, in 16-byte vectors: dst_j[i] = XOR
 * of src_0..src_{n_src-1}[i] (of the vector index when n_src = 0); with
 * n_dst = 0 the XOR is folded into one word per block written to sink.
 * Moves (n_src + n_dst) * bytes through HBM when no buffer is cache
 * resident (use buffers much larger than the 256 MB Infinity Cache, or
 * rotate).  `blocks` blocks of 256 threads; `variant` selects the access
 * pattern: bit 0 = non-temporal loads and stores; bits 1-2 = vectors of
 * every stream in flight per thread (0: 4, 1: 8, 2: 16); bit 3 = each block
 * walks one contiguous chunk (else a grid-stride loop over the buffers).
 * The caller picks the best grid and variant for each read/write mix.
 * Errors: PAB_ERR_INVALID_ARG for n_src outside [0, 4], n_dst outside
 *   [0, 2], no stream, NULL/misaligned/overlapping buffers, bytes not a
 *   positive multiple of 16, blocks outside [1, 65536] or an unknown
 *   variant; PAB_ERR_CAPACITY for a sink (n_dst = 0) smaller than
 *   pab_peak_sink_bytes() or than `blocks` words.
 */
int pab_peak_stream(const void* const* src, int32_t n_src, void* const* dst, int32_t n_dst,
                    size_t bytes, int32_t blocks, int32_t variant, void* sink, size_t sink_bytes,
                    void* stream);

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
