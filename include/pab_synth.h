/*
 * pab_synth.h -- seeded synthetic inputs on the device: the workload
 * generator of libpab.so.  It draws the Q, K, V tensors (and projection
 * weights and module inputs) that stand in for a video DiT's features; it
 * is not part of the PAB method and no attention call uses it.
 *
 * Generator: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC'11), a counter-based generator: block i
 * of stream `key` is Philox4x32-10 applied to the 128-bit counter
 * (lo32(i), hi32(i), 0, 0) under the 64-bit key (lo32(key), hi32(key)), four
 * 32-bit words per block.  Standard normals come from the Box-Muller
 * transform (Box and Muller, 1958) of word pairs: for words (x, y),
 * u = ((x >> 9) + 1/2) 2^-23, w = ((y >> 9) + 1/2) 2^-23 (both in (0, 1)),
 * r = sqrt(-2 ln u), and the two normals are r cos(2 pi w), r sin(2 pi w).
 * Element e of a stream takes block e / 4: words (0, 1) give elements
 * 4i (cos) and 4i+1 (sin), words (2, 3) give 4i+2 and 4i+3.
 *
 * The 32-bit words are exact (a CPU implementation of the same definition
 * reproduces them bit for bit); the normals are computed in fp32 with the
 * device's log2, sqrt, sin and cos instructions, so they agree with an
 * exact evaluation to a few fp32 ulps, not bitwise.
 *
 * Conventions as in pab.h (status codes, pab_last_error, validation before
 * any HIP call, caller-owned device memory, enqueue on `stream` without
 * waiting).
 */
#ifndef PAB_SYNTH_H_
#define PAB_SYNTH_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Raw generator output: out[4*j + w] = word w of block (block0 + j) of
 * stream `key`, for j in [0, nblocks).  out: device array of 4*nblocks
 * uint32, 16-byte aligned.  Errors: PAB_ERR_INVALID_ARG for a NULL or
 * misaligned out, nblocks < 1, or block0 + nblocks past 2^62.
 */
int pab_synth_philox(uint32_t* out, int64_t nblocks, uint64_t key, uint64_t block0, void* stream);

/*
 * out[e] = round(scale_a * N_a[e] + scale_b * N_b[e]) for e in [0, n), where
 * N_k[e] is element e of the standard-normal stream `key_k` (above), the
 * sum is formed in fp32 as fma(scale_b, N_b, scale_a * N_a), and round is
 * to the output dtype (PAB_BF16: nearest even; PAB_F32: exact).  With
 * scale_b == 0 stream b is not drawn (out = round(scale_a * N_a)).
 * out: device buffer of n elements of `dtype`, 16-byte aligned.
 * Errors: PAB_ERR_INVALID_ARG for a NULL or misaligned out, n < 1 or past
 * 2^62, or a non-finite scale; PAB_ERR_UNSUPPORTED for another dtype.
 */
int pab_synth_normal(void* out, int64_t n, int32_t dtype, uint64_t key_a, float scale_a,
                     uint64_t key_b, float scale_b, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAB_SYNTH_H_ */
