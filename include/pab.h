/*
 * pab.h -- C ABI of libpab.so, the MI355X (gfx950) hot path of Pyramid
 * Attention Broadcast (PAB).
 *
 * Sources the calls follow (cited by name throughout):
 *   "PAB article"  -- the English page "The first real-time AI video
 *                     generation technology in history: DiT universal, 10.6
 *                     times faster" (php.cn): sections "pyramid attention
 *                     broadcast", "Implementation", "Parallel"; Figure 1 and
 *                     Figure 2 captions.
 *   "PAB abstract" -- "Real-Time Video Generation with Pyramid Attention
 *                     Broadcast" (Zhao, Jin, Wang, You, 2024), Abstract.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Status   Every function returns 0 (PAB_OK) or a negative pab_status.  A
 *          human-readable reason for the last failure on the calling thread
 *          is returned by pab_last_error().
 * Checks   All argument validation happens before any HIP call, so invalid
 *          arguments never reach the device.  Device pointers must be
 *          non-NULL and 16-byte aligned.
 * Memory   The library allocates no device memory.  Every device buffer
 *          (inputs, outputs, cache slots, workspace, result scalars) belongs
 *          to the caller; host arrays passed in are read or written only for
 *          the duration of the call.
 * Streams  Device work is enqueued on `stream` (a hipStream_t passed as
 *          void*; NULL = the null stream).  Calls return without waiting;
 *          results are valid once the stream reaches that point.
 * Layout   Video tensors are head-major [B, H, F, S, D], contiguous, D
 *          innermost (F latent frames, S tokens per frame, D head dim).  Text
 *          keys/values are [B, H, L, D].
 * Dtypes   PAB_BF16 (bfloat16 in and out, fp32 accumulation; the
 *          performance path, on MFMA) and PAB_F32 (fp32 in, out and
 *          arithmetic; the precision path).  Outputs have the input dtype;
 *          fp32->bf16 rounding is round-to-nearest-even.
 * Scale    softmax_scale == 0 selects 1/sqrt(D).
 * Determinism  The same inputs produce bitwise the same outputs.
 * Inputs   NaN/Inf inputs are a caller error and are not detected.
 */
#ifndef PAB_H_
#define PAB_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pab_status {
  PAB_OK = 0,
  PAB_ERR_INVALID_ARG = -1, /* NULL/misaligned pointer, bad size, aliasing */
  PAB_ERR_UNSUPPORTED = -2, /* valid but outside the supported set (D, F, L, dtype) */
  PAB_ERR_DEVICE = -3,      /* a HIP call failed; pab_last_error has its text */
  PAB_ERR_CAPACITY = -4     /* workspace too small */
} pab_status;

typedef enum pab_dtype { PAB_BF16 = 0, PAB_F32 = 1 } pab_dtype;

/* Attention types of a video DiT block (PAB article, "Implementation",
 * second observation).  Full-3D self-attention is PAB_SPATIAL with F = 1. */
typedef enum pab_attn_kind { PAB_SPATIAL = 0, PAB_TEMPORAL = 1, PAB_CROSS = 2 } pab_attn_kind;

/*
 * pab_plan_schedule -- broadcast schedule (host only, synchronous).
 *
 * PAB article, "Implementation" (the attention difference is U-shaped: the
 * first and last 15% of the steps change a lot, the middle 70% little; in
 * the middle, one step's attention output is broadcast to several following
 * steps, with a wider range for types that change less) and Figure 2
 * caption; PAB abstract ("pyramid" ranges per attention type).
 *
 * Step i (0-based, execution order) is in the stable window iff
 * 100*i >= window_lo_pct*num_steps and 100*i < window_hi_pct*num_steps.
 * For type a with range r = ranges[a] >= 0: outside the window every step
 * recomputes; inside, the first window step recomputes, the next r steps
 * reuse its output, the step after them recomputes, and so on.  Nothing is
 * reused across the window edges.  r = 0 means PAB off.
 *
 * Outputs (caller-owned host arrays, row-major by step):
 *   recompute[num_steps*num_types]   1 = compute attention, 0 = reuse
 *   source_step[num_steps*num_types] step whose output is used (i if it
 *                                    recomputes); may be NULL
 *   recompute_count[num_types]       number of recomputes per type; may be NULL
 * Errors: PAB_ERR_INVALID_ARG for num_steps < 1, num_types < 1 or > 32,
 *   NULL ranges/recompute, ranges[a] < 0, or not 0 <= lo <= hi <= 100.
 * Integer arithmetic only: results are exact.
 */
int pab_plan_schedule(int32_t num_steps, int32_t num_types, const int32_t* ranges,
                      int32_t window_lo_pct, int32_t window_hi_pct, uint8_t* recompute,
                      int32_t* source_step, int32_t* recompute_count);

/*
 * pab_plan_calibrate -- broadcast ranges from a measured attention
 * difference (host only, synchronous).
 *
 * PAB article, "Implementation" (each attention type's range is set by how
 * much its output changes between consecutive steps in the stable middle:
 * the less it changes, the wider its range) and Figure 1 caption (that
 * change is the MSE between the outputs of consecutive steps, as computed by
 * pab_attn_diff_mse); PAB abstract (a pyramid of ranges set by each type's
 * variance).
 *
 * diff[num_blocks*num_steps*num_types] (host, row-major: block, then step,
 * then type): diff[(b*num_steps + i)*num_types + a] is the attention
 * difference of type a between steps i and i-1 in block b of a profiling
 * trajectory that computes every step (PAB off); rows i = 0 are not read.
 * Counted steps: i >= 1 with both i and i-1 in the window (the window rule
 * of pab_plan_schedule).  Every block shares one schedule, so type a's
 * score is the mean of its counted differences over all blocks (fp64,
 * summed block by block, each block's steps in step order).
 * candidate_ranges[a] (>= 0) are the ranges to hand out; they are assigned
 * by rank: the type with the largest score receives the smallest candidate,
 * the next largest the next smallest, and so on (equal scores: the lower
 * type index ranks as larger).  ranges_out[num_types] receives the ranges;
 * score_out[num_types] (may be NULL) the scores.  Values outside the
 * counted steps are never read.
 * Errors: PAB_ERR_INVALID_ARG for num_blocks < 1, num_steps < 1, num_types
 *   < 1 or > 32, NULL diff/candidate_ranges/ranges_out, a negative
 *   candidate, not 0 <= lo <= hi <= 100, a counted difference that is
 *   negative, NaN or infinite, or a window without two consecutive steps.
 */
int pab_plan_calibrate(int32_t num_blocks, int32_t num_steps, int32_t num_types,
                       const double* diff, int32_t window_lo_pct, int32_t window_hi_pct,
                       const int32_t* candidate_ranges, int32_t* ranges_out, double* score_out);

/*
 * pab_attn_spatial -- attention among the S tokens of each frame.
 *
 * PAB article, "Implementation", second observation (spatial attention).
 * For every (b, h, f): O = softmax(Q K^T * scale) V over the S tokens of that
 * frame.  q, k, v, o: [B, H, F, S, D] device buffers of `dtype`.
 * Supported: D a multiple of 8 with 8 <= D <= 128; for bf16 one sequence
 * (S*D elements) must be under 4 GiB (else PAB_ERR_UNSUPPORTED).  o must not
 * overlap q, k or v.  Full-3D self-attention over F' frames of S' tokens is
 * this call with F = 1, S = F'*S'.
 */
int pab_attn_spatial(const void* q, const void* k, const void* v, void* o, int32_t B, int32_t H,
                     int32_t F, int32_t S, int32_t D, int32_t dtype, float softmax_scale,
                     void* stream);

/*
 * pab_attn_temporal -- attention among the F frames at each token position.
 *
 * PAB article, "Implementation", second observation (temporal attention),
 * and "Parallel" (the attention whose sequence-parallel form needs two
 * all-to-all exchanges).  For every (b, h, s): O[b,h,:,s] =
 * softmax(Q[b,h,:,s] K[b,h,:,s]^T * scale) V[b,h,:,s].  Same buffers and
 * layout as pab_attn_spatial.  Supported: D as above and 1 <= F <= 64; for
 * bf16 one (b, h) slab (F*S*D elements) must be under 4 GiB (else
 * PAB_ERR_UNSUPPORTED).
 */
int pab_attn_temporal(const void* q, const void* k, const void* v, void* o, int32_t B, int32_t H,
                      int32_t F, int32_t S, int32_t D, int32_t dtype, float softmax_scale,
                      void* stream);

/*
 * pab_attn_cross -- video tokens attend to text tokens.
 *
 * PAB article, "Implementation", second observation (cross attention links
 * text and video; the most stable type).  For every (b, h): the Nq video
 * queries q[b,h,:,:] ([B, H, Nq, D], i.e. the [B,H,F,S,D] buffer with
 * Nq = F*S) attend to all L text keys/values k_text, v_text ([B, H, L, D]),
 * unmasked.  o has q's shape.  Supported: D as above and 1 <= L <= 128.
 */
int pab_attn_cross(const void* q, const void* k_text, const void* v_text, void* o, int32_t B,
                   int32_t H, int64_t Nq, int32_t L, int32_t D, int32_t dtype,
                   float softmax_scale, void* stream);

/*
 * pab_attn_cross_masked -- cross attention to padded prompts.
 *
 * As pab_attn_cross, but batch entry b has only text_len[b] real text tokens
 * (1 <= text_len[b] <= L): rows text_len[b]..L-1 of k_text[b,h] and
 * v_text[b,h] are padding, take no part in the softmax and are never read.
 * This is how a text encoder's padded prompt reaches cross attention (and
 * how the two halves of a classifier-free-guidance batch, conditional and
 * unconditional, differ).  The pages do not discuss masking; the reading is
 * the usual key-padding mask.  text_len: host array of B int32.
 * Errors: as pab_attn_cross, plus PAB_ERR_INVALID_ARG for a NULL text_len or
 * a length outside [1, L].
 */
int pab_attn_cross_masked(const void* q, const void* k_text, const void* v_text, void* o,
                          int32_t B, int32_t H, int64_t Nq, int32_t L, int32_t D, int32_t dtype,
                          float softmax_scale, const int32_t* text_len, void* stream);

/*
 * pab_proj_in -- input projection of an attention module (bf16).
 *
 * PAB article, "Implementation": a broadcast step reuses the attention
 * module's output, so on such a step this projection is skipped with the
 * attention.  y = x w^T for the F*S tokens of each batch entry, written as
 * n_out head-major tensors: x is token-major [B, F*S, C] with C = H*D (token
 * f*S + s); w is a linear layer's weight [n_out*C, C] (out_features x
 * in_features); output feature j goes to tensor j / C (out0, out1, out2),
 * head (j % C) / D, channel j % D, i.e. out_i is [B, H, F, S, D], the layout
 * of the attention calls.  n_out = 3 gives q, k, v; 2 gives k, v (e.g. of the
 * text tokens: F = 1, S = L); 1 gives q.  fp32 accumulation.
 * Supported: bf16 only (else PAB_ERR_UNSUPPORTED), D as for the attention
 * calls, C a multiple of 32 and <= 16384, every tensor under 4 GiB.
 * Outputs must not overlap each other or the inputs.
 */
int pab_proj_in(const void* x, const void* w, void* out0, void* out1, void* out2, int32_t n_out,
                int32_t B, int32_t F, int32_t S, int32_t H, int32_t D, int32_t dtype,
                void* stream);

/*
 * pab_proj_out -- output projection of an attention module (bf16).
 *
 * Same passage as pab_proj_in.  y = o' w^T where o' is the head-major
 * attention output o [B, H, F, S, D] read token by token (input feature
 * h*D + d) and w is [C, C]; y is token-major [B, F*S, C].  Same support and
 * error rules as pab_proj_in.
 */
int pab_proj_out(const void* o, const void* w, void* y, int32_t B, int32_t F, int32_t S,
                 int32_t H, int32_t D, int32_t dtype, void* stream);

/*
 * pab_mse_workspace_bytes -- device workspace pab_attn_diff_mse needs for
 * n elements (partial sums, one double per reduction block).  The same size
 * also holds the per-block partials of an attention kernel that takes the
 * difference in its output pass (pab_step_dispatch, drift).
 */
size_t pab_mse_workspace_bytes(int64_t n);

/*
 * pab_attn_diff_mse -- attention difference as a mean squared error.
 *
 * PAB article, Figure 1 caption (the difference between the attention
 * outputs of the current and the previous diffusion step, quantified by the
 * MSE).  Writes (1/n) * sum_k (a_k - b_k)^2 as one double to out_dev
 * (device).  a, b: n contiguous elements of `dtype`.  Differences are formed
 * and squared in fp64 and summed in fp64 in a fixed order (deterministic).
 * workspace: device buffer of at least pab_mse_workspace_bytes(n) bytes
 * (else PAB_ERR_CAPACITY).  n >= 1.
 */
int pab_attn_diff_mse(const void* a, const void* b, int64_t n, int32_t dtype, double* out_dev,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * pab_attn_diff_mse_noalloc -- pab_attn_diff_mse for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): the same result, bit for bit (same
 * kernels, same fixed reduction order), with no workspace argument.  The
 * per-block partials go to a device array inside the library (4096 doubles,
 * 32 KiB, enough for the grid of any n; one copy per GPU, held until the
 * process ends).  Its address is looked up on the first call on each device;
 * the call allocates nothing and calls no allocating routine.  Every call on
 * a GPU shares that GPU's array, so calls that overlap on one GPU (e.g. on
 * two streams) race: order them on one stream, or use pab_attn_diff_mse.
 * Nothing in the array needs clearing between calls (pass 1 writes every
 * partial pass 2 reads).
 * Errors: as pab_attn_diff_mse without the workspace checks; PAB_ERR_CAPACITY
 *   if n needed more partials than the array holds (no n in range does);
 *   PAB_ERR_DEVICE if the array's address cannot be obtained.
 */
int pab_attn_diff_mse_noalloc(const void* a, const void* b, int64_t n, int32_t dtype,
                              double* out_dev, void* stream);

/*
 * Step dispatch with the broadcast cache.
 *
 * PAB article, Figure 2 caption: at run time an attention result is
 * broadcast to the next few steps so they skip the attention computation.
 * The cache is caller-owned HBM: per attention type, one or two O-sized
 * slots.  The library keeps no state: which slot holds the live output is a
 * function of the schedule and the step.
 *
 * pab_type_desc -- one attention type of one block:
 *   kind         pab_attn_kind
 *   q, k, v      this step's inputs (device; text k/v for PAB_CROSS); read
 *                only if the type recomputes at this step
 *   slot[0..1]   O-sized device buffers.  The c-th recompute (c = 1, 2, ...)
 *                of this type writes slot[(c-1) % 2]; with slot[1] == NULL
 *                every recompute writes slot[0].
 *   B,H,F,S,D    video shape; L = text tokens (PAB_CROSS only; Nq = F*S)
 *   drift        NULL, or a device array of num_steps doubles: at a
 *                recompute step with an earlier recompute of this type (and
 *                two slots), drift[step] = MSE(new output, previous output),
 *                the attention difference of PAB article Figure 1; other
 *                entries are not written.
 *   text_len     PAB_CROSS only: NULL (all L text tokens real) or a host
 *                array of B real text-token counts, as for
 *                pab_attn_cross_masked.
 *   x ... scratch  the attention module (optional; x = NULL: attention
 *                only).  With x set (bf16 only), a recompute runs the whole
 *                module -- input projection, attention, output projection --
 *                and the slot holds the module output, so a broadcast step
 *                skips all three (PAB article, "Implementation").  q, k, v
 *                are then not read.
 *       x        module input, token-major [B, F*S, C], C = H*D
 *       x_text   PAB_CROSS: text tokens [B, L, C] (key/value projection), or
 *                NULL when scratch[1], scratch[2] already hold the projected
 *                text K/V [B, H, L, D] (text that does not change over the
 *                steps, projected once, e.g. with pab_proj_in); w_kv is then
 *                not read
 *       w_in     [3C, C] q/k/v projection (self types); PAB_CROSS: [C, C]
 *                query projection
 *       w_kv     PAB_CROSS: [2C, C] key/value projection of the text
 *       w_out    [C, C] output projection
 *       scratch  device buffers for q, k, v and the attention output, in the
 *                attention layout ([B,H,F,S,D]; PAB_CROSS k, v: [B,H,L,D]);
 *                contents are overwritten
 *                Slots then hold [B, F*S, C] (the same size as O).
 *
 * pab_step_desc -- the whole block:
 *   num_steps, num_types, recompute  the schedule from pab_plan_schedule
 *                                    (host, [num_steps*num_types])
 *   types        host array of num_types descriptors
 *   dtype, softmax_scale, stream     as for the attention calls
 *   workspace, workspace_bytes       device scratch for the drift MSE (at
 *                least pab_mse_workspace_bytes of the largest O), or NULL/0
 *                when no type has a drift array
 *
 * pab_step_dispatch(desc, step, recomputed_mask, outputs):
 *   for each type a: if recompute[step*num_types + a], launch a's kernel
 *   into its next slot (and the drift MSE if requested); otherwise launch
 *   nothing -- the slot last written holds the source step's output bytes,
 *   reused in place (zero copy, bit-exact).  The drift MSE is the same
 *   quantity pab_attn_diff_mse computes (fp64 differences and sums, a fixed
 *   order per launch shape): bf16 attention kernels take it in their output
 *   pass, reading the previous slot beside each store; fp32 and attention
 *   modules take a separate pass.
 *   recomputed_mask (may be NULL): bit a set iff type a recomputed.
 *   outputs (may be NULL): host array of num_types pointers, set to the slot
 *   holding this step's output of each type.
 *   Errors: as the underlying calls, plus PAB_ERR_INVALID_ARG for a step out
 *   of range, an unknown kind, or num_types > 32.  Validation of every type
 *   happens before the first launch.  A type that recomputes at this step is
 *   checked as the calls it makes; a type that reuses its slot launches
 *   nothing and reads no input, so only its kind, dtype, shape and slots are
 *   checked (its q, k, v or module pointers may be NULL -- e.g. a trajectory
 *   resumed at a broadcast step from saved slots).
 */
typedef struct pab_type_desc {
  int32_t kind;
  const void* q;
  const void* k;
  const void* v;
  void* slot[2];
  int32_t B, H, F, S, D, L;
  double* drift;
  const int32_t* text_len;
  const void* x;
  const void* x_text;
  const void* w_in;
  const void* w_kv;
  const void* w_out;
  void* scratch[4];
} pab_type_desc;

typedef struct pab_step_desc {
  int32_t num_steps;
  int32_t num_types;
  const uint8_t* recompute;
  const pab_type_desc* types;
  int32_t dtype;
  float softmax_scale;
  void* workspace;
  size_t workspace_bytes;
  void* stream;
} pab_step_desc;

int pab_step_dispatch(const pab_step_desc* desc, int32_t step, uint32_t* recomputed_mask,
                      void** outputs);

/* Text of the last error on the calling thread ("" if none).  Valid until
 * the next pab_* call on that thread. */
const char* pab_last_error(void);

/* Library version string (static storage). */
const char* pab_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PAB_H_ */
