// launch.hpp -- internal (not exported) kernel launchers.  Arguments reaching
// these functions have already been validated by the C ABI layer; each
// launcher only chooses the grid and enqueues on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pab {

// Sequence addressing shared by the fp32 kernel: sequence s = (outer, inner)
// with outer = s / inner_count, inner = s % inner_count; its first query row
// is q + outer*q_outer + inner*q_inner with consecutive rows q_row apart, and
// likewise for keys/values.
struct SeqLayout {
  int64_t nseq;
  int64_t inner_count;
  int64_t q_outer, q_inner, q_row;
  int64_t kv_outer, kv_inner, kv_row;
  int64_t lq, lk;
};

// Optional fused attention difference: with `prev` set (the previous output
// of the same call, same layout as o) and the launch's block count within
// `capacity`, every block writes sum (o - prev)^2 over its outputs (fp64) to
// partials[block] and *nparts receives the block count; otherwise *nparts
// is 0 and nothing extra is computed.
struct DiffOut {
  const void* prev = nullptr;
  double* partials = nullptr;
  int64_t capacity = 0;
  int* nparts = nullptr;
};

hipError_t launch_spatial_bf16(const void* q, const void* k, const void* v, void* o, int64_t nseq,
                               int S, int D, float scale, const DiffOut& diff,
                               hipStream_t stream);
hipError_t launch_temporal_bf16(const void* q, const void* k, const void* v, void* o, int64_t nbh,
                                int F, int S, int D, float scale, const DiffOut& diff,
                                hipStream_t stream);
// Text K/V rows of one (b, h) are Lrows apart; the first L of them are real
// (L <= Lrows, the rest are padding and take no part).
hipError_t launch_cross_bf16(const void* q, const void* kt, const void* vt, void* o, int64_t nbh,
                             int64_t nq, int L, int Lrows, int D, float scale, const DiffOut& diff,
                             hipStream_t stream);
hipError_t launch_attn_f32(const float* q, const float* k, const float* v, float* o,
                           const SeqLayout& lay, int D, float scale, hipStream_t stream);

// Projections around an attention (bf16): Y = X W^T with W [N, K].  gather:
// X is a head-major attention output [B, H, T, D] (k = h*D + d); scatter: Y
// goes to out[0..N/(H*D)-1] as head-major tensors [B, H, T, D]; otherwise X
// is token-major [M, K] and Y is out[0] token-major [M, N].
hipError_t launch_proj_bf16(const void* x, const void* w, void* const out[3], int64_t M, int N,
                            int K, int T, int H, int D, bool gather, bool scatter,
                            hipStream_t stream);

int mse_num_blocks(int64_t n, int dtype);
// The library's own device scratch for MSE partials (no allocation): its
// address on the current device (looked up on the first call per device)
// and how many partials it holds.
hipError_t mse_scratch(double** out);
int mse_scratch_partials();
hipError_t launch_mse(const void* a, const void* b, int64_t n, int dtype, double* out,
                      double* partials, hipStream_t stream);
// out = (sum of partials[0..nparts), in a fixed order) / n.
hipError_t launch_mse_final(const double* partials, int nparts, int64_t n, double* out,
                            hipStream_t stream);

}  // namespace pab
