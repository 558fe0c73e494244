// attn_f32.hip -- fp32 attention for all three attention types (the
// precision path: fp32 in, fp32 arithmetic, fp32 out).
//
// O = softmax(Q K^T * scale) V per sequence; the sequences of the spatial,
// temporal and cross types differ only in addressing (SeqLayout).  One
// thread owns one query row; keys/values stream through LDS in 64-row tiles
// and the softmax is accumulated online (running max and sum, rescaled when
// the max grows).  bf16 is the MFMA performance path; this kernel serves
// dtype PAB_F32 only.
#include "device.hpp"
#include "launch.hpp"

namespace pab {

namespace {

constexpr int kRows = 64;   // queries per block (one wave)
constexpr int kTile = 64;   // keys per LDS tile
constexpr float kLog2e = 1.4426950408889634f;

template <int DMAX>
__global__ __launch_bounds__(kRows) void attn_f32_kernel(const float* __restrict__ Q,
                                                        const float* __restrict__ K,
                                                        const float* __restrict__ V,
                                                        float* __restrict__ O, SeqLayout lay,
                                                        int64_t row_blocks, int D, float c) {
  __shared__ float ks[kTile][DMAX + 1];
  __shared__ float vs[kTile][DMAX + 1];

  const int64_t seq = (int64_t)blockIdx.x / row_blocks;
  const int64_t rb = (int64_t)blockIdx.x % row_blocks;
  const int64_t outer = seq / lay.inner_count;
  const int64_t inner = seq % lay.inner_count;
  const float* q = Q + outer * lay.q_outer + inner * lay.q_inner;
  float* o = O + outer * lay.q_outer + inner * lay.q_inner;
  const float* k = K + outer * lay.kv_outer + inner * lay.kv_inner;
  const float* v = V + outer * lay.kv_outer + inner * lay.kv_inner;

  const int64_t row = rb * kRows + threadIdx.x;
  const bool live = row < lay.lq;

  float qr[DMAX], acc[DMAX];
#pragma unroll
  for (int d = 0; d < DMAX; ++d) {
    qr[d] = (live && d < D) ? q[row * lay.q_row + d] : 0.f;
    acc[d] = 0.f;
  }
  float m = -INFINITY;  // running max of scaled (log2-domain) scores
  float l = 0.f;        // running sum of exp2(score - m)

  // Columns D..DMAX-1 of the tiles are never loaded but take part in the
  // unrolled products (against zero q and unused accumulators): zero them
  // once, so stale LDS contents (possibly NaN bit patterns) cannot leak in.
  // The first barrier of the key loop orders these stores before any read.
  for (int idx = threadIdx.x; idx < kTile * (DMAX - D); idx += kRows) {
    const int r = idx / (DMAX - D), d = D + idx % (DMAX - D);
    ks[r][d] = 0.f;
    vs[r][d] = 0.f;
  }

  for (int64_t k0 = 0; k0 < lay.lk; k0 += kTile) {
    __syncthreads();
    for (int idx = threadIdx.x; idx < kTile * D; idx += kRows) {
      const int r = idx / D, d = idx % D;
      const int64_t key = k0 + r;
      ks[r][d] = key < lay.lk ? k[key * lay.kv_row + d] : 0.f;
      vs[r][d] = key < lay.lk ? v[key * lay.kv_row + d] : 0.f;
    }
    __syncthreads();
    const int nk = (int)((lay.lk - k0) < kTile ? (lay.lk - k0) : kTile);
    for (int j = 0; j < nk; ++j) {
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < DMAX; ++d) s = fmaf(qr[d], ks[j][d], s);
      s *= c;
      if (s > m) {
        const float alpha = fast_exp2(m - s);
        l *= alpha;
#pragma unroll
        for (int d = 0; d < DMAX; ++d) acc[d] *= alpha;
        m = s;
      }
      const float p = fast_exp2(s - m);
      l += p;
#pragma unroll
      for (int d = 0; d < DMAX; ++d) acc[d] = fmaf(p, vs[j][d], acc[d]);
    }
  }
  if (live) {
    const float inv = 1.f / l;
#pragma unroll
    for (int d = 0; d < DMAX; ++d)
      if (d < D) o[row * lay.q_row + d] = acc[d] * inv;
  }
}

}  // namespace

hipError_t launch_attn_f32(const float* q, const float* k, const float* v, float* o,
                           const SeqLayout& lay, int D, float scale, hipStream_t stream) {
  const float c = scale * kLog2e;
  const int64_t row_blocks = (lay.lq + kRows - 1) / kRows;
  const int64_t blocks = row_blocks * lay.nseq;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)blocks);
  if (D <= 64) {
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(kRows), 0, stream, q, k, v, o, lay, row_blocks, D, c);
  } else {
    hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(kRows), 0, stream, q, k, v, o, lay, row_blocks, D, c);
  }
  return hipGetLastError();
}

}  // namespace pab
