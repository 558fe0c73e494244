// attn_f32.hip -- fp32 attention for all three attention types (the
// precision path: fp32 in, fp32 arithmetic, fp32 out).
//
// O = softmax(Q K^T * scale) V per sequence; the sequences of the spatial,
// temporal and cross types differ only in addressing (SeqLayout).
//
// A 256-thread block owns 16 query rows of one sequence, four per wave.
// Keys and values stream through LDS in 64-row tiles.  For each of its rows a
// wave works across the tile: lane j forms the score of key j (the query row
// is read from LDS as a broadcast, the key row from a padded tile whose rows
// fall on distinct banks), the tile's maximum and sum come from cross-lane
// reductions, and then lane d accumulates output column d (and d + 64) over
// the tile's keys, each p_j taken from lane j with v_readlane.  The softmax
// is accumulated online over the tiles (running max and sum, rescaled when
// the max grows).  Short sequences thus spread over many waves instead of one
// thread per row walking every key alone.  bf16 is the MFMA performance
// path; this kernel serves dtype PAB_F32 only.
#include "device.hpp"
#include "launch.hpp"

namespace pab {

namespace {

constexpr int kWavesF = 4;
constexpr int kThreadsF = kWavesF * kWave;
constexpr int kRowsPerWave = 4;
constexpr int kRowsF = kWavesF * kRowsPerWave;  // query rows per block
constexpr int kTile = 64;                        // keys per LDS tile: one per lane
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

template <int DMAX>
__global__ __launch_bounds__(kThreadsF) void attn_f32_kernel(const float* __restrict__ Q,
                                                            const float* __restrict__ K,
                                                            const float* __restrict__ V,
                                                            float* __restrict__ O, SeqLayout lay,
                                                            int64_t row_blocks, int D, float c) {
  constexpr int NE = DMAX / kWave;  // output columns per lane
  // Key rows padded by one word: lane j reads row j, so a column access of
  // the 64 lanes touches 64 distinct banks.
  __shared__ float ks[kTile][DMAX + 1];
  __shared__ float vs[kTile][DMAX];
  __shared__ __attribute__((aligned(16))) float qs[kRowsF][DMAX];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t seq = (int64_t)blockIdx.x / row_blocks;
  const int64_t rb = (int64_t)blockIdx.x % row_blocks;
  const int64_t outer = seq / lay.inner_count;
  const int64_t inner = seq % lay.inner_count;
  const float* q = Q + outer * lay.q_outer + inner * lay.q_inner;
  float* o = O + outer * lay.q_outer + inner * lay.q_inner;
  const float* k = K + outer * lay.kv_outer + inner * lay.kv_inner;
  const float* v = V + outer * lay.kv_outer + inner * lay.kv_inner;
  const int64_t row0 = rb * kRowsF;

  // The block's query rows; rows past lq and columns past D are zero.  Only
  // columns below D of the key and value tiles are ever read.
  for (int idx = tid; idx < kRowsF * DMAX; idx += kThreadsF) {
    const int r = idx / DMAX, d = idx % DMAX;
    const int64_t row = row0 + r;
    qs[r][d] = (row < lay.lq && d < D) ? q[row * lay.q_row + d] : 0.f;
  }

  float m[kRowsPerWave], l[kRowsPerWave], acc[kRowsPerWave][NE];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    m[i] = -INFINITY;  // running max of scaled (log2-domain) scores
    l[i] = 0.f;        // running sum of exp2(score - m)
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[i][e] = 0.f;
  }

  for (int64_t k0 = 0; k0 < lay.lk; k0 += kTile) {
    __syncthreads();  // the previous tile is no longer read (and qs is stored)
    for (int idx = tid; idx < kTile * D; idx += kThreadsF) {
      const int r = idx / D, d = idx % D;
      const int64_t key = k0 + r;
      // Rows past the last key are zero: their p is 0 and 0 * V stays 0.
      ks[r][d] = key < lay.lk ? k[key * lay.kv_row + d] : 0.f;
      vs[r][d] = key < lay.lk ? v[key * lay.kv_row + d] : 0.f;
    }
    __syncthreads();
    const int nk = (int)((lay.lk - k0) < kTile ? (lay.lk - k0) : kTile);
#pragma unroll
    for (int i = 0; i < kRowsPerWave; ++i) {
      const int r = wave * kRowsPerWave + i;
      if (row0 + r >= lay.lq) break;  // wave-uniform: rows past lq
      // Score of key `lane` (D is a multiple of 8).
      float s = 0.f;
      for (int d = 0; d < D; d += 8) {
        const float4 qa = *reinterpret_cast<const float4*>(&qs[r][d]);
        const float4 qb = *reinterpret_cast<const float4*>(&qs[r][d + 4]);
        s = fmaf(qa.x, ks[lane][d + 0], s);
        s = fmaf(qa.y, ks[lane][d + 1], s);
        s = fmaf(qa.z, ks[lane][d + 2], s);
        s = fmaf(qa.w, ks[lane][d + 3], s);
        s = fmaf(qb.x, ks[lane][d + 4], s);
        s = fmaf(qb.y, ks[lane][d + 5], s);
        s = fmaf(qb.z, ks[lane][d + 6], s);
        s = fmaf(qb.w, ks[lane][d + 7], s);
      }
      s = lane < nk ? s * c : -INFINITY;
      // Online softmax: nk >= 1, so the tile's max is finite and so is mn;
      // exp2(-inf) = 0 covers both the first tile's rescale and absent keys.
      const float mn = fmaxf(m[i], wave_max(s));
      const float alpha = fast_exp2(m[i] - mn);
      const float p = fast_exp2(s - mn);
      l[i] = l[i] * alpha + wave_sum(p);
      m[i] = mn;
#pragma unroll
      for (int e = 0; e < NE; ++e) acc[i][e] *= alpha;
      // Output column lane + 64 e over the tile's keys.
      const int pbits = __builtin_bit_cast(int, p);
#pragma unroll 16
      for (int j = 0; j < kTile; ++j) {
        const float pj = __builtin_bit_cast(float, __builtin_amdgcn_readlane(pbits, j));
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[i][e] = fmaf(pj, vs[j][lane + kWave * e], acc[i][e]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int64_t row = row0 + wave * kRowsPerWave + i;
    if (row < lay.lq) {
      const float inv = 1.f / l[i];
#pragma unroll
      for (int e = 0; e < NE; ++e) {
        const int d = lane + kWave * e;
        if (d < D) o[row * lay.q_row + d] = acc[i][e] * inv;
      }
    }
  }
}

}  // namespace

hipError_t launch_attn_f32(const float* q, const float* k, const float* v, float* o,
                           const SeqLayout& lay, int D, float scale, hipStream_t stream) {
  const float c = scale * kLog2e;
  const int64_t row_blocks = (lay.lq + kRowsF - 1) / kRowsF;
  const int64_t blocks = row_blocks * lay.nseq;
  if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  dim3 grid((unsigned)blocks);
  if (D <= 64) {
    hipLaunchKernelGGL(attn_f32_kernel<64>, grid, dim3(kThreadsF), 0, stream, q, k, v, o, lay,
                       row_blocks, D, c);
  } else {
    hipLaunchKernelGGL(attn_f32_kernel<128>, grid, dim3(kThreadsF), 0, stream, q, k, v, o, lay,
                       row_blocks, D, c);
  }
  return hipGetLastError();
}

}  // namespace pab
