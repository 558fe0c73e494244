// cross.hip -- bf16 cross attention: video queries attend to text keys/values
// (PAB article, "Implementation", second observation: cross attention ties
// the text to the video and changes least between steps).
//
// Per (b, h): the Nq = F*S video queries against L <= 128 text keys.  The
// text K (row-major) and V (transposed, plus an all-ones row at index D that
// makes the MFMA emit the softmax denominator) are loaded into LDS once per
// block and stay resident; query tiles of 32 rows stream from HBM through
// each wave, so Q is read once and O written once: the kernel is HBM-bound.
// Scores are formed transposed (S^T = K Q^T, v_mfma_f32_32x32x16_bf16) so
// one lane holds one query row's scores; with at most 128 keys the whole row
// fits in registers and the softmax needs no running rescale.  The next
// tile's Q is loaded while the current tile computes.
#include "device.hpp"
#include "launch.hpp"

namespace pab {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kLMax = 128;
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct Geo {
  static constexpr int ND = (D + 15) / 16;
  static constexpr int NB = D / 32 + 1;
  static constexpr int KS = ((D / 8) % 2 == 1) ? D : D + 8;
  static constexpr int KROWS = kLMax + 1;
  static constexpr int VS = kLMax + 4;
  static constexpr int VROWS = NB * 32;
  static constexpr int CPR = D / 8;
  static constexpr int NBD = D / 32;
  static constexpr int HD = ((D % 32) % 8) / 4;
  static constexpr int RD = ((D % 32) / 8) * 4 + (D % 4);
};

template <int D>
__device__ __forceinline__ void load_q(bf16x8 (&qr)[Geo<D>::ND], const bf16* __restrict__ Qh,
                                       int64_t tile, int64_t nq, int l32, int h) {
  const int64_t row = tile * 32 + l32;
#pragma unroll
  for (int ds = 0; ds < Geo<D>::ND; ++ds) {
    const int d0 = ds * 16 + h * 8;
    qr[ds] = (row < nq && d0 < D) ? *reinterpret_cast<const bf16x8*>(Qh + row * D + d0) : zero_bf16x8();
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void cross_kernel(const bf16* __restrict__ Q,
                                                        const bf16* __restrict__ Kt,
                                                        const bf16* __restrict__ Vt,
                                                        bf16* __restrict__ O, int64_t nq, int L,
                                                        int tiles_per_block, int blocks_per_bh,
                                                        int nblocks, float c) {
  using G = Geo<D>;
  __shared__ __attribute__((aligned(16))) bf16 ks[G::KROWS * G::KS];
  __shared__ __attribute__((aligned(16))) bf16 vt[G::VROWS * G::VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, l32 = lane & 31, h = lane >> 5;
  const int logical = xcd_remap(blockIdx.x, nblocks);
  const int64_t bh = logical / blocks_per_bh;
  const int chunk = logical % blocks_per_bh;
  const bf16* __restrict__ Qh = Q + bh * nq * D;
  bf16* __restrict__ Oh = O + bh * nq * D;
  const bf16* __restrict__ Kh = Kt + bh * (int64_t)L * D;
  const bf16* __restrict__ Vh = Vt + bh * (int64_t)L * D;

  const int64_t ntiles = (nq + 31) / 32;
  const int64_t t_begin = (int64_t)chunk * tiles_per_block;
  int64_t t_end = t_begin + tiles_per_block;
  if (t_end > ntiles) t_end = ntiles;

  // Text K -> LDS rows (rows >= L and the pad row are zero).
  for (int i = tid; i < G::KROWS * G::CPR; i += kThreads) {
    const int row = i / G::CPR, ch = i % G::CPR;
    uint4 val = make_uint4(0u, 0u, 0u, 0u);
    if (row < L) val = *reinterpret_cast<const uint4*>(Kh + (int64_t)row * D + ch * 8);
    *reinterpret_cast<uint4*>(&ks[row * G::KS + ch * 8]) = val;
  }
  // Text V -> V^T in LDS; row D = 1 (denominator), rows > D and keys >= L = 0.
  for (int i = tid; i < G::VROWS * kLMax; i += kThreads) {
    const int d = i / kLMax, key = i % kLMax;
    float val = 0.f;
    if (d < D) {
      if (key < L) val = (float)Vh[(int64_t)key * D + d];
    } else if (d == D) {
      val = 1.f;
    }
    vt[d * G::VS + key] = (bf16)val;
  }
  __syncthreads();

  const int nkb = (L + 31) / 32;
  bf16x8 qcur[G::ND], qnext[G::ND];
  int64_t tile = t_begin + wave;
  if (tile < t_end) load_q<D>(qcur, Qh, tile, nq, l32, h);

  for (; tile < t_end; tile += kWaves) {
    if (tile + kWaves < t_end) load_q<D>(qnext, Qh, tile + kWaves, nq, l32, h);

    f32x16 sacc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sacc[kb] = zero16();
      if (kb < nkb) {
#pragma unroll
        for (int ds = 0; ds < G::ND; ++ds) {
          const bf16x8 a =
              *reinterpret_cast<const bf16x8*>(&ks[(kb * 32 + l32) * G::KS + ds * 16 + h * 8]);
          sacc[kb] = mfma32(a, qcur[ds], sacc[kb]);
        }
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        if (kb * 32 + acc_row(r, h) >= L) sacc[kb][r] = -INFINITY;
        mx = fmaxf(mx, sacc[kb][r]);
      }
    mx = fmaxf(mx, xor32(mx));
    const float negm = -mx * c;

    f32x16 oacc[G::NB];
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb) oacc[nb] = zero16();
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      if (kb < nkb) {
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
          const int r0 = t2 * 8;
          const bf16x8 pb = to_bf16x8(
              fast_exp2(fmaf(sacc[kb][r0 + 0], c, negm)), fast_exp2(fmaf(sacc[kb][r0 + 1], c, negm)),
              fast_exp2(fmaf(sacc[kb][r0 + 2], c, negm)), fast_exp2(fmaf(sacc[kb][r0 + 3], c, negm)),
              fast_exp2(fmaf(sacc[kb][r0 + 4], c, negm)), fast_exp2(fmaf(sacc[kb][r0 + 5], c, negm)),
              fast_exp2(fmaf(sacc[kb][r0 + 6], c, negm)), fast_exp2(fmaf(sacc[kb][r0 + 7], c, negm)));
#pragma unroll
          for (int nb = 0; nb < G::NB; ++nb) {
            const bf16* row = &vt[(nb * 32 + l32) * G::VS + kb * 32 + t2 * 16 + h * 4];
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row);
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + 8);
            const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            oacc[nb] = mfma32(a, pb, oacc[nb]);
          }
        }
      }
    }

    const float own = oacc[G::NBD][G::RD];
    const float other = xor32(own);
    const float inv = 1.f / ((h == G::HD) ? own : other);
    const int64_t row = tile * 32 + l32;
    if (row < nq) {
      bf16* orow = Oh + row * D;
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = nb * 32 + g * 8 + h * 4;
          if (d0 < D) {
            const uint2 w = make_uint2(pack_bf16x2(oacc[nb][g * 4 + 0] * inv, oacc[nb][g * 4 + 1] * inv),
                                       pack_bf16x2(oacc[nb][g * 4 + 2] * inv, oacc[nb][g * 4 + 3] * inv));
            *reinterpret_cast<uint2*>(orow + d0) = w;
          }
        }
    }
#pragma unroll
    for (int ds = 0; ds < G::ND; ++ds) qcur[ds] = qnext[ds];
  }
}

template <int D>
hipError_t launch_d(const void* q, const void* kt, const void* vt, void* o, int64_t nbh, int64_t nq,
                    int L, float c, hipStream_t stream) {
  // Size the grid to whole waves of resident blocks (3 per CU on 256 CUs),
  // with at most 48 query tiles per block.
  const int64_t ntiles = (nq + 31) / 32;
  const int64_t total = ntiles * nbh;
  const int64_t wave_blocks = 768;
  int64_t target = ((total + wave_blocks * 48 - 1) / (wave_blocks * 48)) * wave_blocks;
  int64_t blocks_per_bh = (target + nbh - 1) / nbh;
  if (blocks_per_bh > ntiles) blocks_per_bh = ntiles;
  if (blocks_per_bh < 1) blocks_per_bh = 1;
  const int64_t tiles_per_block = (ntiles + blocks_per_bh - 1) / blocks_per_bh;
  blocks_per_bh = (ntiles + tiles_per_block - 1) / tiles_per_block;
  const int64_t nblocks = blocks_per_bh * nbh;
  if (nblocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(cross_kernel<D>, dim3((unsigned)nblocks), dim3(kThreads), 0, stream,
                     (const bf16*)q, (const bf16*)kt, (const bf16*)vt, (bf16*)o, nq, L,
                     (int)tiles_per_block, (int)blocks_per_bh, (int)nblocks, c);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_cross_bf16(const void* q, const void* kt, const void* vt, void* o, int64_t nbh,
                             int64_t nq, int L, int D, float scale, hipStream_t stream) {
  const float c = scale * kLog2e;
  switch (D) {
#define PAB_CASE(d) \
  case d:           \
    return launch_d<d>(q, kt, vt, o, nbh, nq, L, c, stream);
    PAB_CASE(8) PAB_CASE(16) PAB_CASE(24) PAB_CASE(32) PAB_CASE(40) PAB_CASE(48) PAB_CASE(56)
    PAB_CASE(64) PAB_CASE(72) PAB_CASE(80) PAB_CASE(88) PAB_CASE(96) PAB_CASE(104) PAB_CASE(112)
    PAB_CASE(120) PAB_CASE(128)
#undef PAB_CASE
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace pab
