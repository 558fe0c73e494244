// spatial.hip -- bf16 spatial attention (PAB article, "Implementation",
// second observation: attention among the tokens of one frame), flash style
// on gfx950 MFMA.  Full-3D self-attention is the same kernel with F = 1.
//
// Per sequence (b, h, f) of S tokens: O = softmax(Q K^T * scale) V.
//
// Work split: a 256-thread block owns 128 query rows of one sequence (32 per
// wave) and sweeps the sequence's keys in tiles of 64, double-buffered in
// LDS (K row-major, V transposed).  Each wave computes the transposed score
// tile S^T = K Q^T with v_mfma_f32_32x32x16_bf16, so every lane holds 16
// scores of ONE query row and the softmax row statistics need a single
// exchange with the other half-wave.  The output is accumulated transposed,
// O^T += V^T P^T, so the running-max rescale is also lane-local.  V^T carries
// an extra all-ones row at index D: the MFMA then produces sum_j p_ij in
// O^T row D, the softmax denominator, with no VALU adds (it sums exactly the
// bf16-rounded p that multiply V).  The running max is only raised when a
// tile's max exceeds it by more than 8 (log2 units), which bounds p by 2^8 and
// skips nearly all rescales after the first tiles.  Blocks are remapped so
// that the query tiles of one sequence share an XCD (and its L2).
#include "device.hpp"
#include "launch.hpp"

namespace pab {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kBN = 64;                  // keys per tile
constexpr int kBM = kWaves * 32;         // query rows per block
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSlack = 8.0f;           // lazy-rescale threshold (log2 units)

template <int D>
struct Geo {
  static constexpr int ND = (D + 15) / 16;          // 16-wide d steps of Q K^T
  static constexpr int NB = D / 32 + 1;             // 32-row blocks of O^T (rows 0..D)
  // K row stride in LDS (elements): an odd number of 16-byte units keeps the
  // 32 rows read by one MFMA operand load on distinct banks.
  static constexpr int KS = ((D / 8) % 2 == 1) ? D : D + 8;
  static constexpr int KROWS = kBN + 1;             // +1 zero row (d over-read when D % 16 == 8)
  static constexpr int VS = kBN + 4;                // V^T row stride: 32 rows -> distinct bank pairs
  static constexpr int VROWS = NB * 32;
  static constexpr int CPR = D / 8;                 // 16-byte chunks per K row
  static constexpr int KCH = (kBN * CPR + kThreads - 1) / kThreads;
  static constexpr int DQ = D / 4;                  // 4-element d groups per V row
  static constexpr int VIT = ((kBN / 4) * DQ + kThreads - 1) / kThreads;
  // Accumulator coordinates of O^T row D (the denominator).
  static constexpr int NBD = D / 32;
  static constexpr int HD = ((D % 32) % 8) / 4;
  static constexpr int RD = ((D % 32) / 8) * 4 + (D % 4);
};

__device__ __forceinline__ uint32_t lo16(uint32_t x) { return x & 0xffffu; }
__device__ __forceinline__ uint32_t hi16(uint32_t x) { return x >> 16; }

template <int D>
__global__ __launch_bounds__(kThreads) void spatial_kernel(const bf16* __restrict__ Q,
                                                          const bf16* __restrict__ K,
                                                          const bf16* __restrict__ V,
                                                          bf16* __restrict__ O, int S, int nqt,
                                                          int nblocks, float c) {
  using G = Geo<D>;
  __shared__ __attribute__((aligned(16))) bf16 ks[2][G::KROWS * G::KS];
  __shared__ __attribute__((aligned(16))) bf16 vt[2][G::VROWS * G::VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, l32 = lane & 31, h = lane >> 5;
  const int logical = xcd_remap(blockIdx.x, nblocks);
  const int64_t seq = logical / nqt;
  const int qt = logical % nqt;
  const size_t base = (size_t)seq * (size_t)S * D;
  const bf16* __restrict__ Qs = Q + base;
  const bf16* __restrict__ Ks = K + base;
  const bf16* __restrict__ Vs = V + base;
  bf16* __restrict__ Os = O + base;

  // Constant LDS rows: V^T row D = 1 (denominator), rows > D = 0, K pad row = 0.
  for (int i = tid; i < (G::VROWS - D) * G::VS; i += kThreads) {
    const int r = D + i / G::VS;
    const bf16 val = (bf16)(r == D ? 1.f : 0.f);
    vt[0][r * G::VS + i % G::VS] = val;
    vt[1][r * G::VS + i % G::VS] = val;
  }
  for (int i = tid; i < G::KS; i += kThreads) {
    ks[0][kBN * G::KS + i] = (bf16)0.f;
    ks[1][kBN * G::KS + i] = (bf16)0.f;
  }

  // This wave's 32 query rows, kept in registers as the B operand (Q^T).
  const int qrow0 = qt * kBM + wave * 32;
  const int qrow = qrow0 + l32;
  const bool wave_live = qrow0 < S;
  bf16x8 qreg[G::ND];
#pragma unroll
  for (int ds = 0; ds < G::ND; ++ds) {
    const int d0 = ds * 16 + h * 8;
    qreg[ds] = (qrow < S && d0 < D) ? *reinterpret_cast<const bf16x8*>(Qs + (size_t)qrow * D + d0)
                                    : zero_bf16x8();
  }

  uint4 kreg[G::KCH];
  uint2 vreg[G::VIT][4];
  auto fetch = [&](int t) {
    const int key0 = t * kBN;
#pragma unroll
    for (int i = 0; i < G::KCH; ++i) {
      const int cidx = tid + i * kThreads;
      if (cidx < kBN * G::CPR) {
        const int row = cidx / G::CPR, ch = cidx % G::CPR;
        const int key = key0 + row;
        kreg[i] = key < S ? *reinterpret_cast<const uint4*>(Ks + (size_t)key * D + ch * 8)
                          : make_uint4(0u, 0u, 0u, 0u);
      }
    }
#pragma unroll
    for (int i = 0; i < G::VIT; ++i) {
      const int it = tid + i * kThreads;
      if (it < (kBN / 4) * G::DQ) {
        const int kq = it / G::DQ, dq = it % G::DQ;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = key0 + kq * 4 + j;
          vreg[i][j] = key < S ? *reinterpret_cast<const uint2*>(Vs + (size_t)key * D + dq * 4)
                               : make_uint2(0u, 0u);
        }
      }
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int i = 0; i < G::KCH; ++i) {
      const int cidx = tid + i * kThreads;
      if (cidx < kBN * G::CPR) {
        const int row = cidx / G::CPR, ch = cidx % G::CPR;
        *reinterpret_cast<uint4*>(&ks[buf][row * G::KS + ch * 8]) = kreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < G::VIT; ++i) {
      const int it = tid + i * kThreads;
      if (it < (kBN / 4) * G::DQ) {
        const int kq = it / G::DQ, dq = it % G::DQ;
        const uint2* r = vreg[i];
        // 4 keys x 4 d block -> four rows of V^T, 4 keys each.
        const uint2 w0 = make_uint2(lo16(r[0].x) | (lo16(r[1].x) << 16), lo16(r[2].x) | (lo16(r[3].x) << 16));
        const uint2 w1 = make_uint2(hi16(r[0].x) | (hi16(r[1].x) << 16), hi16(r[2].x) | (hi16(r[3].x) << 16));
        const uint2 w2 = make_uint2(lo16(r[0].y) | (lo16(r[1].y) << 16), lo16(r[2].y) | (lo16(r[3].y) << 16));
        const uint2 w3 = make_uint2(hi16(r[0].y) | (hi16(r[1].y) << 16), hi16(r[2].y) | (hi16(r[3].y) << 16));
        bf16* dst = &vt[buf][(dq * 4) * G::VS + kq * 4];
        *reinterpret_cast<uint2*>(dst) = w0;
        *reinterpret_cast<uint2*>(dst + G::VS) = w1;
        *reinterpret_cast<uint2*>(dst + 2 * G::VS) = w2;
        *reinterpret_cast<uint2*>(dst + 3 * G::VS) = w3;
      }
    }
  };

  f32x16 oacc[G::NB];
#pragma unroll
  for (int nb = 0; nb < G::NB; ++nb) oacc[nb] = zero16();
  float mrow = -INFINITY;  // running max, log2 domain (score * c)

  const int nt = (S + kBN - 1) / kBN;
  fetch(0);
  stash(0);
  __syncthreads();

  for (int t = 0; t < nt; ++t) {
    const int buf = t & 1;
    if (t + 1 < nt) fetch(t + 1);
    if (wave_live) {
      const bf16* kb_ = ks[buf];
      const bf16* vb = vt[buf];
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = zero16();
#pragma unroll
        for (int ds = 0; ds < G::ND; ++ds) {
          const bf16x8 a =
              *reinterpret_cast<const bf16x8*>(kb_ + (kb * 32 + l32) * G::KS + ds * 16 + h * 8);
          sacc[kb] = mfma32(a, qreg[ds], sacc[kb]);
        }
      }
      const int key0 = t * kBN;
      if (key0 + kBN > S) {  // ragged last tile: keys >= S do not exist
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (key0 + kb * 32 + acc_row(r, h) >= S) sacc[kb][r] = -INFINITY;
      }
      float mx = sacc[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
      mx = fmaxf(mx, xor32(mx));
      const float mnew = mx * c;
      if (mnew > mrow + kSlack) {
        const float alpha = fast_exp2(mrow - mnew);
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[nb][r] *= alpha;
        mrow = mnew;
      }
      const float negm = -mrow;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
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
            const bf16* row = vb + (nb * 32 + l32) * G::VS + kb * 32 + t2 * 16 + h * 4;
            const bf16x4 lo = *reinterpret_cast<const bf16x4*>(row);
            const bf16x4 hi = *reinterpret_cast<const bf16x4*>(row + 8);
            const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            oacc[nb] = mfma32(a, pb, oacc[nb]);
          }
        }
      }
    }
    if (t + 1 < nt) stash(buf ^ 1);
    __syncthreads();
  }

  if (wave_live) {
    const float own = oacc[G::NBD][G::RD];
    const float other = xor32(own);
    const float l = (h == G::HD) ? own : other;
    const float inv = 1.f / l;
    if (qrow < S) {
      bf16* orow = Os + (size_t)qrow * D;
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
  }
}

template <int D>
hipError_t launch_d(const void* q, const void* k, const void* v, void* o, int64_t nseq, int S,
                    float c, hipStream_t stream) {
  const int nqt = (S + kBM - 1) / kBM;
  const int64_t nblocks = nseq * nqt;
  if (nblocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(spatial_kernel<D>, dim3((unsigned)nblocks), dim3(kThreads), 0, stream,
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, S, nqt, (int)nblocks, c);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_spatial_bf16(const void* q, const void* k, const void* v, void* o, int64_t nseq,
                               int S, int D, float scale, hipStream_t stream) {
  const float c = scale * kLog2e;
  switch (D) {
#define PAB_CASE(d) \
  case d:           \
    return launch_d<d>(q, k, v, o, nseq, S, c, stream);
    PAB_CASE(8) PAB_CASE(16) PAB_CASE(24) PAB_CASE(32) PAB_CASE(40) PAB_CASE(48) PAB_CASE(56)
    PAB_CASE(64) PAB_CASE(72) PAB_CASE(80) PAB_CASE(88) PAB_CASE(96) PAB_CASE(104) PAB_CASE(112)
    PAB_CASE(120) PAB_CASE(128)
#undef PAB_CASE
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace pab
