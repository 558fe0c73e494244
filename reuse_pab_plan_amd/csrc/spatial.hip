// spatial.hip -- bf16 spatial attention (PAB article, "Implementation",
// second observation: attention among the tokens of one frame), flash style
// on gfx950 MFMA.  Full-3D self-attention is the same kernel with F = 1.
//
// Per sequence (b, h, f) of S tokens: O = softmax(Q K^T * scale) V.
//
// Work split: a 256-thread block owns 256 query rows of one sequence, 64 per
// wave (two 32-row MFMA blocks, so every K and V operand read from LDS feeds
// two MFMAs).  The block sweeps the sequence's keys in tiles of 64 staged
// row-major in LDS (double-buffered; the next tile's loads are in flight in
// registers while the current tile computes).  Each 64-key tile is consumed
// as two 32-key blocks:
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: a lane holds 16 scores of
//     ONE query row, so row statistics need one exchange with the other
//     half-wave;
//   * online softmax with a lazy running max: the max is only raised when a
//     block's max exceeds it by more than 8 (log2 units); p <= 2^8 and
//     rescales become rare after the first blocks;
//   * O^T += V^T P^T: the V^T operand comes straight from the row-major V
//     tile through ds_read_b64_tr_b16 (transposing LDS read), and an implicit
//     all-ones row D of V^T makes the MFMA produce sum_j p_ij (the softmax
//     denominator, over exactly the bf16-rounded p that multiply V).
// Blocks are remapped so that the query tiles of one sequence share an XCD
// (and its L2), where the sequence's K and V stay resident.
#include "device.hpp"
#include "launch.hpp"

namespace pab {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kBN = 64;                  // keys per LDS tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSlack = 8.0f;           // lazy-rescale threshold (log2 units)

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

template <int D>
struct Geo {
  // 32-row query blocks per wave: two share every operand read, unless the
  // head is so wide that two blocks' accumulators no longer fit.
  static constexpr int QB = D <= 88 ? 2 : 1;
  static constexpr int BM = kWaves * 32 * QB;       // query rows per block
  static constexpr int ND = (D + 15) / 16;          // 16-wide d steps of Q K^T
  static constexpr int NB = D / 32 + 1;             // 32-row blocks of O^T (rows 0..D)
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  // Even chunk counts put rows on repeating bank patterns; rotate each row's
  // chunks by ((row % 32) >> 1) so the 32 rows an MFMA operand read touches
  // spread over the banks.  Odd counts (e.g. D = 72) are conflict-free as
  // they are.
  static constexpr bool ROT = (CPR % 2) == 0;
  static constexpr int TILE_CHUNKS = kBN * CPR;      // per tensor per tile
  static constexpr int LOADS = (TILE_CHUNKS + kThreads - 1) / kThreads;
  // A stage holds one K (or V) tile.  Every thread moves LOADS chunks per
  // tile unconditionally; chunks past the tile land in the slack behind it,
  // which also absorbs the d over-read of the last key row when D % 16 == 8.
  static constexpr int TILE_ELEMS = (LOADS * kThreads + CPR) * 8 + 32;
  static constexpr int NBD = D / 32;
  static constexpr int HD = ((D % 32) % 8) / 4;
  static constexpr int RD = ((D % 32) / 8) * 4 + (D % 4);
};

template <int D>
__device__ __forceinline__ int phys_chunk(int row, int ch) {
  using G = Geo<D>;
  if constexpr (G::ROT) {
    int p = ch + ((row & 31) >> 1);
    p %= G::CPR;
    return p;
  } else {
    return ch;
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void spatial_kernel(const bf16* __restrict__ Q,
                                                             const bf16* __restrict__ K,
                                                             const bf16* __restrict__ V,
                                                             bf16* __restrict__ O, int S, int nqt,
                                                             int nblocks, float c) {
  using G = Geo<D>;
  __shared__ __attribute__((aligned(16))) bf16 ks[2][G::TILE_ELEMS];
  __shared__ __attribute__((aligned(16))) bf16 vs[2][G::TILE_ELEMS];

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

  // Slack after each K tile must be finite (read by the d over-read, times 0).
  if (tid < 32) {
    ks[0][kBN * D + tid] = (bf16)0.f;
    ks[1][kBN * D + tid] = (bf16)0.f;
  }

  // This wave's 64 query rows as the B operand (Q^T), resident in registers.
  const int qrow0 = qt * G::BM + wave * 32 * G::QB;
  const bool wave_live = qrow0 < S;
  bf16x8 qreg[G::QB][G::ND];
#pragma unroll
  for (int qb = 0; qb < G::QB; ++qb) {
    const int qrow = qrow0 + qb * 32 + l32;
#pragma unroll
    for (int ds = 0; ds < G::ND; ++ds) {
      const int d0 = ds * 16 + h * 8;
      qreg[qb][ds] = (qrow < S && d0 < D)
                         ? *reinterpret_cast<const bf16x8*>(Qs + (size_t)qrow * D + d0)
                         : zero_bf16x8();
    }
  }

  // Global -> register staging of one tile (K and V, 16-byte chunks).  Rows
  // past S load row S-1 instead: finite values whose scores are masked.
  // Chunk slots past the tile load a valid chunk and land in the stage's
  // slack, so no lane needs a branch.
  // (Named variables, not arrays: an array indexed across the loop would be
  // placed in scratch memory.)
  int go0 = 0, go1 = 0, go2 = 0, go3 = 0, so0 = 0, so1 = 0, so2 = 0, so3 = 0;
  uint4 k0, k1, k2, k3, v0, v1, v2, v3;
  static_assert(G::LOADS <= 4, "staging holds at most 4 chunks per thread");
#define PAB_OFFS(I, go, so)                                                   \
  if constexpr (G::LOADS > I) {                                               \
    const int cidx = tid + I * kThreads;                                      \
    const int row = cidx / G::CPR, ch = cidx % G::CPR;                        \
    go = cidx < G::TILE_CHUNKS ? row * D + ch * 8 : 0;                        \
    so = row * D + phys_chunk<D>(row, ch) * 8;                                \
  }
  PAB_OFFS(0, go0, so0) PAB_OFFS(1, go1, so1) PAB_OFFS(2, go2, so2) PAB_OFFS(3, go3, so3)
#undef PAB_OFFS
#define PAB_FETCH_ONE(I, go, kx, vx)                                          \
  if constexpr (G::LOADS > I) {                                               \
    const int row_ = go / D;                                                  \
    const int shift_ = key0_ + row_ < S ? key0_ * D : (S - 1 - row_) * D;     \
    kx = *reinterpret_cast<const uint4*>(Ks + (size_t)(go + shift_));         \
    vx = *reinterpret_cast<const uint4*>(Vs + (size_t)(go + shift_));         \
  }
#define PAB_FETCH(t)                                                          \
  do {                                                                        \
    const int key0_ = (t) * kBN;                                              \
    PAB_FETCH_ONE(0, go0, k0, v0) PAB_FETCH_ONE(1, go1, k1, v1)               \
    PAB_FETCH_ONE(2, go2, k2, v2) PAB_FETCH_ONE(3, go3, k3, v3)               \
  } while (0)
#define PAB_STASH_ONE(I, so, kx, vx)                                          \
  if constexpr (G::LOADS > I) {                                               \
    *reinterpret_cast<uint4*>(&ks[buf_][so]) = kx;                            \
    *reinterpret_cast<uint4*>(&vs[buf_][so]) = vx;                            \
  }
#define PAB_STASH(buf)                                                        \
  do {                                                                        \
    const int buf_ = (buf);                                                   \
    PAB_STASH_ONE(0, so0, k0, v0) PAB_STASH_ONE(1, so1, k1, v1)               \
    PAB_STASH_ONE(2, so2, k2, v2) PAB_STASH_ONE(3, so3, k3, v3)               \
  } while (0)

  // Per-lane LDS offsets (elements) of the K operand reads, per (kb, ds).
  int koff[2][G::ND];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int ds = 0; ds < G::ND; ++ds) {
      const int row = kb * 32 + l32, ch = ds * 2 + h;
      koff[kb][ds] = row * D + (ch < G::CPR ? phys_chunk<D>(row, ch) * 8 : ch * 8);
    }
  // Per-lane LDS offsets of the transposing V reads, per (t2 of a 32-key
  // block, nb, first/second 4-key group); the key block adds kb*32 rows.
  // Lane j of a 16-lane group addresses row (j/4) and columns 4*(j%4)..+3 of
  // a 4x16 block and receives column j: the V^T operand row d = l32.
  const int g16 = lane >> 4, j16 = lane & 15;
  int voff[2][G::NB][2];
  bool vread[G::NB];
#pragma unroll
  for (int nb = 0; nb < G::NB; ++nb) vread[nb] = nb * 32 < D;
#pragma unroll
  for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int row = t2 * 16 + half * 8 + h * 4 + (j16 >> 2);
        const int col = nb * 32 + (g16 & 1) * 16 + (j16 & 3) * 4;
        const int ch = col / 8;
        voff[t2][nb][half] =
            row * D + (col < D ? phys_chunk<D>(row, ch) * 8 + (col & 7) : 0);
      }

  f32x16 oacc[G::QB][G::NB];
#pragma unroll
  for (int qb = 0; qb < G::QB; ++qb)
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb) oacc[qb][nb] = zero16();
  float mrow[G::QB];
#pragma unroll
  for (int qb = 0; qb < G::QB; ++qb) mrow[qb] = -INFINITY;  // log2 domain (score * c)

  const int nt = (S + kBN - 1) / kBN;
  PAB_FETCH(0);
  PAB_STASH(0);
  __syncthreads();

  for (int t = 0; t < nt; ++t) {
    const int buf = t & 1;
    if (t + 1 < nt) PAB_FETCH(t + 1);
    if (wave_live) {
      const bf16* kb_ = ks[buf];
      const bf16* vb = vs[buf];
      const int key0 = t * kBN;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 sacc[G::QB];
#pragma unroll
        for (int qb = 0; qb < G::QB; ++qb) sacc[qb] = zero16();
#pragma unroll
        for (int ds = 0; ds < G::ND; ++ds) {
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(kb_ + koff[kb][ds]);
#pragma unroll
          for (int qb = 0; qb < G::QB; ++qb) sacc[qb] = mfma32(a, qreg[qb][ds], sacc[qb]);
        }
        if (key0 + kb * 32 + 32 > S) {  // ragged end: keys >= S do not exist
#pragma unroll
          for (int qb = 0; qb < G::QB; ++qb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (key0 + kb * 32 + acc_row(r, h) >= S) sacc[qb][r] = -INFINITY;
        }
        bf16x8 pb[G::QB][2];
#pragma unroll
        for (int qb = 0; qb < G::QB; ++qb) {
          float mx = sacc[qb][0];
#pragma unroll
          for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[qb][r]);
          mx = fmaxf(mx, xor32(mx));
          const float mnew = mx * c;
          if (mnew > mrow[qb] + kSlack) {
            const float alpha = fast_exp2(mrow[qb] - mnew);
#pragma unroll
            for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
              for (int r = 0; r < 16; ++r) oacc[qb][nb][r] *= alpha;
            mrow[qb] = mnew;
          }
          const float negm = -mrow[qb];
#pragma unroll
          for (int t2 = 0; t2 < 2; ++t2) {
            const int r0 = t2 * 8;
            pb[qb][t2] = to_bf16x8(
                fast_exp2(fmaf(sacc[qb][r0 + 0], c, negm)), fast_exp2(fmaf(sacc[qb][r0 + 1], c, negm)),
                fast_exp2(fmaf(sacc[qb][r0 + 2], c, negm)), fast_exp2(fmaf(sacc[qb][r0 + 3], c, negm)),
                fast_exp2(fmaf(sacc[qb][r0 + 4], c, negm)), fast_exp2(fmaf(sacc[qb][r0 + 5], c, negm)),
                fast_exp2(fmaf(sacc[qb][r0 + 6], c, negm)), fast_exp2(fmaf(sacc[qb][r0 + 7], c, negm)));
          }
        }
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
          for (int nb = 0; nb < G::NB; ++nb) {
            bf16x8 a;
            const int d = nb * 32 + l32;
            if (vread[nb]) {
              const bf16* vrow = vb + kb * 32 * D;
              const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  LDS_PTR(i16x4, vrow + voff[t2][nb][0]));
              const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  LDS_PTR(i16x4, vrow + voff[t2][nb][1]));
              a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
              if ((nb + 1) * 32 > D) {  // block holds d >= D: ones row D, zeros above
                const bf16 fill = (bf16)(d == D ? 1.f : 0.f);
                if (d >= D) {
#pragma unroll
                  for (int j = 0; j < 8; ++j) a[j] = fill;
                }
              }
            } else {
              const bf16 fill = (bf16)(d == D ? 1.f : 0.f);
#pragma unroll
              for (int j = 0; j < 8; ++j) a[j] = fill;
            }
#pragma unroll
            for (int qb = 0; qb < G::QB; ++qb) oacc[qb][nb] = mfma32(a, pb[qb][t2], oacc[qb][nb]);
          }
        }
      }
    }
    if (t + 1 < nt) PAB_STASH(buf ^ 1);
    __syncthreads();
  }

#undef PAB_FETCH
#undef PAB_FETCH_ONE
#undef PAB_STASH
#undef PAB_STASH_ONE
  if (wave_live) {
#pragma unroll
    for (int qb = 0; qb < G::QB; ++qb) {
      const float own = oacc[qb][G::NBD][G::RD];
      const float other = xor32(own);
      const float inv = 1.f / ((h == G::HD) ? own : other);
      const int qrow = qrow0 + qb * 32 + l32;
      if (qrow < S) {
        bf16* orow = Os + (size_t)qrow * D;
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int d0 = nb * 32 + g * 8 + h * 4;
            if (d0 < D) {
              const uint2 w =
                  make_uint2(pack_bf16x2(oacc[qb][nb][g * 4 + 0] * inv, oacc[qb][nb][g * 4 + 1] * inv),
                             pack_bf16x2(oacc[qb][nb][g * 4 + 2] * inv, oacc[qb][nb][g * 4 + 3] * inv));
              *reinterpret_cast<uint2*>(orow + d0) = w;
            }
          }
      }
    }
  }
}

template <int D>
hipError_t launch_d(const void* q, const void* k, const void* v, void* o, int64_t nseq, int S,
                    float c, hipStream_t stream) {
  const int nqt = (S + Geo<D>::BM - 1) / Geo<D>::BM;
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
