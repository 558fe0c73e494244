// spatial.hip -- bf16 spatial attention (PAB article, "Implementation",
// second observation: attention among the tokens of one frame), flash style
// on gfx950 MFMA.  Full-3D self-attention is the same kernel with F = 1.
//
// Per sequence (b, h, f) of S tokens: O = softmax(Q K^T * scale) V.
//
// Work split: a 256-thread block owns up to 256 query rows of one sequence,
// 64 per wave (two 32-row MFMA blocks, so every K and V operand read from LDS
// feeds two MFMAs; one block per wave for heads wider than 88).  Keys arrive
// in 64-row tiles through a 3-stage LDS ring filled by direct global->LDS
// loads (global_load_lds_dwordx4) issued two tiles ahead, so the next tiles
// stream in while the current one computes and no registers are spent on
// staging.  Each tile is consumed as two 32-key blocks:
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: a lane holds 16 scores of
//     ONE query row, so row statistics need one exchange with the other
//     half-wave;
//   * online softmax with a lazy running max: the max is only raised when a
//     block's max exceeds it by more than 8 (log2 units); p <= 2^8 and
//     rescales become rare after the first blocks;
//   * O^T += V^T P^T: the V^T operand comes straight from the row-major V
//     tile through ds_read_b64_tr_b16 (transposing LDS read).  Operand row D
//     (a padding row of the last 32-row block) is set to ones, so O^T row D
//     accumulates sum_j p_ij -- the softmax denominator, over exactly the
//     bf16-rounded p that multiply V -- on the MFMA.
// Blocks are remapped so that the query tiles of one sequence share an XCD
// (and its L2), where the sequence's K and V stay resident.
#include "device.hpp"
#include "launch.hpp"

namespace pab {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kBN = 64;                  // keys per LDS tile
constexpr int kStages = 3;               // LDS ring depth (loads run two tiles ahead)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kSlack = 8.0f;           // lazy-rescale threshold (log2 units)

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// Smallest row stride (elements, multiple of 8, >= min_elems) whose first four
// rows start on disjoint 8-bank spans: the transposing read of one 16-lane
// group touches 32 bytes of four consecutive rows.
constexpr int tr_stride(int min_elems) {
  for (int s = (min_elems + 7) / 8 * 8;; s += 8) {
    const int w = s / 2;  // 4-byte words per row
    bool ok = true;
    for (int a = 0; a < 4 && ok; ++a)
      for (int b = a + 1; b < 4 && ok; ++b) {
        const int d = (w * (b - a)) % 64;
        if (d < 8 || d > 56) ok = false;
      }
    if (ok) return s;
  }
}

template <int D>
struct Geo {
  // 32-row query blocks per wave: two share every operand read, unless the
  // head is so wide that two blocks' accumulators no longer fit.
  static constexpr int QB = D <= 88 ? 2 : 1;
  static constexpr int BM = kWaves * 32 * QB;       // query rows per block
  static constexpr int ND = (D + 15) / 16;          // 16-wide d steps of Q K^T
  static constexpr int NB = D / 32 + 1;             // 32-row blocks of O^T (rows 0..D)
  static constexpr int DCH = D / 8;                 // 16-byte chunks of data per row
  // K rows: an odd number of 16-byte chunks keeps the 32 rows of one MFMA
  // operand read on distinct banks.
  static constexpr int KS = (DCH % 2) ? D : D + 8;
  static constexpr int KCH = KS / 8;
  // V rows: data padded to a stride that keeps the transposing reads
  // conflict-free.
  static constexpr int VS = tr_stride(D);
  static constexpr int VCH = VS / 8;
  // Direct loads per thread per tile, rounded up; surplus slots land in the
  // stage's tail (which also absorbs the operand over-reads past row 63).
  static constexpr int KDMA = (kBN * KCH + kThreads - 1) / kThreads;
  static constexpr int VDMA = (kBN * VCH + kThreads - 1) / kThreads;
  static constexpr int KSTAGE = KDMA * kThreads * 8;  // elements
  static constexpr int VSTAGE = VDMA * kThreads * 8;
  // The last 32-row O^T block holds row D (the denominator); with no data in
  // it (D % 32 == 0) its V^T operand is a constant and is not read.
  static constexpr bool LAST_READ = (NB - 1) * 32 < D;
  // Transposing reads of V past the last data column (operand rows > D, whose
  // products are discarded) may run past the stage's slots into this slack.
  static constexpr int VSLACK = 64;
  static constexpr int STAGE = KSTAGE + VSTAGE + VSLACK;
  // K over-reads (d >= D, multiplied by Q's zero padding) must hit finite
  // data: they stay inside the DMA'd slots, surplus slots included.
  static_assert(kBN * KS + 8 <= KSTAGE, "K over-read must stay in the DMA'd slots");
  static_assert((kBN - 1) * VS + (LAST_READ ? NB : NB - 1) * 32 <= VSTAGE + VSLACK,
                "V over-read must stay in the stage");
  static_assert(kStages * STAGE * 2 <= 160 * 1024, "LDS ring too large");
  static_assert(KDMA + VDMA < 32, "vmcnt budget");
  static constexpr int NBD = D / 32;
  static constexpr int HD = ((D % 32) % 8) / 4;
  static constexpr int RD = ((D % 32) / 8) * 4 + (D % 4);
};

// One 16-byte direct global->LDS load per lane: lane l of the wave reads
// global bytes [gbase + voff, +16) and writes LDS bytes [lds + 16*l, +16).
// `gbase` and `lds` must be wave-uniform.  Issued from inline assembly so that
// the wait for it (s_waitcnt vmcnt) is placed by hand: the compiler would
// otherwise wait for every outstanding direct load before each LDS read,
// serializing the ring.  The instruction has no result register.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(voff), "s"(gbase)
               : "memory", "m0");
}

// Keeps the compiler from hoisting address arithmetic on `x` out of a loop
// (it would otherwise spend one VGPR and two adds per distinct LDS offset).
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void spatial_kernel(const bf16* __restrict__ Q,
                                                             const bf16* __restrict__ K,
                                                             const bf16* __restrict__ V,
                                                             bf16* __restrict__ O, int S, int nqt,
                                                             int nblocks, float c) {
  using G = Geo<D>;
  __shared__ __attribute__((aligned(16))) bf16 ring[kStages * G::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int logical = xcd_remap(blockIdx.x, nblocks);
  const int64_t seq = logical / nqt;
  const int qt = logical % nqt;
  const size_t base = (size_t)seq * (size_t)S * D;
  const bf16* __restrict__ Qs = Q + base;
  const bf16* __restrict__ Ks = K + base;
  const bf16* __restrict__ Vs = V + base;
  bf16* __restrict__ Os = O + base;

  // This wave's query rows as the B operand (Q^T), resident in registers.
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
  // Let Q land before the ring starts: the compiler tracks these loads but
  // not the direct loads, and would otherwise wait for everything in flight
  // at the first use of Q inside the loop.
  wait_vmcnt<0>();

  // Direct-load plan of this thread: slot s = i*256 + tid of the K (V) stage
  // holds chunk (row, ch) = (s / KCH, s % KCH) of the tile.  Pad chunks
  // (ch >= D/8) and surplus slots re-read chunk 0 of the tile: finite values
  // that nothing uses.  Byte offsets are relative to the tile's first row.
  uint32_t koff[G::KDMA], voff[G::VDMA];
#pragma unroll
  for (int i = 0; i < G::KDMA; ++i) {
    const int s = i * kThreads + tid, row = s / G::KCH, ch = s % G::KCH;
    koff[i] = (row < kBN && ch < G::DCH) ? (uint32_t)((row * D + ch * 8) * 2) : 0u;
  }
#pragma unroll
  for (int i = 0; i < G::VDMA; ++i) {
    const int s = i * kThreads + tid, row = s / G::VCH, ch = s % G::VCH;
    voff[i] = (row < kBN && ch < G::DCH) ? (uint32_t)((row * D + ch * 8) * 2) : 0u;
  }
  const uint32_t ring_lds = (uint32_t)(uintptr_t)LDS_PTR(void, ring);
  const uint32_t wave_slot = (uint32_t)(wave * kWave * 16);
  auto issue = [&](int t) {
    const int key0 = t * kBN;
    const uint32_t st = ring_lds + (uint32_t)((t % kStages) * G::STAGE * 2) + wave_slot;
    if (key0 + kBN <= S) {
      const bf16* kt = Ks + (size_t)key0 * D;
      const bf16* vt = Vs + (size_t)key0 * D;
#pragma unroll
      for (int i = 0; i < G::KDMA; ++i) dma16(kt, koff[i], st + (uint32_t)(i * kThreads * 16));
#pragma unroll
      for (int i = 0; i < G::VDMA; ++i)
        dma16(vt, voff[i], st + (uint32_t)(G::KSTAGE * 2 + i * kThreads * 16));
    } else {
      // Ragged last tile: rows past S repeat row S-1 (finite; their scores
      // are masked and their p are 0).
#pragma unroll
      for (int i = 0; i < G::KDMA; ++i) {
        const int s = i * kThreads + tid, row = s / G::KCH, ch = s % G::KCH;
        const int r = min(key0 + min(row, kBN - 1), S - 1);
        const uint32_t off = (row < kBN && ch < G::DCH) ? (uint32_t)((r * D + ch * 8) * 2) : 0u;
        dma16(Ks, off, st + (uint32_t)(i * kThreads * 16));
      }
#pragma unroll
      for (int i = 0; i < G::VDMA; ++i) {
        const int s = i * kThreads + tid, row = s / G::VCH, ch = s % G::VCH;
        const int r = min(key0 + min(row, kBN - 1), S - 1);
        const uint32_t off = (row < kBN && ch < G::DCH) ? (uint32_t)((r * D + ch * 8) * 2) : 0u;
        dma16(Vs, off, st + (uint32_t)(G::KSTAGE * 2 + i * kThreads * 16));
      }
    }
  };

  // Per-lane LDS bases of the operand reads; the rest of each address is a
  // compile-time offset.  Transposing V read: lane j of a 16-lane group
  // addresses row j/4 and columns 4*(j%4)..+3 of a 4x16 block and receives
  // column j, i.e. V^T row d = l32 of the operand.
  const int g16 = lane >> 4, j16 = lane & 15;
  const uint32_t klane = (uint32_t)((l32 * G::KS + h * 8) * 2);
  const uint32_t vlane =
      (uint32_t)(((h * 4 + (j16 >> 2)) * G::VS + (g16 & 1) * 16 + (j16 & 3) * 4) * 2);
  // Operand row D of V^T (the ones row) lives in lane D % 32 of block D / 32.
  const bool ones_lane = l32 == (D % 32);
  const uint32_t ones_word = ones_lane ? 0x3F803F80u : 0u;

  f32x16 oacc[G::QB][G::NB];
#pragma unroll
  for (int qb = 0; qb < G::QB; ++qb)
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb) oacc[qb][nb] = zero16();
  float mrow[G::QB];
#pragma unroll
  for (int qb = 0; qb < G::QB; ++qb) mrow[qb] = -INFINITY;  // log2 domain (score * c)

  const int nt = (S + kBN - 1) / kBN;
  issue(0);
  if (nt > 1) issue(1);

  for (int t = 0; t < nt; ++t) {
    // Tile t has landed once at most one tile's loads are still in flight.
    if (t + 1 < nt) {
      wait_vmcnt<G::KDMA + G::VDMA>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
    if (t + 2 < nt) issue(t + 2);  // refills the stage read in iteration t-1
    if (wave_live) {
      const uint32_t stage = ring_lds + (uint32_t)((t % kStages) * G::STAGE * 2);
      const uint32_t kaddr = opaque(stage + klane);
      const uint32_t vaddr = opaque(stage + (uint32_t)(G::KSTAGE * 2) + vlane);
      const int key0 = t * kBN;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        f32x16 sacc[G::QB];
#pragma unroll
        for (int qb = 0; qb < G::QB; ++qb) sacc[qb] = zero16();
#pragma unroll
        for (int ds = 0; ds < G::ND; ++ds) {
          const bf16x8 a =
              *LDS_PTR(const bf16x8, kaddr + (uint32_t)((kb * 32 * G::KS + ds * 16) * 2));
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
          mx = max_halves(mx);
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
            if (nb < G::NB - 1 || G::LAST_READ) {
              const uint32_t p = vaddr + (uint32_t)(((kb * 32 + t2 * 16) * G::VS + nb * 32) * 2);
              const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p));
              const i16x4 hi =
                  __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p + 8 * G::VS * 2));
              a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
              if (nb == G::NB - 1) {  // rows > D are don't-care; row D must be ones
                uint4 w = __builtin_bit_cast(uint4, a);
                w.x = ones_lane ? ones_word : w.x;
                w.y = ones_lane ? ones_word : w.y;
                w.z = ones_lane ? ones_word : w.z;
                w.w = ones_lane ? ones_word : w.w;
                a = __builtin_bit_cast(bf16x8, w);
              }
            } else {
              a = __builtin_bit_cast(bf16x8, make_uint4(ones_word, ones_word, ones_word, ones_word));
            }
#pragma unroll
            for (int qb = 0; qb < G::QB; ++qb) oacc[qb][nb] = mfma32(a, pb[qb][t2], oacc[qb][nb]);
          }
        }
      }
    }
  }

  if (wave_live) {
#pragma unroll
    for (int qb = 0; qb < G::QB; ++qb) {
      const HalfPair pr = half_pair(oacc[qb][G::NBD][G::RD]);
      const float inv = 1.f / (G::HD == 0 ? pr.lo : pr.hi);
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
