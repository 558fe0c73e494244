// temporal.hip -- bf16 temporal attention (PAB article, "Implementation",
// second observation: attention across the frames at one token position).
//
// Per (b, h, s): O[:, s] = softmax(Q[:, s] K[:, s]^T * scale) V[:, s] over the
// F <= 64 frames.  Short sequences, HBM-bound (about 24 flop per byte at
// F = 48, D = 72), so the design is about moving bytes: a 128-thread block
// takes 2 consecutive token positions of one (b, h) (small blocks, so several
// share a CU and their load, compute and store phases overlap); for every frame
// those positions are one contiguous run of 2*D elements, read as 16-byte vectors
// into LDS (K and V row-major, a frame column per position).  Each wave then
// owns one position: S^T = K Q^T on v_mfma_f32_32x32x16_bf16 with Q loaded
// straight into registers, a full-row softmax (no running max needed), and
// O^T = V^T P^T with the V^T operand taken by transposing LDS reads
// (ds_read_b64_tr_b16) of the row-major copy and an all-ones operand row D that
// yields the softmax denominator.
#include "device.hpp"
#include "launch.hpp"

namespace pab {

namespace {

constexpr int kWaves = 2;
constexpr int kThreads = kWaves * kWave;
constexpr int kPos = kWaves;        // token positions per block (one per wave)
constexpr int kSlack = 64;          // elements after V: transposing over-read of the last row

constexpr int kPadRows = 32;        // zero rows after the last position (frame over-read)
constexpr int kBatch = 8;           // 16-byte loads in flight per thread while filling LDS
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct Geo {
  static constexpr int ND = (D + 15) / 16;
  static constexpr int NB = D / 32 + 1;
  static constexpr int KS = D;        // dense rows; odd 16-byte count not required here
  static constexpr int CPR = D / 8;
  static constexpr int NBD = D / 32;
  static constexpr int HD = ((D % 32) % 8) / 4;
  static constexpr int RD = ((D % 32) / 8) * 4 + (D % 4);
};

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))


template <int D>
__global__ __launch_bounds__(kThreads) void temporal_kernel(const bf16* __restrict__ Q,
                                                           const bf16* __restrict__ K,
                                                           const bf16* __restrict__ V,
                                                           bf16* __restrict__ O, int F, int S,
                                                           int pos_blocks, int nblocks, float c) {
  using G = Geo<D>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int rows = kPos * F + kPadRows;   // rows per tensor in LDS
  bf16* ks = reinterpret_cast<bf16*>(smem);
  bf16* vs = ks + (size_t)rows * G::KS;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, l32 = lane & 31, h = lane >> 5;
  const int logical = xcd_remap(blockIdx.x, nblocks);
  const int64_t bh = logical / pos_blocks;
  const int s0 = (logical % pos_blocks) * kPos;
  const int64_t frame_stride = (int64_t)S * D;
  const size_t base = (size_t)bh * F * frame_stride;

  // This wave's position: Q^T operand straight from HBM, loaded first so that
  // it is in flight together with the K and V loads below.
  const int pos = wave;
  const int s = s0 + pos;
  const bool live = s < S;
  const int nqb = (F + 31) / 32;   // query (and key) blocks of 32 frames: 1 or 2
  bf16x8 qreg[2][G::ND];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int ds = 0; ds < G::ND; ++ds) {
      const int frame = qb * 32 + l32, d0 = ds * 16 + h * 8;
      qreg[qb][ds] = (live && frame < F && d0 < D)
                         ? *reinterpret_cast<const bf16x8*>(Q + base + (size_t)frame * frame_stride +
                                                            (size_t)s * D + d0)
                         : zero_bf16x8();
    }
  // Zero the pad rows (read by the 32-frame blocks past F of the last position).
  for (int i = tid; i < kPadRows * G::KS; i += kThreads) {
    ks[(size_t)kPos * F * G::KS + i] = (bf16)0.f;
    vs[(size_t)kPos * F * G::KS + i] = (bf16)0.f;
  }
  // K, V of positions s0..s0+kPos-1, all frames -> LDS row (pos*F + frame).
  const int per_frame = kPos * G::CPR;      // 16-byte chunks per frame run
  const int total = F * per_frame;
  for (int b0 = 0; b0 < total; b0 += kThreads * kBatch) {
    uint4 kr[kBatch], vr[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int idx = b0 + u * kThreads + tid;
      kr[u] = make_uint4(0u, 0u, 0u, 0u);
      vr[u] = make_uint4(0u, 0u, 0u, 0u);
      if (idx < total) {
        const int frame = idx / per_frame, rem = idx % per_frame;
        const int p = rem / G::CPR, ch = rem % G::CPR;
        if (s0 + p < S) {
          const size_t g = base + (size_t)frame * frame_stride + (size_t)(s0 + p) * D + ch * 8;
          kr[u] = *reinterpret_cast<const uint4*>(K + g);
          vr[u] = *reinterpret_cast<const uint4*>(V + g);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int idx = b0 + u * kThreads + tid;
      if (idx < total) {
        const int frame = idx / per_frame, rem = idx % per_frame;
        const int p = rem / G::CPR, ch = rem % G::CPR;
        const size_t l = (size_t)(p * F + frame) * G::KS + ch * 8;
        *reinterpret_cast<uint4*>(ks + l) = kr[u];
        *reinterpret_cast<uint4*>(vs + l) = vr[u];
      }
    }
  }

  __syncthreads();

  if (live) {
  const bf16* kp = ks + (size_t)pos * F * G::KS;
  const bf16* vp = vs + (size_t)pos * F * G::KS;
  const int nsteps = (F + 15) / 16;   // 16-frame PV steps

  // V^T operand for output block nb, PV step t (frames 16t + {h*4+j, 8+h*4+j})
  // by transposing LDS reads of the row-major V: lane j of a 16-lane group
  // addresses frame row j/4, columns 4*(j%4)..+3 of a 4x16 block and receives
  // column j (operand row d = l32).  Operand row D is ones (the softmax
  // denominator); rows > D are don't-care.
  const int g16 = lane >> 4, j16 = lane & 15;
  const bf16* vlane = vp + (h * 4 + (j16 >> 2)) * G::KS + (g16 & 1) * 16 + (j16 & 3) * 4;
  const bool ones_lane = l32 == (D % 32);
  const uint32_t ones_word = ones_lane ? 0x3F803F80u : 0u;
  auto v_operand = [&](int nb, int t) -> bf16x8 {
    uint4 w;
    if (nb * 32 < D) {
      const bf16* p = vlane + t * 16 * G::KS + nb * 32;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p + 8 * G::KS));
      const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
      w = make_uint4(l2.x, l2.y, h2.x, h2.y);
      if ((nb + 1) * 32 > D) {
        w.x = ones_lane ? ones_word : w.x;
        w.y = ones_lane ? ones_word : w.y;
        w.z = ones_lane ? ones_word : w.z;
        w.w = ones_lane ? ones_word : w.w;
      }
    } else {
      w = make_uint4(ones_word, ones_word, ones_word, ones_word);
    }
    return __builtin_bit_cast(bf16x8, w);
  };

  // Phase 1: probabilities of both 32-frame query blocks.  All reads of K
  // happen here, before any output is staged in the K rows.
  bf16x8 pbs[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    if (qb < nqb) {
      f32x16 sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = zero16();
        if (kb < nqb) {
#pragma unroll
          for (int ds = 0; ds < G::ND; ++ds) {
            const bf16x8 a = *reinterpret_cast<const bf16x8*>(kp + (size_t)(kb * 32 + l32) * G::KS +
                                                              ds * 16 + h * 8);
            sacc[kb] = mfma32(a, qreg[qb][ds], sacc[kb]);
          }
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if (kb * 32 + acc_row(r, h) >= F) sacc[kb][r] = -INFINITY;
          mx = fmaxf(mx, sacc[kb][r]);
        }
      mx = max_halves(mx);
      const float negm = -mx * c;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if (t < nsteps) {
          const int kb = t >> 1, r0 = (t & 1) * 8;
          pbs[qb][t] = to_bf16x8(
              fast_exp2(fmaf(sacc[kb][r0 + 0], c, negm)), fast_exp2(fmaf(sacc[kb][r0 + 1], c, negm)),
              fast_exp2(fmaf(sacc[kb][r0 + 2], c, negm)), fast_exp2(fmaf(sacc[kb][r0 + 3], c, negm)),
              fast_exp2(fmaf(sacc[kb][r0 + 4], c, negm)), fast_exp2(fmaf(sacc[kb][r0 + 5], c, negm)),
              fast_exp2(fmaf(sacc[kb][r0 + 6], c, negm)), fast_exp2(fmaf(sacc[kb][r0 + 7], c, negm)));
        }
      }
    }
  }

  // Phase 2: O^T = V^T P^T per query block, then staged row-major in LDS.
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    if (qb >= nqb) break;
    f32x16 oacc[G::NB];
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb) oacc[nb] = zero16();
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (t < nsteps) {
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb) oacc[nb] = mfma32(v_operand(nb, t), pbs[qb][t], oacc[nb]);
      }
    }

    const HalfPair pr = half_pair(oacc[G::NBD][G::RD]);
    const float inv = 1.f / (G::HD == 0 ? pr.lo : pr.hi);
    const int frame = qb * 32 + l32;
    // Stage O row-major in this position's K rows: its own scores are done,
    // and other waves only read these rows for masked keys or against zero
    // Q padding, where the values do not matter.
    if (frame < F) {
      bf16* orow = ks + (size_t)(pos * F + frame) * G::KS;
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          if (nb * 32 + g * 8 < D) {  // d0 = nb*32 + g*8 + h*4 < D (D % 8 == 0)
            const int d0 = nb * 32 + g * 8 + h * 4;
            const uint2 w = make_uint2(pack_bf16x2(oacc[nb][g * 4 + 0] * inv, oacc[nb][g * 4 + 1] * inv),
                                       pack_bf16x2(oacc[nb][g * 4 + 2] * inv, oacc[nb][g * 4 + 3] * inv));
            *reinterpret_cast<uint2*>(orow + d0) = w;
          }
        }
    }
  }
  }  // live
  __syncthreads();
  // O of positions s0..s0+kPos-1, all frames: each frame's run of kPos*D elements is
  // contiguous in HBM, written with 16-byte stores (same pattern as the loads).
  for (int idx = tid; idx < total; idx += kThreads) {
    const int frame = idx / per_frame, rem = idx % per_frame;
    const int p = rem / G::CPR, ch = rem % G::CPR;
    if (s0 + p < S) {
      const size_t g = base + (size_t)frame * frame_stride + (size_t)(s0 + p) * D + ch * 8;
      *reinterpret_cast<uint4*>(O + g) =
          *reinterpret_cast<const uint4*>(ks + (size_t)(p * F + frame) * G::KS + ch * 8);
    }
  }
}

template <int D>
hipError_t launch_d(const void* q, const void* k, const void* v, void* o, int64_t nbh, int F, int S,
                    float c, hipStream_t stream) {
  const int pos_blocks = (S + kPos - 1) / kPos;
  const int64_t nblocks = nbh * pos_blocks;
  if (nblocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const size_t lds = (2 * (size_t)(kPos * F + kPadRows) * Geo<D>::KS + kSlack) * sizeof(bf16);
  if (lds > 65536) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&temporal_kernel<D>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(temporal_kernel<D>, dim3((unsigned)nblocks), dim3(kThreads), lds, stream,
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, F, S, pos_blocks,
                     (int)nblocks, c);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_temporal_bf16(const void* q, const void* k, const void* v, void* o, int64_t nbh,
                                int F, int S, int D, float scale, hipStream_t stream) {
  const float c = scale * kLog2e;
  switch (D) {
#define PAB_CASE(d) \
  case d:           \
    return launch_d<d>(q, k, v, o, nbh, F, S, c, stream);
    PAB_CASE(8) PAB_CASE(16) PAB_CASE(24) PAB_CASE(32) PAB_CASE(40) PAB_CASE(48) PAB_CASE(56)
    PAB_CASE(64) PAB_CASE(72) PAB_CASE(80) PAB_CASE(88) PAB_CASE(96) PAB_CASE(104) PAB_CASE(112)
    PAB_CASE(120) PAB_CASE(128)
#undef PAB_CASE
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace pab
