// temporal.hip -- bf16 temporal attention (PAB article, "Implementation",
// second observation: attention across the frames at one token position).
//
// Per (b, h, s): O[:, s] = softmax(Q[:, s] K[:, s]^T * scale) V[:, s] over the
// F <= 64 frames.  Short sequences, HBM-bound (about 24 flop per byte at
// F = 48, D = 72), so the design is about moving bytes.  A 256-thread block
// takes 4 consecutive token positions of one (b, h) (two blocks share a CU,
// so their load, compute and store phases overlap).  For every frame those
// positions are one contiguous run of 4*D elements in HBM; K and V
// are copied run by run into LDS in the same frame-major order by direct
// global->LDS loads (whole runs per request, no staging registers), while Q
// goes straight to registers.  Each wave then owns one position:
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16, a full-row softmax (no running
//     max needed: at most 64 frames);
//   * O^T = V^T P^T with the V^T operand taken by transposing LDS reads
//     (ds_read_b64_tr_b16) and an all-ones operand row D that yields the
//     softmax denominator;
//   * the output is staged frame-major in the K buffer and written back run
//     by run with lane-contiguous 16-byte stores; with a previous output P
//     (the attention difference) the same chunks of P are read into
//     registers together with the inputs and each block writes the fp64 sum
//     of squared differences of what it stores.
#include "device.hpp"
#include "launch.hpp"

namespace pab {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kPos = kWaves;        // token positions per block (one per wave)
constexpr int kMaxF = 64;           // frames; LDS holds 64 frame runs per tensor
constexpr int kSlack = 64;          // elements after V: transposing over-read of the last run
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct Geo {
  static constexpr int ND = (D + 15) / 16;
  static constexpr int NB = D / 32 + 1;
  static constexpr int RUN = kPos * D;           // elements per frame run (LDS row stride)
  static constexpr int RCH = RUN / 8;            // 16-byte chunks per run
  static constexpr int NBD = D / 32;
  static constexpr int HD = ((D % 32) % 8) / 4;
  static constexpr int RD = ((D % 32) / 8) * 4 + (D % 4);
  static constexpr int LDS_ELEMS = 2 * kMaxF * RUN + kSlack;
};

typedef short i16x4 __attribute__((ext_vector_type(4)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// One 16-byte direct global->LDS load per lane: lane l of the wave reads
// global bytes [gbase + voff, +16) and writes LDS bytes [lds + 16*l, +16).
// `gbase` and `lds` must be wave-uniform.  Inline assembly, so that the wait
// for it is placed by hand (the compiler does not track these loads).
// m0 is listed as clobbered, which the compiler reports as a reserved
// register; these kernels never use m0 themselves (their code outside
// this statement does not touch it), so the clobber only keeps the
// compiler from relying on m0 across the load.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(voff), "s"(gbase)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// A wave-uniform pointer, moved to scalar registers (the direct load takes
// its base address from an SGPR pair).
__device__ __forceinline__ const bf16* uniform_ptr(const bf16* p) {
  const uint64_t u = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const bf16*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

template <int D>
__global__ __launch_bounds__(kThreads) void temporal_kernel(const bf16* __restrict__ Q,
                                                           const bf16* __restrict__ K,
                                                           const bf16* __restrict__ V,
                                                           bf16* __restrict__ O, int F, int S,
                                                           int pos_blocks, int nblocks, float c,
                                                           const bf16* __restrict__ P,
                                                           double* __restrict__ partials) {
  using G = Geo<D>;
  __shared__ __attribute__((aligned(16))) bf16 smem[G::LDS_ELEMS];
  bf16* ks = smem;                     // K runs, frame-major: row f holds positions 0..kPos-1
  bf16* vs = smem + kMaxF * G::RUN;    // V runs

  const int tid = threadIdx.x;
  const int lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int logical = xcd_remap(blockIdx.x, nblocks);
  const int64_t bh = logical / pos_blocks;
  const int s0 = (logical % pos_blocks) * kPos;
  const int64_t frame_stride = (int64_t)S * D;
  const size_t base = (size_t)bh * F * frame_stride;
  // Positions of this block that exist (the last block of a (b, h) may hold one).
  const int npos = min(kPos, S - s0);

  // This wave's position: Q^T operand straight from HBM, issued first so it is
  // in flight together with the K and V loads.
  const int pos = wave;
  const int s = s0 + pos;
  const bool live = pos < npos;
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

  // Attention difference against a previous output P (when given): the
  // chunks this thread will store are requested together with Q, K and V,
  // so their latency overlaps that of the inputs; chunk k of the thread is
  // output slot tid + 256 k.
  constexpr int kOwn = (kMaxF * G::RCH + kThreads - 1) / kThreads;
  const int valid_out = npos * (D / 8);
  uint4 prev[kOwn];
  if (P) {
    const bf16* pb0 = P + base + (size_t)s0 * D;
#pragma unroll
    for (int k = 0; k < kOwn; ++k) {
      const int i = tid + k * kThreads;
      const int frame = i / G::RCH, ch = i % G::RCH;
      prev[k] = make_uint4(0u, 0u, 0u, 0u);
      if (frame < F && ch < valid_out)
        prev[k] = *reinterpret_cast<const uint4*>(pb0 + (size_t)frame * frame_stride + ch * 8);
    }
  }

  // K and V runs -> LDS by direct loads.  Slot i of a tensor (16 bytes) is
  // chunk i % RCH of frame i / RCH; chunks of a missing position re-read the
  // first position's (finite, never stored).  Load j of the block covers
  // slots 64 j .. 64 j + 63; the waves take alternate loads, and lanes past
  // the last slot stay idle.
  {
    const int slots = F * G::RCH;
    const int nj = (slots + kWave - 1) / kWave;
    const bf16* kb0 = uniform_ptr(K + base + (size_t)s0 * D);
    const bf16* vb0 = uniform_ptr(V + base + (size_t)s0 * D);
    const uint32_t k_lds = (uint32_t)(uintptr_t)LDS_PTR(void, ks);
    const uint32_t v_lds = (uint32_t)(uintptr_t)LDS_PTR(void, vs);
    const int valid_ch = npos * (D / 8);
    for (int j = wave; j < nj; j += kWaves) {
      const int i = j * kWave + lane;
      const int frame = i / G::RCH, ch = i % G::RCH;
      const int gch = ch < valid_ch ? ch : ch % (D / 8);
      const uint32_t off = (uint32_t)(((size_t)frame * frame_stride + gch * 8) * 2);
      const uint32_t kl = __builtin_amdgcn_readfirstlane(k_lds + (uint32_t)(j * 1024));
      const uint32_t vl = __builtin_amdgcn_readfirstlane(v_lds + (uint32_t)(j * 1024));
      if (i < slots) {
        dma16(kb0, off, kl);
        dma16(vb0, off, vl);
      }
    }
  }
  // Runs past F that are read must hold finite values: V runs up to the last
  // 16-frame PV step (their p are 0), and K runs up to the last 32-frame
  // block (scores of frames >= F are masked after the product).  Zero them.
  {
    const int nqb32 = (F + 31) / 32 * 32;
    const int kpad = min(kMaxF, nqb32);
    const int vpad = min(kMaxF, (F + 15) / 16 * 16);
    for (int i = F * G::RCH + tid; i < kpad * G::RCH; i += kThreads)
      *reinterpret_cast<uint4*>(ks + i * 8) = make_uint4(0u, 0u, 0u, 0u);
    for (int i = F * G::RCH + tid; i < vpad * G::RCH; i += kThreads)
      *reinterpret_cast<uint4*>(vs + i * 8) = make_uint4(0u, 0u, 0u, 0u);
  }
  __builtin_amdgcn_s_waitcnt(0x0070 | 0x0F00);  // vmcnt(0): this wave's loads have landed
  __syncthreads();

  if (live) {
    const bf16* kp = ks + pos * D;
    const bf16* vp = vs + pos * D;
    const int nsteps = (F + 15) / 16;   // 16-frame PV steps

    // V^T operand for output block nb, PV step t (frames 16t + {h*4+j,
    // 8+h*4+j}) by transposing LDS reads of the frame-major V: lane j of a
    // 16-lane group addresses frame row j/4, columns 4*(j%4)..+3 of a 4x16
    // block and receives column j (operand row d = l32).  Operand row D is
    // ones (the softmax denominator); rows > D are don't-care.
    const int g16 = lane >> 4, j16 = lane & 15;
    const bf16* vlane = vp + (h * 4 + (j16 >> 2)) * G::RUN + (g16 & 1) * 16 + (j16 & 3) * 4;
    const bool ones_lane = l32 == (D % 32);
    const uint32_t ones_word = ones_lane ? 0x3F803F80u : 0u;
    auto v_operand = [&](int nb, int t) -> bf16x8 {
      uint4 w;
      if (nb * 32 < D) {
        const bf16* p = vlane + t * 16 * G::RUN + nb * 32;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p + 8 * G::RUN));
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
    // happen here, before any output is staged in the K buffer.  A wave reads
    // only its own position's columns: where D % 16 == 8 the upper half of the
    // last 16-wide step (d = D..D+7, the next position's columns, which that
    // position's wave may already be overwriting with its output) is not read
    // but taken as zero, as Q's padding there is.
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
              const bool past = ds * 16 + 8 >= D && h == 1;  // d >= D: not this position's
              const bf16x8 a = past ? zero_bf16x8()
                                    : *reinterpret_cast<const bf16x8*>(kp + (kb * 32 + l32) * G::RUN +
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

    // Phase 2: O^T = V^T P^T per query block, staged frame-major in the K
    // buffer (this position's columns, which no other wave reads).
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
      if (frame < F) {
        bf16* orow = ks + frame * G::RUN + pos * D;
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
  }
  __syncthreads();
  // O runs back to HBM: run f of the block is contiguous there, written with
  // 16-byte stores in the order of the loads.
  bf16* ob0 = O + base + (size_t)s0 * D;
  if (P) {
    double dsum = 0.0;
#pragma unroll
    for (int k = 0; k < kOwn; ++k) {
      const int i = tid + k * kThreads;
      const int frame = i / G::RCH, ch = i % G::RCH;
      if (frame < F && ch < valid_out) {
        const uint4 w = *reinterpret_cast<const uint4*>(ks + i * 8);
        *reinterpret_cast<uint4*>(ob0 + (size_t)frame * frame_stride + ch * 8) = w;
        dsum += sqdiff_bf16x2(w.x, prev[k].x) + sqdiff_bf16x2(w.y, prev[k].y) +
                sqdiff_bf16x2(w.z, prev[k].z) + sqdiff_bf16x2(w.w, prev[k].w);
      }
    }
    __syncthreads();  // every thread is done with the staged output: reuse LDS for the sum
    const double s = block_sum_f64<kWaves>(dsum, reinterpret_cast<double*>(smem));
    if (tid == 0) partials[blockIdx.x] = s;
    return;
  }
  for (int i = tid; i < F * G::RCH; i += kThreads) {
    const int frame = i / G::RCH, ch = i % G::RCH;
    if (ch < valid_out)
      *reinterpret_cast<uint4*>(ob0 + (size_t)frame * frame_stride + ch * 8) =
          *reinterpret_cast<const uint4*>(ks + i * 8);
  }
}

template <int D>
hipError_t launch_d(const void* q, const void* k, const void* v, void* o, int64_t nbh, int F, int S,
                    float c, const DiffOut& diff, hipStream_t stream) {
  const int pos_blocks = (S + kPos - 1) / kPos;
  const int64_t nblocks = nbh * pos_blocks;
  // Direct-load offsets are 32-bit: one (b, h) slab must stay below 4 GiB.
  if (nblocks > 0x7fffffff || F > kMaxF || (int64_t)F * S * D * 2 >= ((int64_t)1 << 32))
    return hipErrorInvalidConfiguration;
  const bool fused = diff.prev && nblocks <= diff.capacity;
  if (diff.nparts) *diff.nparts = fused ? (int)nblocks : 0;
  hipLaunchKernelGGL(temporal_kernel<D>, dim3((unsigned)nblocks), dim3(kThreads), 0, stream,
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, F, S, pos_blocks,
                     (int)nblocks, c, fused ? (const bf16*)diff.prev : nullptr,
                     fused ? diff.partials : nullptr);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_temporal_bf16(const void* q, const void* k, const void* v, void* o, int64_t nbh,
                                int F, int S, int D, float scale, const DiffOut& diff,
                                hipStream_t stream) {
  const float c = scale * kLog2e;
  switch (D) {
#define PAB_CASE(d) \
  case d:           \
    return launch_d<d>(q, k, v, o, nbh, F, S, c, diff, stream);
    PAB_CASE(8) PAB_CASE(16) PAB_CASE(24) PAB_CASE(32) PAB_CASE(40) PAB_CASE(48) PAB_CASE(56)
    PAB_CASE(64) PAB_CASE(72) PAB_CASE(80) PAB_CASE(88) PAB_CASE(96) PAB_CASE(104) PAB_CASE(112)
    PAB_CASE(120) PAB_CASE(128)
#undef PAB_CASE
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace pab
