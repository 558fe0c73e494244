// cross.hip -- bf16 cross attention: video queries attend to text keys/values
// (PAB article, "Implementation", second observation: cross attention ties
// the text to the video and changes least between steps).
//
// Per (b, h): the Nq = F*S video queries against L <= 128 text keys.  The
// text K and V (row-major, read with 16-byte vector loads) are loaded into LDS
// once per block and stay resident; 32-row query tiles stream from HBM
// through each wave, so Q is read once and O written once: the kernel is
// HBM-bound.
//   * Scores are formed transposed (S^T = K Q^T, v_mfma_f32_32x32x16_bf16) so
//     one lane holds one query row's scores; with at most 128 keys the whole
//     row fits in registers and the softmax needs no running max.
//   * When D is not a multiple of 16 the Q K^T contraction is padded anyway;
//     the padding column d = D carries a key bias (0 for real keys, -1e30 for
//     the padding keys past L) against a 1 in Q, so padding keys are masked
//     by the MFMA itself.
//   * The V^T operand comes from the row-major V through ds_read_b64_tr_b16;
//     V carries a column D of ones (zeros past L), so O^T row D is the
//     softmax denominator, summed on the MFMA.
//   * A 32-row query tile is one contiguous run in HBM: it is copied into a
//     per-wave two-stage LDS ring by direct global->LDS loads (whole-line
//     requests, no staging registers), the next tile's loads running while
//     the current one computes; the tile's output is staged row-major in the
//     same stage and written with lane-contiguous 16-byte stores.
//   * With a previous output to compare against (the attention difference),
//     its tile comes into the query tile's own stage once Q is in registers
//     (direct loads again, under the scores and PV); each lane takes its
//     chunks into registers before the output is staged there, and the
//     copy-out accumulates the squared differences.
#include "device.hpp"
#include "launch.hpp"

namespace pab {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr float kLog2e = 1.4426950408889634f;

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// Smallest row stride (elements, multiple of 8, >= min_elems) whose first four
// rows start on disjoint 8-bank spans (one 16-lane group of a transposing read
// touches 32 bytes of four consecutive rows).
constexpr int tr_stride(int min_elems) {
  for (int s = (min_elems + 7) / 8 * 8;; s += 8) {
    const int w = s / 2;
    bool ok = true;
    for (int a = 0; a < 4 && ok; ++a)
      for (int b = a + 1; b < 4 && ok; ++b) {
        const int d = (w * (b - a)) % 64;
        if (d < 8 || d > 56) ok = false;
      }
    if (ok) return s;
  }
}

// Row stride (elements) with an odd number of 16-byte chunks, >= min_elems:
// the 32 rows read by one MFMA operand load then sit on distinct banks.
constexpr int odd_chunk_stride(int min_elems) {
  const int s = (min_elems + 7) / 8 * 8;
  return ((s / 8) % 2) ? s : s + 8;
}

// One 16-byte direct global->LDS load per lane: lane l of the wave reads
// global bytes [gbase + voff, +16) and writes LDS bytes [lds + 16*l, +16).
// `gbase` and `lds` must be wave-uniform.  Issued from inline assembly so that
// its wait (s_waitcnt vmcnt) is placed by hand; the instruction has no
// result register.
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

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int D, int NKB>
struct Geo {
  static constexpr int ND = (D + 15) / 16;             // 16-wide d steps of Q K^T
  static constexpr int NB = D / 32 + 1;                // 32-row blocks of O^T
  static constexpr bool BIAS = (D % 16) != 0;          // padding column d = D exists
  static constexpr int KS = BIAS ? D + 8 : odd_chunk_stride(D);
  static constexpr int KROWS = NKB * 32 + 1;           // +1: keeps row reads in bounds
  // The last 32-row O^T block holds data rows and the denominator row D: V
  // then carries a column D of ones (zeros past L) so the operand needs no
  // per-use fix-up.
  static constexpr bool ONES_COL = (D % 32) != 0;
  static constexpr int VS = tr_stride(ONES_COL ? D + 1 : D);
  static constexpr int VROWS = NKB * 32;
  static constexpr int VSLACK = 64;                    // transposing over-read past the last row
  static constexpr int CPR = D / 8;                    // 16-byte chunks per input row
  // A 32-row query tile is contiguous in HBM: NQJ wave-wide 1 KiB direct
  // loads fill one stage of the wave's two-stage ring, which later also
  // stages the tile's output.
  static constexpr int NQJ = (32 * D * 2 + 1023) / 1024;
  static constexpr int QSTAGE = 32 * D;                // elements; the last load is partial
  static constexpr int NOST = (32 * D / 8 + kWave - 1) / kWave;  // output stores per tile
  static constexpr bool LAST_READ = (NB - 1) * 32 < D;
  // LDS of a block: text K and V, and each wave's two-stage query ring.
  static constexpr int LDS_BYTES = (KROWS * KS + VROWS * VS + VSLACK) * 2 + kWaves * 2 * QSTAGE * 2;
  static constexpr int PER_CU = (160 * 1024) / LDS_BYTES >= 2 ? 2 : 1;  // resident blocks
  static constexpr int NBD = D / 32;
  static constexpr int HD = ((D % 32) % 8) / 4;
  static constexpr int RD = ((D % 32) / 8) * 4 + (D % 4);
};

template <int D, int NKB, bool DIFF>
__global__ __launch_bounds__(kThreads, (Geo<D, NKB>::PER_CU)) void cross_kernel(const bf16* __restrict__ Q,
                                                           const bf16* __restrict__ Kt,
                                                           const bf16* __restrict__ Vt,
                                                           bf16* __restrict__ O, int64_t nq, int L, int Lrows,
                                                           int tiles_per_block, int blocks_per_bh,
                                                           int nblocks, float c,
                                                           const bf16* __restrict__ P,
                                                           double* __restrict__ partials) {
  using G = Geo<D, NKB>;
  constexpr int QJ = G::NQJ;  // direct loads per query tile
  __shared__ __attribute__((aligned(16))) bf16 ks[G::KROWS * G::KS];
  __shared__ __attribute__((aligned(16))) bf16 vs[G::VROWS * G::VS + G::VSLACK];
  // Per-wave two-stage ring of query tiles (each stage later holds the
  // tile's output, row-major).
  __shared__ __attribute__((aligned(16))) bf16 qstage[kWaves][2][G::QSTAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int logical = xcd_remap(blockIdx.x, nblocks);
  const int bh = logical / blocks_per_bh;
  const int chunk = logical % blocks_per_bh;
  const bf16* __restrict__ Qh = Q + (int64_t)bh * nq * D;
  bf16* __restrict__ Oh = O + (int64_t)bh * nq * D;
  const bf16* __restrict__ Ph = DIFF ? P + (int64_t)bh * nq * D : nullptr;
  double dsum = 0.0;
  // Text rows of (b, h) are Lrows apart; the first L of them are real.
  const bf16* __restrict__ Kh = Kt + (int64_t)bh * Lrows * D;
  const bf16* __restrict__ Vh = Vt + (int64_t)bh * Lrows * D;

  const int ntiles = (int)((nq + 31) / 32);
  const int t_begin = chunk * tiles_per_block;
  const int t_end = min(t_begin + tiles_per_block, ntiles);

  // Text K and V -> LDS, row-major, 16-byte vectors; all loads of a thread
  // are issued before its stores.  Rows >= L: K zero, V zero (their p are 0).
  {
    constexpr int kChunks = G::KROWS * G::CPR;
    constexpr int kIter = (kChunks + kThreads - 1) / kThreads;
    uint4 kr[kIter], vr[kIter];
#pragma unroll
    for (int it = 0; it < kIter; ++it) {
      const int i = tid + it * kThreads;
      const int row = i / G::CPR, ch = i % G::CPR;
      const bool valid = i < kChunks && row < L;
      const int64_t g = valid ? (int64_t)row * D + ch * 8 : 0;
      kr[it] = valid ? *reinterpret_cast<const uint4*>(Kh + g) : make_uint4(0u, 0u, 0u, 0u);
      vr[it] = valid ? *reinterpret_cast<const uint4*>(Vh + g) : make_uint4(0u, 0u, 0u, 0u);
    }
#pragma unroll
    for (int it = 0; it < kIter; ++it) {
      const int i = tid + it * kThreads;
      const int row = i / G::CPR, ch = i % G::CPR;
      if (i < kChunks) {
        *reinterpret_cast<uint4*>(&ks[row * G::KS + ch * 8]) = kr[it];
        if (row < G::VROWS) *reinterpret_cast<uint4*>(&vs[row * G::VS + ch * 8]) = vr[it];
      }
    }
    // Columns D..VS-1 of every V row: ones at d = D for real keys, zeros
    // elsewhere.
    if (G::ONES_COL) {
      for (int i = tid; i < G::VROWS; i += kThreads) {
#pragma unroll
        for (int d = D; d < G::VS; ++d) vs[i * G::VS + d] = (bf16)((d == D && i < L) ? 1.f : 0.f);
      }
    }
    // Columns D..KS-1 of every K row: the key bias at d = D (when it exists),
    // zeros after it.
    for (int i = tid; i < G::KROWS; i += kThreads) {
#pragma unroll
      for (int d = D; d < G::KS; ++d) {
        float val = 0.f;
        if (G::BIAS && d == D && i >= L) val = -1e30f;
        ks[i * G::KS + d] = (bf16)val;
      }
    }
  }
  __syncthreads();

  // Transposing V read: lane j of a 16-lane group addresses row j/4, columns
  // 4*(j%4)..+3 of a 4x16 block and receives column j (operand row d = l32).
  const int g16 = lane >> 4, j16 = lane & 15;
  const uint32_t vs_lds = (uint32_t)(uintptr_t)LDS_PTR(void, vs);
  const uint32_t vlane =
      vs_lds + (uint32_t)(((h * 4 + (j16 >> 2)) * G::VS + (g16 & 1) * 16 + (j16 & 3) * 4) * 2);
  const uint32_t ks_lds = (uint32_t)(uintptr_t)LDS_PTR(void, ks);
  const uint32_t klane = ks_lds + (uint32_t)((l32 * G::KS + h * 8) * 2);
  // With D % 32 == 0 the last O^T block is the ones row alone (lane 0).
  const uint32_t ones_word = l32 == 0 ? 0x3F803F80u : 0u;
  // Q padding word at d = D (1 in its low half) when the bias column is used.
  const uint32_t qpad_word = G::BIAS ? 0x00003F80u : 0u;

  // Direct loads of query tile `tile` into stage `st` (LDS byte address),
  // and of the previous output's tile into stage `pst` when DIFF: lane l of
  // load j copies tile bytes [1024 j + 16 l, +16), clamped to the tile's last
  // valid 16 bytes (rows past nq re-read it: finite values whose outputs are
  // not stored).
  auto issue_tile = [&](const bf16* base, int tile, uint32_t st) {
    const int64_t rows_left = nq - (int64_t)tile * 32;
    const uint32_t valid = (uint32_t)((rows_left >= 32 ? 32 : rows_left) * D * 2);
    const bf16* tb = base + (int64_t)tile * 32 * D;
#pragma unroll
    for (int j = 0; j < G::NQJ; ++j) {
      const uint32_t pos = (uint32_t)(j * 1024 + lane * 16);
      const uint32_t off = min(pos, valid - 16u);
      // Lanes past the stage stay idle (their LDS bytes are not written).
      if (j + 1 < G::NQJ || pos < (uint32_t)(32 * D * 2)) dma16(tb, off, st + (uint32_t)(j * 1024));
    }
  };

  // One 32-row query tile against the text keys: full-row softmax,
  // O = P V / sum(P) on the MFMA, row-major staging, coalesced stores.
  auto compute = [&](bf16* ost, int tile) {
    // Q^T operand: lane (row l32, half h) holds d = ds*16 + h*8 .. +7.
    const uint32_t qlane = (uint32_t)(uintptr_t)LDS_PTR(void, ost) + (uint32_t)((l32 * D + h * 8) * 2);
    u32x4 q[G::ND];
#pragma unroll
    for (int ds = 0; ds < G::ND; ++ds) {
      if (ds * 16 + 8 < D) {  // both halves hold data
        q[ds] = *LDS_PTR(const u32x4, qlane + (uint32_t)(ds * 32));
      } else {  // last step of a D % 16 == 8 head: the upper half is padding
        const u32x4 pad = {qpad_word, 0u, 0u, 0u};
        const u32x4 lo = *LDS_PTR(const u32x4, qlane + (uint32_t)(ds * 32) - (uint32_t)(h * 16));
        q[ds] = h == 0 ? lo : pad;
      }
    }
    if constexpr (DIFF) {
      // The stage is free once Q is in registers: the previous output's tile
      // comes into it by direct loads while the scores and PV run.
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the Q reads are done
      issue_tile(Ph, tile, (uint32_t)(uintptr_t)LDS_PTR(void, ost));
    }
    f32x16 sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      sacc[kb] = zero16();
#pragma unroll
      for (int ds = 0; ds < G::ND; ++ds) {
        const u32x4 a = *LDS_PTR(const u32x4, klane + (uint32_t)((kb * 32 * G::KS + ds * 16) * 2));
        sacc[kb] = mfma32(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, q[ds]), sacc[kb]);
      }
    }
    if (!G::BIAS) {  // no bias column: keys from L on are masked in every block that has them
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        if ((kb + 1) * 32 > L) {
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (kb * 32 + acc_row(r, h) >= L) sacc[kb][r] = -INFINITY;
        }
      }
    }
    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = max_halves(mx);
    const float negm = -mx * c;

    f32x16 oacc[G::NB];
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb) oacc[nb] = zero16();
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
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
          u32x4 a;
          if (nb < G::NB - 1 || G::LAST_READ) {
            const uint32_t p = vlane + (uint32_t)(((kb * 32 + t2 * 16) * G::VS + nb * 32) * 2);
            const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p));
            const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p + 8 * G::VS * 2));
            const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
            a = u32x4{l2.x, l2.y, h2.x, h2.y};  // operand rows > D are don't-care
          } else {
            a = u32x4{ones_word, ones_word, ones_word, ones_word};
          }
          oacc[nb] = mfma32(__builtin_bit_cast(bf16x8, a), pb, oacc[nb]);
        }
      }
    }

    // The previous output's chunks this lane will store, into registers before
    // the output overwrites the stage (a wave's LDS operations run in order).
    constexpr int kOutChunks = 32 * D / 8;
    const int64_t rows_left = nq - (int64_t)tile * 32;
    const int valid_chunks = rows_left >= 32 ? kOutChunks : (int)rows_left * (D / 8);
    uint4 pv[DIFF ? G::NOST : 1];
    if constexpr (DIFF) {
      wait_vmcnt<0>();  // the previous output's tile has landed
      asm volatile("" ::: "memory");
#pragma unroll
      for (int i = 0; i < G::NOST; ++i) {
        const int ch = i * kWave + lane;
        pv[i] = make_uint4(0u, 0u, 0u, 0u);
        if (ch < valid_chunks) {
          const u32x4 t4 = *LDS_PTR(const u32x4, (uint32_t)(uintptr_t)LDS_PTR(void, ost) + (uint32_t)(ch * 16));
          pv[i] = make_uint4(t4[0], t4[1], t4[2], t4[3]);
        }
      }
    }
    const HalfPair pr = half_pair(oacc[G::NBD][G::RD]);
    const float inv = 1.f / (G::HD == 0 ? pr.lo : pr.hi);
    // Accumulators -> row-major tile in LDS (lane: row l32, 4 d per piece).
#pragma unroll
    for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (nb * 32 + g * 8 < D) {  // d0 = nb*32 + g*8 + h*4 < D (D % 8 == 0)
          const int d0 = nb * 32 + g * 8 + h * 4;
          const uint2 w = make_uint2(pack_bf16x2(oacc[nb][g * 4 + 0] * inv, oacc[nb][g * 4 + 1] * inv),
                                     pack_bf16x2(oacc[nb][g * 4 + 2] * inv, oacc[nb][g * 4 + 3] * inv));
          *reinterpret_cast<uint2*>(&ost[l32 * D + d0]) = w;
        }
      }
    __builtin_amdgcn_wave_barrier();
    // Tile rows are contiguous in HBM: copy out 1 KB per instruction.
    bf16* obase = Oh + (int64_t)tile * 32 * D;
#pragma unroll
    for (int i = 0; i < (kOutChunks + kWave - 1) / kWave; ++i) {
      const int ch = i * kWave + lane;
      if (ch < valid_chunks) {
        const uint4 w = *reinterpret_cast<const uint4*>(&ost[ch * 8]);
        *reinterpret_cast<uint4*>(obase + ch * 8) = w;
        if constexpr (DIFF) {
          const uint4 pw = pv[i];
          dsum += sqdiff_bf16x2(w.x, pw.x) + sqdiff_bf16x2(w.y, pw.y) + sqdiff_bf16x2(w.z, pw.z) +
                  sqdiff_bf16x2(w.w, pw.w);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  // This wave's tiles: t_begin + wave, + 4, + 8, ...; tile k of the wave
  // sits in stage k % 2, and the next tile's loads run while one computes.
  // vmcnt accounting: after the loads of tile k come the stores of tile k-1
  // (NOST instructions, always a full tile) and the loads of tile k+1 (QJ).
  // A wave's vector-memory loads and stores share one counter here and
  // retire in issue order (the compiler's own waitcnt model for targets
  // without a separate store counter assumes the same), so at most
  // NOST + QJ outstanding means every load of tile k has landed.
  const uint32_t st0 = (uint32_t)(uintptr_t)LDS_PTR(void, qstage[wave][0]);
  const uint32_t st1 = (uint32_t)(uintptr_t)LDS_PTR(void, qstage[wave][1]);
  const int first = t_begin + wave;
  const int n = first < t_end ? (t_end - first + kWaves - 1) / kWaves : 0;
  if (n > 0) issue_tile(Qh, first, st0);
  for (int k = 0; k < n; ++k) {
    const int tile = first + k * kWaves;
    const bool more = k + 1 < n;
    if (more) issue_tile(Qh, tile + kWaves, (k & 1) ? st0 : st1);
    if (k >= 1) {
      if (more) wait_vmcnt<G::NOST + QJ>(); else wait_vmcnt<G::NOST>();
    } else {
      if (more) wait_vmcnt<QJ>(); else wait_vmcnt<0>();
    }
    compute(qstage[wave][k & 1], tile);
  }
  if (DIFF) {
    __syncthreads();  // every wave is done with its ring: reuse it for the sum
    const double s = block_sum_f64<kWaves>(dsum, reinterpret_cast<double*>(&qstage[0][0][0]));
    if (tid == 0) partials[blockIdx.x] = s;
  }
}

template <int D, int NKB, bool DIFF>
hipError_t launch_dk(const void* q, const void* kt, const void* vt, void* o, int64_t nbh,
                     int64_t nq, int L, int Lrows, float c, const DiffOut& diff,
                     hipStream_t stream) {
  // Size the grid to whole waves of resident blocks (as many per CU as the
  // LDS allows, at most 2, on 256 CUs): each (b, h) gets the same number of
  // blocks, as many as keep the grid within the fewest waves that leave at
  // most 96 query tiles per block (the text K/V load is amortized over them).
  using G = Geo<D, NKB>;
  constexpr int kPerCu = G::PER_CU;
  const int64_t ntiles = (nq + 31) / 32;
  const int64_t wave_blocks = 256 * kPerCu;
  int64_t blocks_per_bh = 1;
  if (nbh < wave_blocks) {
    for (int64_t m = 1;; ++m) {
      blocks_per_bh = (m * wave_blocks) / nbh;
      if (blocks_per_bh >= ntiles || (ntiles + blocks_per_bh - 1) / blocks_per_bh <= 96) break;
    }
  }
  if (blocks_per_bh > ntiles) blocks_per_bh = ntiles;
  const int64_t tiles_per_block = (ntiles + blocks_per_bh - 1) / blocks_per_bh;
  blocks_per_bh = (ntiles + tiles_per_block - 1) / tiles_per_block;
  const int64_t nblocks = blocks_per_bh * nbh;
  if (nblocks > 0x7fffffff || ntiles > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (DIFF) {
    if (nblocks > diff.capacity) return hipErrorInvalidConfiguration;  // caller checks first
    *diff.nparts = (int)nblocks;
  }
  hipLaunchKernelGGL((cross_kernel<D, NKB, DIFF>), dim3((unsigned)nblocks), dim3(kThreads), 0,
                     stream, (const bf16*)q, (const bf16*)kt, (const bf16*)vt, (bf16*)o, nq, L,
                     Lrows, (int)tiles_per_block, (int)blocks_per_bh, (int)nblocks, c,
                     DIFF ? (const bf16*)diff.prev : nullptr, DIFF ? diff.partials : nullptr);
  return hipGetLastError();
}

template <int D, bool DIFF>
hipError_t launch_dd(const void* q, const void* kt, const void* vt, void* o, int64_t nbh,
                     int64_t nq, int L, int Lrows, float c, const DiffOut& diff,
                     hipStream_t stream) {
  if (L <= 32) return launch_dk<D, 1, DIFF>(q, kt, vt, o, nbh, nq, L, Lrows, c, diff, stream);
  if (L <= 64) return launch_dk<D, 2, DIFF>(q, kt, vt, o, nbh, nq, L, Lrows, c, diff, stream);
  return launch_dk<D, 4, DIFF>(q, kt, vt, o, nbh, nq, L, Lrows, c, diff, stream);
}

// The fused difference needs one partial per block: at most the blocks of
// the grid, which launch_dk sizes to at most ntiles per (b, h); it takes no
// LDS beyond the plain kernel's.
template <int D>
hipError_t launch_d(const void* q, const void* kt, const void* vt, void* o, int64_t nbh, int64_t nq,
                    int L, int Lrows, float c, const DiffOut& diff, hipStream_t stream) {
  const int64_t max_blocks = nbh * ((nq + 31) / 32);
  if (diff.prev && diff.nparts && max_blocks <= diff.capacity)
    return launch_dd<D, true>(q, kt, vt, o, nbh, nq, L, Lrows, c, diff, stream);
  return launch_dd<D, false>(q, kt, vt, o, nbh, nq, L, Lrows, c, diff, stream);
}

}  // namespace

hipError_t launch_cross_bf16(const void* q, const void* kt, const void* vt, void* o, int64_t nbh,
                             int64_t nq, int L, int Lrows, int D, float scale,
                             const DiffOut& diff, hipStream_t stream) {
  const float c = scale * kLog2e;
  switch (D) {
#define PAB_CASE(d) \
  case d:           \
    return launch_d<d>(q, kt, vt, o, nbh, nq, L, Lrows, c, diff, stream);
    PAB_CASE(8) PAB_CASE(16) PAB_CASE(24) PAB_CASE(32) PAB_CASE(40) PAB_CASE(48) PAB_CASE(56)
    PAB_CASE(64) PAB_CASE(72) PAB_CASE(80) PAB_CASE(88) PAB_CASE(96) PAB_CASE(104) PAB_CASE(112)
    PAB_CASE(120) PAB_CASE(128)
#undef PAB_CASE
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace pab
