// spatial.hip -- bf16 spatial attention (PAB article, "Implementation",
// second observation: attention among the tokens of one frame), flash style
// on gfx950 MFMA.  Full-3D self-attention is the same kernel with F = 1.
//
// Per sequence (b, h, f) of S tokens: O = softmax(Q K^T * scale) V.
//
// Work split: a 256-thread block owns up to 256 query rows of one sequence,
// 64 per wave (two 32-row MFMA blocks, so every K and V operand read from LDS
// feeds two MFMAs; one block per wave for heads wider than 88).  A sequence's
// last block, when it holds at most 128 rows, gives each wave one 32-row
// block instead, so fewer of its waves sit idle.  Keys arrive
// in 64-row tiles through an LDS ring filled by direct global->LDS loads
// (global_load_lds_dwordx4): each tile is a whole number of 1 KiB wave-wide
// loads, dealt round-robin to the waves (every wave issues the same number;
// a wave short of a load repeats one, writing the same bytes), issued two
// tiles ahead (four-stage ring; three stages and one tile ahead where four
// would not leave room for two blocks per CU).  No registers are spent on
// staging.
//
// Each wave walks its keys in 32-key units and software-pipelines them so the
// matrix cores and the vector ALUs work at the same time: while the softmax of
// unit u (exponentials, bf16 packing) runs on the VALU, the MFMAs compute the
// scores of unit u+1 and then O^T += V^T P^T for unit u.
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16: a lane holds 16 scores of
//     ONE query row;
//   * the softmax needs no running maximum.  Softmax is unchanged by the
//     constant subtracted from a row's scores; it only has to keep exp() in
//     range.  Each row takes the maximum of its first 32 scores, plus 16
//     (log2 units) of headroom, and keeps it: every p = 2^(s c - m) then
//     stays finite unless a later score exceeds that first maximum by more
//     than about 100 (log2 units), far outside ordinary inputs.  The hot
//     loop thus holds no maximum, no rescale and no branch.  A wave whose
//     denominators or outputs come out non-finite (the rare case) recomputes
//     its rows exactly: a two-pass fp32 softmax per row, straight from HBM;
//   * O^T += V^T P^T: the V^T operand comes straight from the row-major V
//     tile through ds_read_b64_tr_b16 (transposing LDS read).  Operand row D
//     (a padding row of the last output block) is set to ones, so O^T row D
//     accumulates sum_j p_ij -- the softmax denominator, over exactly the
//     bf16-rounded p that multiply V -- on the MFMA.  Rows 0..D are covered
//     by whole 32-row blocks (v_mfma_f32_32x32x16_bf16) and, where row D
//     falls in the first 16 rows of the last block (D % 32 of 0 or 8, e.g.
//     D = 64, 72), a 16-row tail on v_mfma_f32_16x16x32_bf16 over all 32 keys
//     of a unit, whose P^T operand is the unit's bf16 P regrouped by
//     v_permlane16_swap: 16 output rows instead of 32 for the last block.
// Blocks are remapped so that the query tiles of one sequence share an XCD
// (and its L2), where the sequence's K and V stay resident.
// With a previous output P (the attention difference of PAB's Figure 1), the
// output pass also reads P beside its stores and each block writes the fp64
// sum of squared differences of the stored values.
#include <type_traits>

#include "device.hpp"
#include "launch.hpp"

namespace pab {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kBN = 64;                  // keys per LDS tile
constexpr int kLds = 160 * 1024;         // LDS bytes per CU
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kHeadroom = 16.0f;       // reference max above the first unit's (log2 units)

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
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
  // Output rows 0..D (data and the denominator): whole 32-row blocks, and a
  // 16-row tail from row TR0 where row D lies in its first 16 rows.
  static constexpr bool T16 = (D % 32) == 0 || (D % 32) == 8;
  static constexpr int NB = T16 ? D / 32 : D / 32 + 1;  // 32-row blocks of O^T
  static constexpr int TR0 = 32 * (D / 32);
  static constexpr int DCH = D / 8;                 // 16-byte chunks of data per row
  // K rows: an odd number of 16-byte chunks keeps the 32 rows of one MFMA
  // operand read on distinct banks.
  static constexpr int KS = (DCH % 2) ? D : D + 8;
  static constexpr int KCH = KS / 8;
  // V rows: data padded to a stride that keeps the transposing reads
  // conflict-free.
  static constexpr int VS = tr_stride(D);
  static constexpr int VCH = VS / 8;
  // A stage is the K rows, then the V rows, then slack.  A tile is NJ
  // wave-wide direct loads of 1 KiB (64 rows x KCH chunks = KCH loads for K,
  // VCH for V); load j fills stage bytes [1024 j, +1024).
  static constexpr int KREG = kBN * KS;             // elements
  static constexpr int VREG = kBN * VS;
  static constexpr int NJ = KCH + VCH;
  static constexpr int NJW = (NJ + kWaves - 1) / kWaves;  // loads per wave per tile
  // Transposing reads of V past the last data column (operand rows > D, whose
  // products are discarded) may run past the V rows into this slack.
  static constexpr int VSLACK = 64;
  static constexpr int STAGE = KREG + VREG + VSLACK;
  static constexpr int NST = (2 * 4 * STAGE * 2 <= kLds) ? 4 : 3;  // ring depth
  // Without a tail the last 32-row O^T block holds row D (the denominator)
  // and data rows; with the tail, every 32-row block is data.  The tail's
  // V^T operand is read only when it holds data rows (D % 32 == 8).
  static constexpr bool LAST_READ = T16 || (NB - 1) * 32 < D;
  static constexpr bool TAIL_READ = T16 && (D % 32) == 8;
  // K over-reads (d >= D, multiplied by Q's zero padding) must hit finite
  // data: past the last K row they land in the V rows of the same stage.
  static_assert((kBN - 1) * KS + ND * 16 <= KREG + VREG, "K over-read must stay in loaded rows");
  static_assert((kBN - 1) * VS + NB * 32 <= VREG + VSLACK, "V over-read must stay in the stage");
  static_assert(!TAIL_READ || (kBN - 1) * VS + TR0 + 16 <= VREG + VSLACK,
                "tail over-read must stay in the stage");
  static_assert(NST * STAGE * 2 <= kLds, "LDS ring too large");
  static constexpr int PER_CU = 2 * NST * STAGE * 2 <= kLds ? 2 : 1;  // resident blocks
  static_assert(2 * 32 * QB * D * 2 <= STAGE * 2, "two waves' output rows fit one stage");
  static_assert((NST - 2) * NJW < 64, "vmcnt budget");
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

// Finite test on the exponent bits (the file is compiled assuming no NaN,
// which would let a floating-point test fold away).
__device__ __forceinline__ bool finite(float x) {
  return (__builtin_bit_cast(uint32_t, x) & 0x7F800000u) != 0x7F800000u;
}

template <int D>
__global__ __launch_bounds__(kThreads, Geo<D>::PER_CU) void spatial_kernel(const bf16* __restrict__ Q,
                                                             const bf16* __restrict__ K,
                                                             const bf16* __restrict__ V,
                                                             bf16* __restrict__ O, int S, int nqt,
                                                             int nblocks, float c,
                                                             const bf16* __restrict__ P,
                                                             double* __restrict__ partials) {
  using G = Geo<D>;
  __shared__ __attribute__((aligned(16))) bf16 ring[G::NST * G::STAGE];

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
  // P (optional): the previous output of the same call, for the attention
  // difference -- each block adds up (O - P)^2 over the elements it writes.
  const bf16* __restrict__ Ps = P ? P + base : nullptr;
  double dsum = 0.0;

  // Direct-load plan of this wave: loads j = wave + 4i; a wave whose last
  // j is past the tile repeats load j - NJ instead (the same bytes to the
  // same place), so every wave issues NJW loads per tile.  Load j covers
  // stage slots 64 j .. 64 j + 63; slot s of the K (V) rows is chunk
  // (row, ch) = (s / KCH, s % KCH) (V: VCH).  Pad chunks (ch >= D/8) re-read
  // chunk 0 of the tile: finite values that nothing uses.  Byte offsets are
  // relative to the tile's first row.
  auto load_j = [&](int i) {  // wave-uniform
    const int j0 = wave + kWaves * i;
    return j0 < G::NJ ? j0 : j0 - G::NJ;
  };
  auto load_slot = [&](int j, int& row, int& ch) {
    const bool is_k = j < G::KCH;
    const int cs = is_k ? G::KCH : G::VCH;
    const int s = (is_k ? j : j - G::KCH) * kWave + lane;
    row = s / cs;
    ch = s % cs;
  };
  uint32_t joff[G::NJW];
#pragma unroll
  for (int i = 0; i < G::NJW; ++i) {
    int row, ch;
    load_slot(load_j(i), row, ch);
    joff[i] = (ch < G::DCH) ? (uint32_t)((row * D + ch * 8) * 2) : 0u;
  }
  const uint32_t ring_lds = (uint32_t)(uintptr_t)LDS_PTR(void, ring);
  const int nt = (S + kBN - 1) / kBN;
  auto stage_base = [&](int t) -> uint32_t {
    return ring_lds + (uint32_t)((t % G::NST) * G::STAGE * 2);
  };
  auto issue = [&](int t, auto full_known) {
    const int key0 = t * kBN;
    const uint32_t st = stage_base(t);
    if (decltype(full_known)::value || key0 + kBN <= S) {
      const bf16* kt = Ks + (size_t)key0 * D;
      const bf16* vt = Vs + (size_t)key0 * D;
#pragma unroll
      for (int i = 0; i < G::NJW; ++i) {
        const int j = load_j(i);
        dma16(j < G::KCH ? kt : vt, joff[i], st + (uint32_t)(j * 1024));
      }
    } else {
      // Ragged last tile: rows past S repeat row S-1 (finite; their scores
      // are masked and their p are 0).
#pragma unroll
      for (int i = 0; i < G::NJW; ++i) {
        const int j = load_j(i);
        int row, ch;
        load_slot(j, row, ch);
        const int r = min(key0 + row, S - 1);
        const uint32_t off = (ch < G::DCH) ? (uint32_t)((r * D + ch * 8) * 2) : 0u;
        dma16(j < G::KCH ? Ks : Vs, off, st + (uint32_t)(j * 1024));
      }
    }
  };
  // The previous output P (attention difference) with a four-stage ring:
  // once the last tile is synchronized, stages nt and nt+1 (mod 4) are
  // never refilled and every wave is done reading them (the scores taken
  // after the last unit read stage nt, but are discarded), so each wave
  // brings its own rows of P into half of one of them by direct loads,
  // under the last tile's work.  A wave reads back only what it loaded.
  int prow0 = 0, prows = 0;  // this wave's query rows (set by run)
  auto prev_lds = [&]() -> uint32_t {
    return stage_base(nt + (wave >> 1)) + (uint32_t)((wave & 1) * prows * D * 2);
  };
  auto issue_prev = [&]() {
    if (prow0 >= S) return;
    const uint32_t bytes = (uint32_t)(prows * D * 2);
    const uint32_t valid = (uint32_t)(min(prows, S - prow0) * D * 2);
    // The base goes to scalar registers; each half is taken as an unsigned
    // 32-bit value (readfirstlane returns int: widening it directly would
    // sign-extend the low half).
    const uint64_t pa = (uint64_t)(uintptr_t)(Ps + (size_t)prow0 * D);
    const uint32_t plo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)pa);
    const uint32_t phi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(pa >> 32));
    const bf16* pb = (const bf16*)(uintptr_t)(((uint64_t)phi << 32) | (uint64_t)plo);
    const uint32_t dst = prev_lds();
    for (uint32_t j = 0; j * 1024 < bytes; ++j) {
      const uint32_t pos = j * 1024 + (uint32_t)lane * 16;
      // Rows past S re-read the last valid 16 bytes; lanes past the rows idle.
      if (pos < bytes) dma16(pb, min(pos, valid - 16u), dst + j * 1024);
    }
  };
  // Barrier B_t: tile t has landed and is visible to every wave; the stage
  // read last by unit 2t-3 is free again and is refilled with the tile
  // NST-2 ahead.  `steady`: that tile is known to exist and to be whole (so
  // is tile t+1), which the main loop guarantees; else both are checked.
  auto sync_tile = [&](int t, auto steady) {
    constexpr bool kSteady = decltype(steady)::value;
    if (G::NST == 4 && (kSteady || t + 1 < nt)) {  // tile t+1 may still be in flight
      wait_vmcnt<G::NJW>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
    if constexpr (kSteady) {
      issue(t + G::NST - 2, std::true_type{});
    } else {
      if (t + G::NST - 2 < nt) issue(t + G::NST - 2, std::false_type{});
    }
  };

  // The work of one block for QBX 32-row query blocks per wave.
  auto run = [&](auto qbx) __attribute__((always_inline)) {
    constexpr int QBX = decltype(qbx)::value;
    // This wave's query rows as the B operand (Q^T), resident in registers.
    const int qrow0 = qt * G::BM + wave * 32 * QBX;
    const bool wave_live = qrow0 < S;
    prow0 = qrow0;
    prows = 32 * QBX;
    bf16x8 qreg[QBX][G::ND];
#pragma unroll
    for (int qb = 0; qb < QBX; ++qb) {
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

    issue(0, std::false_type{});
    if (G::NST == 4 && nt > 1) issue(1, std::false_type{});

    if (!wave_live) {
      // Idle waves still fetch their share of every tile.
      for (int t = 0; t < nt; ++t) sync_tile(t, std::false_type{});
      return;
    }

    // Per-lane LDS offsets of the operand reads; the rest of each address is a
    // compile-time offset.  Transposing V read: lane j of a 16-lane group
    // addresses row j/4 and columns 4*(j%4)..+3 of a 4x16 block and receives
    // column j, i.e. V^T row d = l32 of the operand.
    const int g16 = lane >> 4, j16 = lane & 15;
    const uint32_t klane = (uint32_t)((l32 * G::KS + h * 8) * 2);
    const uint32_t vlane = (uint32_t)((G::KREG + (h * 4 + (j16 >> 2)) * G::VS + (g16 & 1) * 16 +
                                       (j16 & 3) * 4) * 2);
    // Operand row D of V^T (the ones row) lives in lane D % 32 of block D / 32
    // (no tail), or in lane D % 32 of every 16-lane group of the tail operand.
    const bool ones_lane = l32 == (D % 32);
    const uint32_t ones_word = ones_lane ? 0x3F803F80u : 0u;
    // Tail operand (v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8(l/16)+e],
    // B[8(l/16)+e][l%16] and receives D[4(l/16)+i][l%16]): V^T rows TR0 + j16
    // over the keys of lane group g16 = the keys its regrouped P holds, two
    // runs of four, base + {0..3} and base + {8..11} with base = 0, 16, 4, 20
    // for g16 = 0..3.
    const uint32_t tlane = (uint32_t)((G::KREG + ((g16 & 1) * 16 + (g16 >> 1) * 4 + (j16 >> 2)) * G::VS +
                                       G::TR0 + (j16 & 3) * 4) * 2);
    const bool tail_ones = j16 == (D % 32);

    f32x16 oacc[QBX][G::NB];
#pragma unroll
    for (int qb = 0; qb < QBX; ++qb)
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb) oacc[qb][nb] = zero16();
    f32x4 tacc[QBX][2];  // the 16-row tail, queries 0..15 and 16..31 of each block
#pragma unroll
    for (int qb = 0; qb < QBX; ++qb) tacc[qb][0] = tacc[qb][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    float mrow[QBX];  // reference max per row (log2 domain, score * c), fixed

    // S^T block of the 32 keys at row kb*32 of the stage whose K rows `kaddr`
    // points into (per-lane offset included).
    auto qk = [&](uint32_t kaddr, int kb, f32x16 (&s)[QBX]) __attribute__((always_inline)) {
#pragma unroll
      for (int qb = 0; qb < QBX; ++qb) s[qb] = zero16();
#pragma unroll
      for (int ds = 0; ds < G::ND; ++ds) {
        const bf16x8 a = *LDS_PTR(const bf16x8, kaddr + (uint32_t)((kb * 32 * G::KS + ds * 16) * 2));
#pragma unroll
        for (int qb = 0; qb < QBX; ++qb) s[qb] = mfma32(a, qreg[qb][ds], s[qb]);
      }
    };
    // Keys >= S do not exist.
    auto mask = [&](f32x16 (&s)[QBX], int key_first) __attribute__((always_inline)) {
#pragma unroll
      for (int qb = 0; qb < QBX; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (key_first + acc_row(r, h) >= S) s[qb][r] = -INFINITY;
    };
    // P^T operand (bf16) of scores r0..r0+7 (r0 = 8*t2): 16 keys per lane half.
    auto probs = [&](const f32x16 (&s)[QBX], int t2, bf16x8 (&pb)[QBX]) __attribute__((always_inline)) {
#pragma unroll
      for (int qb = 0; qb < QBX; ++qb) {
        const float negm = -mrow[qb];
        const int r0 = t2 * 8;
        pb[qb] = to_bf16x8(
            fast_exp2(fmaf(s[qb][r0 + 0], c, negm)), fast_exp2(fmaf(s[qb][r0 + 1], c, negm)),
            fast_exp2(fmaf(s[qb][r0 + 2], c, negm)), fast_exp2(fmaf(s[qb][r0 + 3], c, negm)),
            fast_exp2(fmaf(s[qb][r0 + 4], c, negm)), fast_exp2(fmaf(s[qb][r0 + 5], c, negm)),
            fast_exp2(fmaf(s[qb][r0 + 6], c, negm)), fast_exp2(fmaf(s[qb][r0 + 7], c, negm)));
      }
    };
    // O^T += V^T P^T over keys kb*32 + 16*t2 .. +15 of the stage whose V rows
    // `vaddr` points into (per-lane offset included).
    auto pv = [&](uint32_t vaddr, int kb, int t2, const bf16x8 (&pb)[QBX]) __attribute__((always_inline)) {
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb) {
        bf16x8 a;
        if (nb < G::NB - 1 || G::LAST_READ) {
          const uint32_t p = vaddr + (uint32_t)(((kb * 32 + t2 * 16) * G::VS + nb * 32) * 2);
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p + 8 * G::VS * 2));
          a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          if (!G::T16 && nb == G::NB - 1) {  // rows > D are don't-care; row D must be ones
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
        for (int qb = 0; qb < QBX; ++qb) oacc[qb][nb] = mfma32(a, pb[qb], oacc[qb][nb]);
      }
    };
    // The 16-row tail over all 32 keys of a unit (keys kb*32.. of the stage
    // whose tail rows `taddr` points into): the P^T operand of queries 0..15
    // and 16..31 of each block is the unit's two bf16 P operands regrouped by
    // v_permlane16_swap (rows 1 and 3 of one swapped with rows 0 and 2 of the
    // other), which puts each query's 32 keys into the four lane groups.
    auto tail = [&](uint32_t taddr, int kb, const bf16x8 (&pa)[QBX], const bf16x8 (&pb)[QBX])
        __attribute__((always_inline)) {
      if constexpr (G::T16) {
        uint4 w;
        if constexpr (G::TAIL_READ) {
          const uint32_t p = taddr + (uint32_t)(kb * 32 * G::VS * 2);
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, p + 8 * G::VS * 2));
          w = __builtin_bit_cast(uint4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          w.x = tail_ones ? 0x3F803F80u : w.x;
          w.y = tail_ones ? 0x3F803F80u : w.y;
          w.z = tail_ones ? 0x3F803F80u : w.z;
          w.w = tail_ones ? 0x3F803F80u : w.w;
        } else {  // no data rows: every row ones
          w = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
        }
        const bf16x8 a = __builtin_bit_cast(bf16x8, w);
#pragma unroll
        for (int qb = 0; qb < QBX; ++qb) {
          uint4 x = __builtin_bit_cast(uint4, pa[qb]), y = __builtin_bit_cast(uint4, pb[qb]);
          auto r0 = __builtin_amdgcn_permlane16_swap(x.x, y.x, false, false);
          auto r1 = __builtin_amdgcn_permlane16_swap(x.y, y.y, false, false);
          auto r2 = __builtin_amdgcn_permlane16_swap(x.z, y.z, false, false);
          auto r3 = __builtin_amdgcn_permlane16_swap(x.w, y.w, false, false);
          x = make_uint4(r0[0], r1[0], r2[0], r3[0]);
          y = make_uint4(r0[1], r1[1], r2[1], r3[1]);
          tacc[qb][0] = mfma16(a, __builtin_bit_cast(bf16x8, x), tacc[qb][0]);
          tacc[qb][1] = mfma16(a, __builtin_bit_cast(bf16x8, y), tacc[qb][1]);
        }
      }
    };
    // One pipelined unit: softmax and PV of the current unit (scores `sc`, V at
    // row kb_cur*32 of `v_cur`) around the QK of the next unit (K at row
    // kb_next*32 of `k_next`, scores into `sn`).  With `masked`, keys of the
    // next unit from S on are masked (only the last tile has such keys).
    auto unit = [&](auto masked, uint32_t k_next, int kb_next, int key_next, uint32_t v_cur,
                    uint32_t t_cur, int kb_cur, const f32x16 (&sc)[QBX], f32x16 (&sn)[QBX])
        __attribute__((always_inline)) {
      bf16x8 p0[QBX], p1[QBX];
      qk(k_next, kb_next, sn);
      probs(sc, 0, p0);
      pv(v_cur, kb_cur, 0, p0);
      probs(sc, 1, p1);
      pv(v_cur, kb_cur, 1, p1);
      tail(t_cur, kb_cur, p0, p1);
      if constexpr (decltype(masked)::value) mask(sn, key_next);
    };

    f32x16 sA[QBX], sB[QBX];

    sync_tile(0, std::false_type{});
    {
      const uint32_t st = stage_base(0);
      qk(opaque(st + klane), 0, sA);
      if (S < 32) mask(sA, 0);
      // Reference max: the first unit's row max (the other half-wave holds
      // the other 16 keys of the row), plus headroom.
#pragma unroll
      for (int qb = 0; qb < QBX; ++qb) {
        float m = sA[qb][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) m = fmaxf(m, sA[qb][r]);
        mrow[qb] = max_halves(m) * c + kHeadroom;
      }
    }

    // One tile per iteration: units 2t (scores in sA) and 2t+1, each with the
    // QK of the unit after it underneath.  While both of those units have all
    // 32 keys below S the iteration needs no masking; while the tile NST-2
    // ahead of the next is whole, its loads need no check either and the
    // iteration is one basic block.
    const int UF = S / 32;   // units with all 32 keys present
    int t = 0;
    auto tile = [&](auto steady) __attribute__((always_inline)) {
      const uint32_t cur = stage_base(t);
      const uint32_t kc = opaque(cur + klane), vc = opaque(cur + vlane);
      const uint32_t tc = G::TAIL_READ ? opaque(cur + tlane) : 0u;
      unit(std::false_type{}, kc, 1, 0, vc, tc, 0, sA, sB);
      sync_tile(t + 1, steady);
      const uint32_t kn = opaque(stage_base(t + 1) + klane);
      unit(std::false_type{}, kn, 0, 0, vc, tc, 1, sB, sA);
    };
    for (; 2 * t + 2 < UF && (t + G::NST) * kBN <= S; ++t) tile(std::true_type{});
    for (; 2 * t + 2 < UF; ++t) tile(std::false_type{});
    // The last tiles, masked.  A unit entirely past S (the second unit of the
    // last tile when S % 64 is 1..32) has all p exactly 0 and changes
    // nothing; the QK after the last unit runs on stale but in-bounds LDS and
    // is dropped.  The previous output (attention difference) is fetched
    // once the last tile is synchronized: here, in the last one or two
    // tiles, so the hot loop above carries none of it.
    const int t_tail = t;
    for (; t < nt; ++t) {
      if constexpr (G::NST == 4) {
        if (Ps && t == nt - 1 && t == t_tail) issue_prev();  // synchronized before the tail
      }
      const uint32_t cur = stage_base(t);
      const uint32_t kc = opaque(cur + klane), vc = opaque(cur + vlane);
      const uint32_t tc = G::TAIL_READ ? opaque(cur + tlane) : 0u;
      unit(std::true_type{}, kc, 1, (2 * t + 1) * 32, vc, tc, 0, sA, sB);
      if (t + 1 < nt) {
        sync_tile(t + 1, std::false_type{});
        if constexpr (G::NST == 4) {
          if (Ps && t + 1 == nt - 1) issue_prev();
        }
      }
      const uint32_t kn = opaque(stage_base(t + 1) + klane);
      unit(std::true_type{}, kn, 0, (2 * t + 2) * 32, vc, tc, 1, sB, sA);
    }

    // Denominators (row D of O^T) and the check that the reference max kept
    // every value finite: data rows and the denominator of every row of the
    // wave.  Otherwise the whole wave's rows are recomputed exactly below.
    // With the tail, the denominator of query half*16 + n of a block is tail
    // row D % 32 of lane 32 + n (rows 8.. of the tail sit in lanes 32..63;
    // with no data rows every tail row is the denominator); each lane fetches
    // those of its own query (l32) and of the tail rows it stores.
    float inv[QBX];
    float tinv[QBX][2];
    bool bad = false;
#pragma unroll
    for (int qb = 0; qb < QBX; ++qb) {
      float l;
      if constexpr (G::T16) {
        const int src = (32 + (lane & 15)) * 4;
        const float l0 = __builtin_bit_cast(
            float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, tacc[qb][0][0])));
        const float l1 = __builtin_bit_cast(
            float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, tacc[qb][1][0])));
        l = l32 < 16 ? l0 : l1;
        tinv[qb][0] = 1.f / l0;
        tinv[qb][1] = 1.f / l1;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (4 * (lane >> 4) + i < D % 32) bad |= !finite(tacc[qb][hf][i]);
      } else {
        const HalfPair pr = half_pair(oacc[qb][G::NBD][G::RD]);
        l = G::HD == 0 ? pr.lo : pr.hi;
      }
      bad |= !(finite(l) && l > 0.f);
      inv[qb] = 1.f / l;
#pragma unroll
      for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (nb * 32 + acc_row(r, 0) < D) bad |= !finite(oacc[qb][nb][r]);
    }
    if (__builtin_amdgcn_ballot_w64(bad) != 0) {
      // Exact recompute of this wave's rows, one row per lane: two passes
      // over the keys in HBM (row max, then the weighted sums) in fp32.
      if constexpr (G::NST == 4) {
        wait_vmcnt<0>();  // the previous output's loads into the ring are done
      }
      const int row = qrow0 + lane;
      if (lane < 32 * QBX && row < S) {
        float q[D];
#pragma unroll
        for (int d = 0; d < D; d += 8) {
          const bf16x8 w = *reinterpret_cast<const bf16x8*>(Qs + (size_t)row * D + d);
#pragma unroll
          for (int e = 0; e < 8; ++e) q[d + e] = (float)w[e];
        }
        auto score = [&](int j) {
          float s = 0.f;
#pragma unroll
          for (int d = 0; d < D; d += 8) {
            const bf16x8 w = *reinterpret_cast<const bf16x8*>(Ks + (size_t)j * D + d);
#pragma unroll
            for (int e = 0; e < 8; ++e) s = fmaf(q[d + e], (float)w[e], s);
          }
          return s * c;
        };
        float m = -INFINITY;
        for (int j = 0; j < S; ++j) m = fmaxf(m, score(j));
        float acc[D];
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] = 0.f;
        float l = 0.f;
        for (int j = 0; j < S; ++j) {
          const float p = fast_exp2(score(j) - m);
          l += p;
#pragma unroll
          for (int d = 0; d < D; d += 8) {
            const bf16x8 w = *reinterpret_cast<const bf16x8*>(Vs + (size_t)j * D + d);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[d + e] = fmaf(p, (float)w[e], acc[d + e]);
          }
        }
        const float il = 1.f / l;
        bf16* orow = Os + (size_t)row * D;
#pragma unroll
        for (int d = 0; d < D; d += 4) {
          const uint2 w = make_uint2(pack_bf16x2(acc[d] * il, acc[d + 1] * il),
                                     pack_bf16x2(acc[d + 2] * il, acc[d + 3] * il));
          *reinterpret_cast<uint2*>(orow + d) = w;
          if (Ps) {
            const uint2 pw = *reinterpret_cast<const uint2*>(Ps + (size_t)row * D + d);
            dsum += sqdiff_bf16x2(w.x, pw.x) + sqdiff_bf16x2(w.y, pw.y);
          }
        }
      }
      return;
    }

    // The output rows, normalized by the denominator in row D of O^T.
    auto out_word = [&](int qb, int nb, int g, float iv) __attribute__((always_inline)) {
      return make_uint2(pack_bf16x2(oacc[qb][nb][g * 4 + 0] * iv, oacc[qb][nb][g * 4 + 1] * iv),
                        pack_bf16x2(oacc[qb][nb][g * 4 + 2] * iv, oacc[qb][nb][g * 4 + 3] * iv));
    };
    if (Ps) {
      // Attention difference against the previous output: from LDS where the
      // ring brought it in, else from HBM with every word requested before
      // the first is used (one load latency per block, not one per word).
      uint2 pw[QBX][G::NB][4];
      if constexpr (G::NST == 4) {
        wait_vmcnt<0>();
        asm volatile("" ::: "memory");
      }
#pragma unroll
      for (int qb = 0; qb < QBX; ++qb) {
        const int qrow = qrow0 + qb * 32 + l32;
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int d0 = nb * 32 + g * 8 + h * 4;
            pw[qb][nb][g] = make_uint2(0u, 0u);
            if (d0 < D && qrow < S) {
              if constexpr (G::NST == 4) {
                const u32x2 t2 =
                    *LDS_PTR(const u32x2, prev_lds() + (uint32_t)(((qb * 32 + l32) * D + d0) * 2));
                pw[qb][nb][g] = make_uint2(t2.x, t2.y);
              } else {
                pw[qb][nb][g] = *reinterpret_cast<const uint2*>(Ps + (size_t)qrow * D + d0);
              }
            }
          }
      }
#pragma unroll
      for (int qb = 0; qb < QBX; ++qb) {
        const int qrow = qrow0 + qb * 32 + l32;
        if (qrow < S) {
          bf16* orow = Os + (size_t)qrow * D;
#pragma unroll
          for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int d0 = nb * 32 + g * 8 + h * 4;
              if (d0 < D) {
                const uint2 w = out_word(qb, nb, g, inv[qb]);
                *reinterpret_cast<uint2*>(orow + d0) = w;
                dsum += sqdiff_bf16x2(w.x, pw[qb][nb][g].x) + sqdiff_bf16x2(w.y, pw[qb][nb][g].y);
              }
            }
        }
      }
      if constexpr (G::TAIL_READ) {
        // Tail data rows TR0 + 4*(lane/16) .. +3 (lanes 0..31), one query
        // of each half per lane.
        if (lane < 32) {
          const int d0 = G::TR0 + 4 * (lane >> 4);
#pragma unroll
          for (int qb = 0; qb < QBX; ++qb)
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
              const int qi = qb * 32 + hf * 16 + (lane & 15);
              const int qrow = qrow0 + qi;
              if (qrow < S) {
                uint2 p;
                if constexpr (G::NST == 4) {
                  const u32x2 t2 = *LDS_PTR(const u32x2, prev_lds() + (uint32_t)((qi * D + d0) * 2));
                  p = make_uint2(t2.x, t2.y);
                } else {
                  p = *reinterpret_cast<const uint2*>(Ps + (size_t)qrow * D + d0);
                }
                const float iv = tinv[qb][hf];
                const uint2 w = make_uint2(pack_bf16x2(tacc[qb][hf][0] * iv, tacc[qb][hf][1] * iv),
                                           pack_bf16x2(tacc[qb][hf][2] * iv, tacc[qb][hf][3] * iv));
                *reinterpret_cast<uint2*>(Os + (size_t)qrow * D + d0) = w;
                dsum += sqdiff_bf16x2(w.x, p.x) + sqdiff_bf16x2(w.y, p.y);
              }
            }
        }
      }
      return;
    }
#pragma unroll
    for (int qb = 0; qb < QBX; ++qb) {
      const int qrow = qrow0 + qb * 32 + l32;
      if (qrow < S) {
        bf16* orow = Os + (size_t)qrow * D;
#pragma unroll
        for (int nb = 0; nb < G::NB; ++nb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int d0 = nb * 32 + g * 8 + h * 4;
            if (d0 < D) *reinterpret_cast<uint2*>(orow + d0) = out_word(qb, nb, g, inv[qb]);
          }
      }
    }
    if constexpr (G::TAIL_READ) {
      if (lane < 32) {
        const int d0 = G::TR0 + 4 * (lane >> 4);
#pragma unroll
        for (int qb = 0; qb < QBX; ++qb)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            const int qrow = qrow0 + qb * 32 + hf * 16 + (lane & 15);
            if (qrow < S) {
              const float iv = tinv[qb][hf];
              *reinterpret_cast<uint2*>(Os + (size_t)qrow * D + d0) =
                  make_uint2(pack_bf16x2(tacc[qb][hf][0] * iv, tacc[qb][hf][1] * iv),
                             pack_bf16x2(tacc[qb][hf][2] * iv, tacc[qb][hf][3] * iv));
            }
          }
      }
    }
  };

  // A sequence's last block usually holds fewer rows than the block covers;
  // when 32 rows per wave cover them, every wave takes one 32-row block
  // instead of leaving waves idle.
  bool narrow = false;
  if constexpr (G::QB == 2) narrow = S - qt * G::BM <= kWaves * 32;
  if (narrow) {
    run(std::integral_constant<int, 1>{});
  } else {
    run(std::integral_constant<int, G::QB>{});
  }
  if (Ps) {
    __syncthreads();  // every wave is done with the ring: reuse it for the sum
    const double s = block_sum_f64<kWaves>(dsum, reinterpret_cast<double*>(ring));
    if (tid == 0) partials[blockIdx.x] = s;
  }
}

template <int D>
hipError_t launch_d(const void* q, const void* k, const void* v, void* o, int64_t nseq, int S,
                    float c, const DiffOut& diff, hipStream_t stream) {
  const int nqt = (S + Geo<D>::BM - 1) / Geo<D>::BM;
  const int64_t nblocks = nseq * nqt;
  if (nblocks > 0x7fffffff) return hipErrorInvalidConfiguration;
  const bool fused = diff.prev && nblocks <= diff.capacity;
  if (diff.nparts) *diff.nparts = fused ? (int)nblocks : 0;
  hipLaunchKernelGGL(spatial_kernel<D>, dim3((unsigned)nblocks), dim3(kThreads), 0, stream,
                     (const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, S, nqt, (int)nblocks, c,
                     fused ? (const bf16*)diff.prev : nullptr, fused ? diff.partials : nullptr);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_spatial_bf16(const void* q, const void* k, const void* v, void* o, int64_t nseq,
                               int S, int D, float scale, const DiffOut& diff,
                               hipStream_t stream) {
  const float c = scale * kLog2e;
  switch (D) {
#define PAB_CASE(d) \
  case d:           \
    return launch_d<d>(q, k, v, o, nseq, S, c, diff, stream);
    PAB_CASE(8) PAB_CASE(16) PAB_CASE(24) PAB_CASE(32) PAB_CASE(40) PAB_CASE(48) PAB_CASE(56)
    PAB_CASE(64) PAB_CASE(72) PAB_CASE(80) PAB_CASE(88) PAB_CASE(96) PAB_CASE(104) PAB_CASE(112)
    PAB_CASE(120) PAB_CASE(128)
#undef PAB_CASE
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace pab
