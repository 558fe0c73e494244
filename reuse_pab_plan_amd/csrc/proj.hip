// proj.hip -- bf16 projections around an attention (PAB article,
// "Implementation": a broadcast step reuses the attention module's output,
// so the module's input projection and output projection are skipped with
// the attention).  Both are dense contractions on MFMA:
//
//   input projection   Y[m, j] = sum_k X[m, k] W[j, k]     X token-major [B*T, C],
//                      scattered to head-major tensors [B, H, F, S, D]
//                      (feature j = tensor j / C, head (j % C) / D, channel j % D)
//   output projection  Y[m, j] = sum_k O[m, k] W[j, k]     O gathered from the
//                      head-major attention output (k = h * D + d), Y token-major
//
// W has the layout of a linear layer's weight, [out_features, in_features], so
// both operands are contiguous along k and every MFMA operand is one 16-byte
// LDS read per lane.  The product is formed transposed (Y^T = W X^T on
// v_mfma_f32_32x32x16_bf16): a lane then holds one token's values for 16
// output features in runs of 4, which stage into LDS as row-major 8-byte
// pieces before lane-contiguous 16-byte stores.
//
// A 256-thread block computes a 256-token x 192-feature tile (each wave
// 128 x 96: 12 MFMA accumulators, one wave per SIMD).  k advances in steps
// of 64 through two LDS stages filled by direct global->LDS loads one step
// ahead (the output projection's loads gather 16-byte chunks from the head
// planes); within a step the operands of the next 16-wide k slice are read
// while the MFMAs of the current one run.  Blocks are ordered so that the feature tiles of one token
// tile run together on one XCD and share its L2.
#include "device.hpp"
#include "launch.hpp"

namespace pab {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kBM = 256;                 // tokens per block
constexpr int kBN = 192;                 // output features per block
constexpr int kBK = 64;                  // k per ring stage
constexpr int kKS = kBK + 8;             // LDS row stride (elements): 9 chunks, odd
constexpr int kKCH = kKS / 8;            // chunks per LDS row (the last is padding)
constexpr int kRows = kBM + kBN;         // token rows, then weight rows
constexpr int kStage = kRows * kKS;      // elements
constexpr int kNst = 2;
constexpr int kNJ = kRows * kKCH / kWave;          // wave-wide loads per stage (63)
constexpr int kNJW = (kNJ + kWaves - 1) / kWaves;  // per wave, at most (16)
constexpr int kWM = 128, kWN = 96;       // wave tile
constexpr int kMB = kWM / 32, kNB = kWN / 32;
constexpr int kOS = kWN + 8;             // epilogue staging row stride (elements)
static_assert(kRows * kKCH % kWave == 0, "loads cover whole stages");
static_assert(kBM * kKCH % kWave == 0, "no load straddles token and weight rows");
static_assert(kNst * kStage * 2 <= 160 * 1024, "LDS ring too large");
static_assert(kWaves * kWM * kOS <= kNst * kStage, "epilogue staging fits the ring");
static_assert(kNJW < 64, "vmcnt budget");

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// One 16-byte direct global->LDS load per lane: lane l of the wave reads
// global bytes [gbase + voff, +16) and writes LDS bytes [lds + 16*l, +16).
// `gbase` and `lds` must be wave-uniform.  Inline assembly, so the wait for
// it (s_waitcnt vmcnt) is placed by hand: the compiler does not track it.
__device__ __forceinline__ void dma16(const void* gbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(lds), "v"(voff), "s"(gbase)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

__device__ __forceinline__ const bf16* uniform_ptr(const bf16* p) {
  const uint64_t u = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const bf16*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

struct ProjArgs {
  const bf16* x;      // token-major input [M, K] (GATHER: head-major [B, H, T, D])
  const bf16* w;      // weight [N, K]
  bf16* out[3];       // SCATTER: head-major tensors; else out[0] token-major [M, N]
  int M, N, K;        // tokens, output features, input features
  int T, H, D;        // tokens per entry, heads, head dim
  int nbn;            // feature tiles
  int nblocks;
};

// GATHER: the input is a head-major attention output (output projection).
// SCATTER: the output goes to head-major tensors (input projection).
template <bool GATHER, bool SCATTER>
__global__ __launch_bounds__(kThreads, 1) void proj_kernel(ProjArgs p) {
  __shared__ __attribute__((aligned(16))) bf16 ring[kNst * kStage];

  const int tid = threadIdx.x;
  const int lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int logical = xcd_remap(blockIdx.x, p.nblocks);
  const int bm = logical / p.nbn, bn = logical % p.nbn;
  const int m0 = bm * kBM, n0 = bn * kBN;
  const int K = p.K;
  const int nkt = (K + kBK - 1) / kBK;

  // Direct-load plan: load j = wave + 4i covers stage slots 64 j .. 64 j + 63;
  // slot s is chunk s % 5 of stage row s / 5 (rows 0..255 tokens, 256..447
  // weight rows).  Chunk 4 is padding: its lanes load nothing.  Rows past the
  // matrix repeat its last row (finite, never stored).
  uint32_t base_off[kNJW];   // byte offset of the chunk, without the k-tile part
  uint32_t hd_row[kNJW];     // GATHER token rows: element offset of (b, t) in head 0
  bool live[kNJW];
#pragma unroll
  for (int i = 0; i < kNJW; ++i) {
    const int j = wave + kWaves * i;
    const int s = j * kWave + lane;
    const int row = s / kKCH, ch = s % kKCH;
    live[i] = j < kNJ && ch < kKCH - 1;
    if (row < kBM) {
      const int m = min(m0 + row, p.M - 1);
      if (GATHER) {
        const int b = m / p.T, t = m % p.T;
        hd_row[i] = (uint32_t)(((size_t)b * p.H * p.T + t) * p.D);
        base_off[i] = (uint32_t)(ch * 8);   // k within the tile
      } else {
        hd_row[i] = 0;
        base_off[i] = (uint32_t)(((size_t)m * K + ch * 8) * 2);
      }
    } else {
      const int n = min(n0 + row - kBM, p.N - 1);
      hd_row[i] = 0;
      base_off[i] = (uint32_t)(((size_t)n * K + ch * 8) * 2);
    }
  }
  const uint32_t ring_lds = (uint32_t)(uintptr_t)LDS_PTR(void, ring);
  const bf16* xbase = uniform_ptr(p.x);
  const bf16* wbase = uniform_ptr(p.w);
  auto issue = [&](int kt) {
    const int k0 = kt * kBK;
    const uint32_t st = ring_lds + (uint32_t)((kt % kNst) * kStage * 2);
    const bool ragged = k0 + kBK > K;  // the last step of a K that is not a multiple of 64
#pragma unroll
    for (int i = 0; i < kNJW; ++i) {
      const int j = wave + kWaves * i;
      if (i + 1 < kNJW || j < kNJ) {
        const uint32_t lds = st + (uint32_t)(j * 1024);
        if (ragged) {
          // Chunks past K hold zeros (written here, never loaded over).
          const int ch = (j * kWave + lane) % kKCH;
          if (ch < kKCH - 1 && k0 + ch * 8 >= K) {
            *LDS_PTR(u32x4, lds + (uint32_t)(lane * 16)) = u32x4{0u, 0u, 0u, 0u};
            continue;
          }
        }
        if (j * kWave < kBM * kKCH) {  // token rows (wave-uniform)
          uint32_t off;
          if (GATHER) {
            const int k = k0 + (int)base_off[i];
            const int hh = k / p.D, d = k - hh * p.D;
            off = (hd_row[i] + (uint32_t)(hh * p.T * p.D + d)) * 2u;
            if (live[i]) dma16(xbase, off, lds);
          } else {
            if (live[i]) dma16(xbase + k0, base_off[i], lds);
          }
        } else {
          if (live[i]) dma16(wbase + k0, base_off[i], lds);
        }
      }
    }
  };
  // Before stage kt is read: its loads have landed and every wave's loads
  // are visible; the other stage (read last in step kt-1) is then refilled
  // with step kt+1, which lands while step kt computes.
  auto sync_stage = [&](int kt) {
    wait_vmcnt<0>();
    __syncthreads();
    if (kt + 1 < nkt) issue(kt + 1);
  };

  // Wave tile: tokens wm*128.., features wn*96.. of the block tile.
  const int wm = wave & 1, wn = wave >> 1;
  const uint32_t xlane = (uint32_t)(((wm * kWM + l32) * kKS + h * 8) * 2);
  const uint32_t wlane = (uint32_t)(((kBM + wn * kWN + l32) * kKS + h * 8) * 2);

  f32x16 acc[kNB][kMB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) acc[nb][mb] = zero16();

  issue(0);
  for (int kt = 0; kt < nkt; ++kt) {
    sync_stage(kt);
    const uint32_t st = ring_lds + (uint32_t)((kt % kNst) * kStage * 2);
    // Operands of the next 16-wide k step are read while the MFMAs of the
    // current one run.
    bf16x8 wop[2][kNB], xop[2][kMB];
    auto load_ops = [&](int k16, bf16x8 (&wo)[kNB], bf16x8 (&xo)[kMB]) __attribute__((always_inline)) {
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
        wo[nb] = *LDS_PTR(const bf16x8, st + wlane + (uint32_t)((nb * 32 * kKS + k16 * 16) * 2));
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb)
        xo[mb] = *LDS_PTR(const bf16x8, st + xlane + (uint32_t)((mb * 32 * kKS + k16 * 16) * 2));
    };
    load_ops(0, wop[0], xop[0]);
#pragma unroll
    for (int k16 = 0; k16 < kBK / 16; ++k16) {
      if (k16 + 1 < kBK / 16) load_ops(k16 + 1, wop[(k16 + 1) & 1], xop[(k16 + 1) & 1]);
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
          acc[nb][mb] = mfma32(wop[k16 & 1][nb], xop[k16 & 1][mb], acc[nb][mb]);
    }
  }

  // Epilogue: lane (token l32 of each 32-token block) holds features
  // acc_row(r, h) of each 32-feature block; stage the wave tile row-major in
  // LDS (8-byte pieces), then write 16-byte chunks.
  __syncthreads();  // every wave is done reading the ring
  bf16* ost = ring + wave * kWM * kOS;
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row = mb * 32 + l32, col = nb * 32 + g * 8 + h * 4;
        const uint2 v = make_uint2(pack_bf16x2(acc[nb][mb][g * 4 + 0], acc[nb][mb][g * 4 + 1]),
                                   pack_bf16x2(acc[nb][mb][g * 4 + 2], acc[nb][mb][g * 4 + 3]));
        *reinterpret_cast<uint2*>(&ost[row * kOS + col]) = v;
      }
  __builtin_amdgcn_wave_barrier();
  constexpr int kChunks = kWM * kWN / 8;
  const int C = p.H * p.D;
#pragma unroll 4
  for (int c = lane; c < kChunks; c += kWave) {
    const int row = c / (kWN / 8), cc = c % (kWN / 8);
    const int m = m0 + wm * kWM + row;
    const int n = n0 + wn * kWN + cc * 8;
    if (m < p.M && n < p.N) {
      const uint4 v = *reinterpret_cast<const uint4*>(&ost[row * kOS + cc * 8]);
      if (SCATTER) {
        const int which = n / C, rem = n - which * C;
        const int hh = rem / p.D, d = rem - hh * p.D;
        const int b = m / p.T, t = m - b * p.T;
        bf16* dst = p.out[which] + (((size_t)b * p.H + hh) * p.T + t) * p.D + d;
        *reinterpret_cast<uint4*>(dst) = v;
      } else {
        *reinterpret_cast<uint4*>(p.out[0] + (size_t)m * p.N + n) = v;
      }
    }
  }
}

}  // namespace

hipError_t launch_proj_bf16(const void* x, const void* w, void* const out[3], int64_t M, int N,
                            int K, int T, int H, int D, bool gather, bool scatter,
                            hipStream_t stream) {
  if (K % 32 != 0 || M < 1 || N < 1) return hipErrorInvalidValue;
  ProjArgs p;
  p.x = (const bf16*)x;
  p.w = (const bf16*)w;
  for (int i = 0; i < 3; ++i) p.out[i] = (bf16*)out[i];
  p.M = (int)M;
  p.N = N;
  p.K = K;
  p.T = T;
  p.H = H;
  p.D = D;
  p.nbn = (N + kBN - 1) / kBN;
  const int64_t nbm = (M + kBM - 1) / kBM;
  const int64_t nblocks = nbm * p.nbn;
  if (nblocks > 0x7fffffff || M > 0x7fffffff) return hipErrorInvalidConfiguration;
  p.nblocks = (int)nblocks;
  if (gather && !scatter) {
    hipLaunchKernelGGL((proj_kernel<true, false>), dim3((unsigned)nblocks), dim3(kThreads), 0,
                       stream, p);
  } else if (!gather && scatter) {
    hipLaunchKernelGGL((proj_kernel<false, true>), dim3((unsigned)nblocks), dim3(kThreads), 0,
                       stream, p);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pab
