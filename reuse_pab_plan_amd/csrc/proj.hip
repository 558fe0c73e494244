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
// output features in runs of 4.
//
// A 512-thread block (two waves per SIMD, so one wave's LDS waits hide under
// the other's MFMAs) computes a 256-token x 384-feature tile; each wave owns
// 128 x 96 (12 accumulators).  k advances 32 at a time through a four-stage
// LDS ring filled by direct global->LDS loads three steps ahead; a wave's
// loads for a stage are spread over one k slice of MFMAs.  A stage row holds
// 32 k values (64 bytes, four 16-byte chunks) with the chunks of row r
// permuted by f(r) = (r >> 3) & 3, which keeps the 16-byte operand reads
// mostly free of LDS bank conflicts without padding (measured: about 10% of
// LDS cycles, against half with other permutations); the direct loads apply
// the permutation by choosing, per lane, which global chunk lands in its
// fixed LDS slot.  The output is staged per wave through LDS, 32 tokens at a
// time, and written in 16-byte chunks (scattered straight into the
// head-major q, k, v tensors for the input projection).
#include "device.hpp"
#include "launch.hpp"

namespace pab {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;
constexpr int kBM = 256;                  // tokens per block
constexpr int kBN = 384;                  // output features per block
constexpr int kBK = 32;                   // k per ring stage
constexpr int kRowBytes = kBK * 2;        // one LDS row: 64 bytes, 4 chunks
constexpr int kRows = kBM + kBN;          // token rows, then weight rows
constexpr int kStageBytes = kRows * kRowBytes;
constexpr int kNst = 4;
constexpr int kLoads = kRows * 4 / kWave;       // wave-wide 1 KiB loads per stage (40)
constexpr int kXLoads = kBM * 4 / kWave;        // of them token rows (16)
constexpr int kPerWave = kLoads / kWaves;       // 5
constexpr int kXPerWave = kXLoads / kWaves;     // 2
constexpr int kWM = 128, kWN = 96;        // wave tile
constexpr int kMB = kWM / 32, kNB = kWN / 32;
constexpr int kOS = kWN + 8;              // epilogue staging row stride (elements)
static_assert(kLoads % kWaves == 0 && kXLoads % kWaves == 0, "loads split evenly over the waves");
static_assert(kNst * kStageBytes <= 160 * 1024, "LDS ring too large");
static_assert(kWaves * 32 * kOS * 2 <= kNst * kStageBytes, "epilogue staging fits the ring");
static_assert(kBM / kWM * (kBN / kWN) == kWaves, "wave grid covers the tile");
static_assert(kMB + 1 == kPerWave, "a slice carries one load per token block, plus one");

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

// One 16-byte direct global->LDS load per lane: lane l of the wave reads
// global bytes [gbase + voff, +16) and writes LDS bytes [lds + 16*l, +16).
// `gbase` and `lds` must be wave-uniform.  Inline assembly, so the wait for
// it (s_waitcnt vmcnt) is placed by hand: the compiler does not track it.
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

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Wait until at most `ahead` (0, 1 or 2) later stages of this wave's loads
// are still in flight.
__device__ __forceinline__ void wait_stages(int ahead) {
  if (ahead >= 2) {
    wait_vmcnt<2 * kPerWave>();
  } else if (ahead == 1) {
    wait_vmcnt<kPerWave>();
  } else {
    wait_vmcnt<0>();
  }
}

__device__ __forceinline__ const bf16* uniform_ptr(const bf16* p) {
  const uint64_t u = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const bf16*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// Chunk permutation of LDS row r; rows 32 q + i permute like row i, so a
// lane's operand offsets do not depend on which 32-row block it reads.
__host__ __device__ constexpr int swz(int r) { return (r >> 3) & 3; }

struct ProjArgs {
  const bf16* x;      // token-major input [M, K] (GATHER: head-major [B, H, T, D])
  const bf16* w;      // weight [N, K]
  bf16* out[3];       // SCATTER: head-major tensors; else out[0] token-major [M, N]
  int M, N, K;        // tokens, output features, input features
  int T, H, D;        // tokens per entry, heads, head dim
  float inv_d;        // 1 / D
  int nbn;            // feature tiles
  int nblocks;
};

// GATHER: the input is a head-major attention output (output projection).
// SCATTER: the output goes to head-major tensors (input projection).
template <bool GATHER, bool SCATTER>
__global__ __launch_bounds__(kThreads, 1) void proj_kernel(ProjArgs p) {
  __shared__ __attribute__((aligned(16))) bf16 ring[kNst * kStageBytes / 2];

  const int tid = threadIdx.x;
  const int lane = tid & 63, l32 = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int logical = xcd_remap(blockIdx.x, p.nblocks);
  const int bm = logical / p.nbn, bn = logical % p.nbn;
  const int m0 = bm * kBM, n0 = bn * kBN;
  const int K = p.K;
  const int nkt = K / kBK;

  // Direct-load plan.  Wave-load j (0..39) fills stage bytes [1024 j, +1024):
  // lane l writes slot 64 j + l = row 16 j + l / 4, physical chunk l % 4,
  // which holds logical k chunk (l % 4) ^ swz(row).  Loads j < 16 are token
  // rows, the rest weight rows; wave w issues j = w + 8 i (two token loads,
  // three weight loads).  Rows past the matrix repeat its last row (finite,
  // never stored).
  const int lrow = lane >> 2;
  uint32_t xoff[kXPerWave];   // GATHER: element offset of (b, t) in head 0; else byte offset
  int xkc[kXPerWave];         // logical k chunk of the lane (GATHER)
  uint32_t woff[kPerWave - kXPerWave];
#pragma unroll
  for (int i = 0; i < kXPerWave; ++i) {
    const int row = 16 * (wave + kWaves * i) + lrow;
    const int kc = (lane & 3) ^ swz(row);
    const int m = min(m0 + row, p.M - 1);
    if (GATHER) {
      const int b = m / p.T, t = m - b * p.T;
      xoff[i] = (uint32_t)(((size_t)b * p.H * p.T + t) * p.D);
      xkc[i] = kc;
    } else {
      xoff[i] = (uint32_t)(((size_t)m * K + kc * 8) * 2);
      xkc[i] = kc;
    }
  }
#pragma unroll
  for (int i = 0; i < kPerWave - kXPerWave; ++i) {
    const int row = 16 * (wave + kWaves * (i + kXPerWave)) + lrow;
    const int kc = (lane & 3) ^ swz(row);
    const int n = min(n0 + row - kBM, p.N - 1);
    woff[i] = (uint32_t)(((size_t)n * K + kc * 8) * 2);
  }
  const uint32_t ring_lds = (uint32_t)(uintptr_t)LDS_PTR(void, ring);
  const bf16* xbase = uniform_ptr(p.x);
  const bf16* wbase = uniform_ptr(p.w);
  const uint32_t plane = (uint32_t)p.T * (uint32_t)p.D;  // elements per head plane
  // Load i (0..kPerWave-1) of this wave for stage kt.
  auto issue_one = [&](int kt, int i) __attribute__((always_inline)) {
    const int k0 = kt * kBK;
    const uint32_t lds = ring_lds + (uint32_t)((kt % kNst) * kStageBytes) +
                         (uint32_t)((wave + kWaves * i) * 1024);
    if (i < kXPerWave) {
      if (GATHER) {
        // k -> (head, channel); exact for k < 2^14 and D <= 128.
        const int k = k0 + xkc[i] * 8;
        const int hh = (int)(((float)k + 0.5f) * p.inv_d);
        const int d = k - hh * p.D;
        dma16(xbase, (xoff[i] + (uint32_t)hh * plane + (uint32_t)d) * 2u, lds);
      } else {
        dma16(xbase + k0, xoff[i], lds);
      }
    } else {
      dma16(wbase + k0, woff[i - kXPerWave], lds);
    }
  };
  auto issue = [&](int kt) {
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) issue_one(kt, i);
  };

  // Wave tile: tokens wm*128.., features wn*96.. of the block tile.
  const int wm = wave & 1, wn = wave >> 1;
  const int sw = swz(l32);
  uint32_t xlane[2], wlane[2];
#pragma unroll
  for (int k16 = 0; k16 < 2; ++k16) {
    const uint32_t chunk = (uint32_t)(((2 * k16 + h) ^ sw) * 16);
    xlane[k16] = (uint32_t)((wm * kWM + l32) * kRowBytes) + chunk;
    wlane[k16] = (uint32_t)((kBM + wn * kWN + l32) * kRowBytes) + chunk;
  }

  f32x16 acc[kNB][kMB];
#pragma unroll
  for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) acc[nb][mb] = zero16();

  auto stage_addr = [&](int kt) { return ring_lds + (uint32_t)((kt % kNst) * kStageBytes); };
  auto read_w = [&](bf16x8 (&w)[kNB], uint32_t st, int k16) __attribute__((always_inline)) {
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
      w[nb] = *LDS_PTR(const bf16x8, st + wlane[k16] + (uint32_t)(nb * 32 * kRowBytes));
  };
  auto read_x = [&](bf16x8& x, uint32_t st, int k16, int mb) __attribute__((always_inline)) {
    x = *LDS_PTR(const bf16x8, st + xlane[k16] + (uint32_t)(mb * 32 * kRowBytes));
  };
  // One k slice: MFMAs with weights w and token operands x; as each token
  // operand is used up, the next slice's replaces it (read from st, k16).
  // kt_load >= 0: this wave's loads for stage kt_load are spread over the
  // slice (one or two after each token block), so the address unit takes
  // them while the MFMAs run.
  auto slice = [&](const bf16x8 (&w)[kNB], bf16x8 (&x)[kMB], uint32_t st, int k16, int kt_load)
      __attribute__((always_inline)) {
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) acc[nb][mb] = mfma32(w[nb], x[mb], acc[nb][mb]);
      read_x(x[mb], st, k16, mb);
      if (kt_load >= 0) {
        issue_one(kt_load, mb);
        if (mb == kMB - 1) issue_one(kt_load, kMB);
      }
    }
  };

  // Pipeline.  Each step's two k slices straddle one barrier, and the
  // operands of the slice after a barrier are read before it, so the matrix
  // pipe never waits on LDS behind a barrier.  The barrier in step kt
  // publishes stage kt+1 (every wave's loads landed) and retires stage kt-1
  // (every wave is past it), whose slot then takes stage kt+3.  Two weight
  // operand sets alternate; the token operands are replaced one by one.
#pragma unroll
  for (int s = 0; s < kNst - 1; ++s)
    if (s < nkt) issue(s);
  wait_stages(min(nkt - 1, kNst - 2));
  __syncthreads();
  bf16x8 wa[kNB], wb[kNB], x[kMB];
  read_w(wa, stage_addr(0), 0);
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) read_x(x[mb], stage_addr(0), 0, mb);
  for (int kt = 0; kt < nkt; ++kt) {
    const uint32_t st = stage_addr(kt);
    read_w(wb, st, 1);
    slice(wa, x, st, 1, -1);
    if (kt + 1 < nkt) {
      wait_stages(min(nkt - 1, kt + 2) - (kt + 1));
      // A bare barrier: the compiler keeps LDS accesses on their side of it
      // (memory clobbers) but need not drain the operand reads already in
      // flight, which target a stage nobody overwrites here.
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    }
    // After the last step the reads below fetch the current stage again
    // (in bounds, unused).
    const uint32_t sn = stage_addr(kt + 1 < nkt ? kt + 1 : kt);
    read_w(wa, sn, 0);
    slice(wb, x, sn, 0, kt + kNst - 1 < nkt ? kt + kNst - 1 : -1);
  }

  // Epilogue: lane (token l32 of each 32-token block) holds features
  // acc_row(r, h) of each 32-feature block.  Per 32-token block, stage the
  // wave's 32 x 96 slab row-major in LDS (8-byte pieces), then write 16-byte
  // chunks: chunk c = lane + 64 i is row c / 12, feature chunk c % 12.
  __syncthreads();  // every wave is done reading the ring
  bf16* ost = ring + wave * 32 * kOS;
  constexpr int kCPR = kWN / 8;                 // chunks per row (12)
  constexpr int kCPL = 32 * kCPR / kWave;       // chunks per lane (6)
  const int C = p.H * p.D;
  // Feature side of each of the lane's chunks (fixed over the token blocks).
  int nfeat[kCPL];
  bf16* fbase[kCPL];
  int rowof[kCPL];
#pragma unroll
  for (int i = 0; i < kCPL; ++i) {
    const int c = lane + kWave * i;
    rowof[i] = c / kCPR;
    const int n = n0 + wn * kWN + (c % kCPR) * 8;
    nfeat[i] = n;
    if (SCATTER) {
      const int nn = min(n, p.N - 1);
      const int which = nn / C, rem = nn - which * C;
      const int hh = rem / p.D, d = rem - hh * p.D;
      fbase[i] = p.out[which] + (size_t)hh * plane + d;
    } else {
      fbase[i] = p.out[0] + n;
    }
  }
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) {
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = nb * 32 + g * 8 + h * 4;
        const uint2 v = make_uint2(pack_bf16x2(acc[nb][mb][g * 4 + 0], acc[nb][mb][g * 4 + 1]),
                                   pack_bf16x2(acc[nb][mb][g * 4 + 2], acc[nb][mb][g * 4 + 3]));
        *reinterpret_cast<uint2*>(&ost[l32 * kOS + col]) = v;
      }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < kCPL; ++i) {
      const int c = lane + kWave * i;
      const uint4 v = *reinterpret_cast<const uint4*>(&ost[rowof[i] * kOS + (c % kCPR) * 8]);
      const int m = m0 + wm * kWM + mb * 32 + rowof[i];
      if (m < p.M && nfeat[i] < p.N) {
        if (SCATTER) {
          const int b = m / p.T, t = m - b * p.T;
          bf16* dst = fbase[i] + ((size_t)b * p.H * p.T + t) * p.D;
          *reinterpret_cast<uint4*>(dst) = v;
        } else {
          *reinterpret_cast<uint4*>(fbase[i] + (size_t)m * p.N) = v;
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

hipError_t launch_proj_bf16(const void* x, const void* w, void* const out[3], int64_t M, int N,
                            int K, int T, int H, int D, bool gather, bool scatter,
                            hipStream_t stream) {
  if (K % kBK != 0 || M < 1 || N < 1 || K > 16384 || D < 8 || D > 128) return hipErrorInvalidValue;
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
  p.inv_d = 1.0f / (float)D;
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
