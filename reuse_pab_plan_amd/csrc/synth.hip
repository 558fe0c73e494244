// synth.hip -- the device workload generator: Philox4x32-10 streams and
// Box-Muller standard normals (definitions in include/pab_synth.h).  Not
// part of the PAB method: it only draws the synthetic inputs the attention
// calls consume.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "abi.hpp"
#include "../../include/pab_synth.h"

namespace pab {
namespace {

constexpr int kThreads = 256;
constexpr int kBlocks = 4096;            // grid-stride; 16 waves per CU on 256 CUs
constexpr uint32_t kM0 = 0xD2511F53u;    // Philox4x32 round multipliers
constexpr uint32_t kM1 = 0xCD9E8D57u;
constexpr uint32_t kW0 = 0x9E3779B9u;    // key schedule increments (Weyl sequence)
constexpr uint32_t kW1 = 0xBB67AE85u;
constexpr int64_t kMaxCount = (int64_t)1 << 62;

struct U4 {
  uint32_t x, y, z, w;
};

// Ten Philox rounds on counter (c0, c1, c2, c3) under key (k0, k1); the key
// advances by (kW0, kW1) between rounds.
__device__ __forceinline__ U4 philox10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                       uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)kM0 * c0;
    const uint64_t p1 = (uint64_t)kM1 * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += kW0;
    k1 += kW1;
  }
  return {c0, c1, c2, c3};
}

__device__ __forceinline__ U4 block_of(uint64_t i, uint64_t key) {
  return philox10((uint32_t)i, (uint32_t)(i >> 32), 0u, 0u, (uint32_t)key, (uint32_t)(key >> 32));
}

// Box-Muller on one word pair: (r cos 2 pi w, r sin 2 pi w).  The device sin
// and cos take their argument in revolutions; log2 gives ln u = ln 2 * log2 u.
__device__ __forceinline__ void box_muller(uint32_t x, uint32_t y, float& z0, float& z1) {
  const float u = ((float)(x >> 9) + 0.5f) * 0x1p-23f;
  const float w = ((float)(y >> 9) + 0.5f) * 0x1p-23f;
  const float r = __builtin_sqrtf(-1.3862943611198906f * __builtin_amdgcn_logf(u));
  z0 = r * __builtin_amdgcn_cosf(w);
  z1 = r * __builtin_amdgcn_sinf(w);
}

__device__ __forceinline__ void normals4(uint64_t i, uint64_t key, float (&z)[4]) {
  const U4 b = block_of(i, key);
  box_muller(b.x, b.y, z[0], z[1]);
  box_muller(b.z, b.w, z[2], z[3]);
}

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  // Round to nearest even on the upper 16 bits (inputs are finite).
  const uint32_t u = __builtin_bit_cast(uint32_t, f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__global__ __launch_bounds__(kThreads) void philox_kernel(uint32_t* __restrict__ out, int64_t nblocks,
                                                        uint64_t key, uint64_t block0) {
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t j = (int64_t)blockIdx.x * kThreads + threadIdx.x; j < nblocks; j += stride) {
    const U4 b = block_of(block0 + (uint64_t)j, key);
    *reinterpret_cast<uint4*>(out + 4 * j) = make_uint4(b.x, b.y, b.z, b.w);
  }
}

// Eight elements (two Philox blocks per stream) per thread and iteration.
template <bool BF16, bool TWO>
__global__ __launch_bounds__(kThreads) void normal_kernel(void* __restrict__ out, int64_t n,
                                                        uint64_t key_a, float sa, uint64_t key_b,
                                                        float sb) {
  const int64_t groups = (n + 7) / 8;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < groups; g += stride) {
    float v[8];
    {
      float z[4];
      normals4((uint64_t)(2 * g), key_a, z);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = sa * z[e];
      normals4((uint64_t)(2 * g + 1), key_a, z);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 + e] = sa * z[e];
    }
    if (TWO) {
      float z[4];
      normals4((uint64_t)(2 * g), key_b, z);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = __builtin_fmaf(sb, z[e], v[e]);
      normals4((uint64_t)(2 * g + 1), key_b, z);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 + e] = __builtin_fmaf(sb, z[e], v[4 + e]);
    }
    const int64_t e0 = 8 * g;
    if (e0 + 8 <= n) {
      if (BF16) {
        uint4 w;
        w.x = bf16_rne_bits(v[0]) | (bf16_rne_bits(v[1]) << 16);
        w.y = bf16_rne_bits(v[2]) | (bf16_rne_bits(v[3]) << 16);
        w.z = bf16_rne_bits(v[4]) | (bf16_rne_bits(v[5]) << 16);
        w.w = bf16_rne_bits(v[6]) | (bf16_rne_bits(v[7]) << 16);
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(out) + e0) = w;
      } else {
        float* o = static_cast<float*>(out) + e0;
        *reinterpret_cast<float4*>(o) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(o + 4) = make_float4(v[4], v[5], v[6], v[7]);
      }
    } else {
      for (int e = 0; e < 8 && e0 + e < n; ++e) {
        if (BF16)
          static_cast<uint16_t*>(out)[e0 + e] = (uint16_t)bf16_rne_bits(v[e]);
        else
          static_cast<float*>(out)[e0 + e] = v[e];
      }
    }
  }
}

int grid_for(int64_t items) {
  const int64_t b = (items + kThreads - 1) / kThreads;
  return (int)(b < kBlocks ? b : kBlocks);
}

int launched(const char* fn) {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? ok() : device_error(fn, (int)e);
}

}  // namespace
}  // namespace pab

using namespace pab;

extern "C" int pab_synth_philox(uint32_t* out, int64_t nblocks, uint64_t key, uint64_t block0,
                                void* stream) {
  if (!aligned16(out)) return fail(PAB_ERR_INVALID_ARG, "pab_synth_philox: out NULL or not 16-byte aligned");
  if (nblocks < 1 || nblocks > kMaxCount || block0 > (uint64_t)(kMaxCount - nblocks))
    return fail(PAB_ERR_INVALID_ARG, "pab_synth_philox: nblocks must be >= 1 and block0 + nblocks <= 2^62");
  hipLaunchKernelGGL(philox_kernel, dim3(grid_for(nblocks)), dim3(kThreads), 0, (hipStream_t)stream, out,
                     nblocks, key, block0);
  return launched("pab_synth_philox");
}

extern "C" int pab_synth_normal(void* out, int64_t n, int32_t dtype, uint64_t key_a, float scale_a,
                                uint64_t key_b, float scale_b, void* stream) {
  if (!aligned16(out)) return fail(PAB_ERR_INVALID_ARG, "pab_synth_normal: out NULL or not 16-byte aligned");
  if (n < 1 || n > kMaxCount) return fail(PAB_ERR_INVALID_ARG, "pab_synth_normal: n must be in [1, 2^62]");
  if (!std::isfinite(scale_a) || !std::isfinite(scale_b))
    return fail(PAB_ERR_INVALID_ARG, "pab_synth_normal: scales must be finite");
  if (dtype != PAB_BF16 && dtype != PAB_F32)
    return fail(PAB_ERR_UNSUPPORTED, fmt("pab_synth_normal: unsupported dtype %d", dtype));
  const dim3 grid(grid_for((n + 7) / 8)), block(kThreads);
  const hipStream_t s = (hipStream_t)stream;
  const bool two = scale_b != 0.f;
  if (dtype == PAB_BF16) {
    if (two)
      hipLaunchKernelGGL((normal_kernel<true, true>), grid, block, 0, s, out, n, key_a, scale_a, key_b, scale_b);
    else
      hipLaunchKernelGGL((normal_kernel<true, false>), grid, block, 0, s, out, n, key_a, scale_a, key_b, scale_b);
  } else {
    if (two)
      hipLaunchKernelGGL((normal_kernel<false, true>), grid, block, 0, s, out, n, key_a, scale_a, key_b, scale_b);
    else
      hipLaunchKernelGGL((normal_kernel<false, false>), grid, block, 0, s, out, n, key_a, scale_a, key_b, scale_b);
  }
  return launched("pab_synth_normal");
}
