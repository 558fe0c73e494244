// device.hpp -- gfx950 device helpers shared by the attention kernels:
// vector types, the bf16 MFMA wrapper, XCD-aware block remapping and small
// conversion utilities.  Nothing here is method logic.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pab {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, each with its own L2

// v_mfma_f32_32x32x16_bf16:  D[32x32] += A[32x16] * B[16x32].
// Lane l (h = l/32, i = l%32) supplies A row i and B column i, eight k values
// each; A and B lanes of the same half h hold the same eight k indices, so any
// fixed pairing of (h, j) with k is a valid contraction order.  The result
// lands in lane l as acc[r] = D[(r/4)*8 + h*4 + r%4][i].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x32_bf16:  D[16x16] += A[16x32] * B[32x16].  Lane l
// (g = l/16, i = l%16) supplies A row i and B column i, eight k values each
// (k = 8g .. 8g+7); the result lands in lane l as acc[r] = D[4g + r][i].
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

// Row index (within a 32-row block) of accumulator element r for half h.
__host__ __device__ constexpr int acc_row(int r, int h) { return (r >> 2) * 8 + h * 4 + (r & 3); }

// Workgroups are dispatched round-robin over the XCDs (block b runs on XCD
// b % 8).  Remap so that logically consecutive blocks -- which share K/V
// through L2 -- land on the same XCD.  Bijective for any block count.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
  const int per = nblocks / kNumXcd;
  const int rem = nblocks % kNumXcd;
  const int x = bid % kNumXcd;
  const int i = bid / kNumXcd;
  return (x < rem) ? x * (per + 1) + i : rem * (per + 1) + (x - rem) * per + i;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  // One v_cvt_pk_bf16_f32 (round to nearest even on both halves).
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Eight fp32 values -> one MFMA operand of bf16 (round to nearest even).
__device__ __forceinline__ bf16x8 to_bf16x8(float v0, float v1, float v2, float v3, float v4,
                                            float v5, float v6, float v7) {
  bf16x8 r;
  r[0] = (bf16)v0; r[1] = (bf16)v1; r[2] = (bf16)v2; r[3] = (bf16)v3;
  r[4] = (bf16)v4; r[5] = (bf16)v5; r[6] = (bf16)v6; r[7] = (bf16)v7;
  return r;
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  return __builtin_bit_cast(bf16x8, make_uint4(0u, 0u, 0u, 0u));
}

// Sum over the two bf16 pairs of (a_i - b_i)^2, the differences formed and
// squared in fp64 (the attention difference of two stored outputs).
__device__ __forceinline__ double sqdiff_bf16x2(uint32_t a, uint32_t b) {
  const double d0 = (double)bf16_bits_to_float(a & 0xFFFFu) - (double)bf16_bits_to_float(b & 0xFFFFu);
  const double d1 = (double)__builtin_bit_cast(float, a & 0xFFFF0000u) -
                    (double)__builtin_bit_cast(float, b & 0xFFFF0000u);
  return __builtin_fma(d1, d1, d0 * d0);
}

// Block-wide fp64 sum in a fixed order (butterfly within each wave, then the
// waves in index order); the result is valid in thread 0.  `red` is an LDS
// array of WAVES doubles.  Every thread of the block must call it.
template <int WAVES>
__device__ __forceinline__ double block_sum_f64(double v, double* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  double s = 0.0;
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 0; w < WAVES; ++w) s += red[w];
  }
  return s;
}

// Lane exchange with the lane 32 positions away (the other half-wave).
__device__ __forceinline__ float xor32(float v) { return __shfl_xor(v, 32, 64); }

// v_permlane32_swap of a value with itself: .lo holds, in every lane, the value
// of the lower half-wave lane of the same column (lane % 32), .y that of the
// upper half-wave lane (.hi).
struct HalfPair {
  float lo, hi;
};
__device__ __forceinline__ HalfPair half_pair(float v) {
  const unsigned u = __builtin_bit_cast(unsigned, v);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return {__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1])};
}

// Max over the two half-wave lanes that share a column.
__device__ __forceinline__ float max_halves(float v) {
  const HalfPair p = half_pair(v);
  return fmaxf(p.lo, p.hi);
}

}  // namespace pab
