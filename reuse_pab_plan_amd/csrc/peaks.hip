// peaks.hip -- microbenchmarks for the roofline denominators: what this
// MI355X sustains for HBM copy and read, bf16 MFMA issue and v_exp_f32,
// measured beside the datasheet figures.  Not part of the method: the
// attention kernels never call these.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "abi.hpp"
#include "device.hpp"
#include "../../include/pab_peaks.h"

namespace pab {
namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kStreamBlocks = 8192;   // copy / read grid (the measured sweet spot)
constexpr int kStreamThreads = 256;
constexpr int kUnroll = 4;
constexpr int kMfmaBlocks = 2048;     // 4-wave blocks: 32 waves per CU on 256 CUs
constexpr int kMfmaThreads = 256;
constexpr int kMfmaChains = 4;        // independent accumulators per wave

// dst[i] = src[i] over n 16-byte vectors, non-temporal on both sides.
__global__ __launch_bounds__(kStreamThreads) void copy_kernel(const u32x4* __restrict__ src,
                                                            u32x4* __restrict__ dst, int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
  int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
  for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
    u32x4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

// One XOR-folded word per block, so the loads cannot be dropped.
__global__ __launch_bounds__(kStreamThreads) void read_kernel(const u32x4* __restrict__ src, int64_t n,
                                                            uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * kStreamThreads;
  int64_t i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kUnroll - 1) * stride < n; i += kUnroll * stride) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= __builtin_nontemporal_load(src + i + u * stride);
  }
  for (; i < n; i += stride) acc ^= src[i];
  __shared__ uint32_t red[kStreamThreads];
  red[threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
  __syncthreads();
  for (int s = kStreamThreads / 2; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
}

// kMfmaChains independent v_mfma_f32_32x32x16_bf16 chains per wave.
__global__ __launch_bounds__(kMfmaThreads) void mfma_kernel(int iters, float* __restrict__ sink) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (bf16)(0.001f * (float)(threadIdx.x & 7) + (float)i);
    b[i] = (bf16)(0.5f * (float)i);
  }
  f32x16 acc[kMfmaChains];
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c) acc[c] = zero16();
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kMfmaChains; ++c) acc[c] = mfma32(a, b, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[(size_t)blockIdx.x * kMfmaThreads + threadIdx.x] = s;
}

// Eight independent v_exp_f32 chains per lane.
__global__ __launch_bounds__(kMfmaThreads) void exp_kernel(int iters, float* __restrict__ sink) {
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = -0.001f * (float)(threadIdx.x + j);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = fast_exp2(x[j]) - 1.0f;
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += x[j];
  sink[(size_t)blockIdx.x * kMfmaThreads + threadIdx.x] = s;
}

int check_stream_args(const char* fn, const void* a, size_t bytes) {
  if (!a) return fail(PAB_ERR_INVALID_ARG, fmt("%s: NULL pointer", fn));
  if (!aligned16(a)) return fail(PAB_ERR_INVALID_ARG, fmt("%s: pointers must be 16-byte aligned", fn));
  if (bytes == 0 || bytes % 16 != 0)
    return fail(PAB_ERR_INVALID_ARG, fmt("%s: bytes must be a positive multiple of 16", fn));
  return PAB_OK;
}

int check_sink(const char* fn, const void* sink, size_t sink_bytes) {
  if (!sink || !aligned16(sink))
    return fail(PAB_ERR_INVALID_ARG, fmt("%s: sink NULL or not 16-byte aligned", fn));
  if (sink_bytes < pab_peak_sink_bytes())
    return fail(PAB_ERR_CAPACITY, fmt("%s: sink smaller than pab_peak_sink_bytes()", fn));
  return PAB_OK;
}

int launched(const char* fn) {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? ok() : device_error(fn, (int)e);
}

}  // namespace
}  // namespace pab

using namespace pab;

extern "C" int pab_peak_copy(const void* src, void* dst, size_t bytes, void* stream) {
  int st = check_stream_args("pab_peak_copy", src, bytes);
  if (!st) st = check_stream_args("pab_peak_copy", dst, bytes);
  if (st) return st;
  if (ranges_overlap(src, bytes, dst, bytes))
    return fail(PAB_ERR_INVALID_ARG, "pab_peak_copy: source and destination overlap");
  hipLaunchKernelGGL(copy_kernel, dim3(kStreamBlocks), dim3(kStreamThreads), 0, (hipStream_t)stream,
                     (const u32x4*)src, (u32x4*)dst, (int64_t)(bytes / 16));
  return launched("pab_peak_copy");
}

extern "C" int pab_peak_read(const void* src, size_t bytes, void* sink, size_t sink_bytes,
                             void* stream) {
  int st = check_stream_args("pab_peak_read", src, bytes);
  if (!st) st = check_sink("pab_peak_read", sink, sink_bytes);
  if (st) return st;
  hipLaunchKernelGGL(read_kernel, dim3(kStreamBlocks), dim3(kStreamThreads), 0, (hipStream_t)stream,
                     (const u32x4*)src, (int64_t)(bytes / 16), (uint32_t*)sink);
  return launched("pab_peak_read");
}

extern "C" int pab_peak_mfma_bf16(int32_t iters, void* sink, size_t sink_bytes, double* flops,
                                  void* stream) {
  if (iters < 1 || !flops)
    return fail(PAB_ERR_INVALID_ARG, "pab_peak_mfma_bf16: iters must be >= 1, flops non-NULL");
  const int st = check_sink("pab_peak_mfma_bf16", sink, sink_bytes);
  if (st) return st;
  *flops = (double)kMfmaBlocks * (kMfmaThreads / kWave) * (double)iters * kMfmaChains * 2.0 * 32 *
           32 * 16;
  hipLaunchKernelGGL(mfma_kernel, dim3(kMfmaBlocks), dim3(kMfmaThreads), 0, (hipStream_t)stream,
                     (int)iters, (float*)sink);
  return launched("pab_peak_mfma_bf16");
}

extern "C" int pab_peak_exp(int32_t iters, void* sink, size_t sink_bytes, double* exps,
                            void* stream) {
  if (iters < 1 || !exps)
    return fail(PAB_ERR_INVALID_ARG, "pab_peak_exp: iters must be >= 1, exps non-NULL");
  const int st = check_sink("pab_peak_exp", sink, sink_bytes);
  if (st) return st;
  *exps = (double)kMfmaBlocks * kMfmaThreads * (double)iters * 8;
  hipLaunchKernelGGL(exp_kernel, dim3(kMfmaBlocks), dim3(kMfmaThreads), 0, (hipStream_t)stream,
                     (int)iters, (float*)sink);
  return launched("pab_peak_exp");
}

extern "C" size_t pab_peak_sink_bytes(void) {
  const size_t a = (size_t)kStreamBlocks * sizeof(uint32_t);
  const size_t b = (size_t)kMfmaBlocks * kMfmaThreads * sizeof(float);
  return a > b ? a : b;
}
