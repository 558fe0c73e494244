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

constexpr int kStreamThreads = 256;
constexpr int kMaxStreamBlocks = 65536;
constexpr int kMfmaBlocks = 2048;     // 4-wave blocks: 32 waves per CU on 256 CUs
constexpr int kMfmaThreads = 256;
constexpr int kMfmaChains = 4;        // independent accumulators per wave

__device__ __forceinline__ u32x4 ld(const u32x4* p, bool nt) {
  return nt ? __builtin_nontemporal_load(p) : *p;
}
__device__ __forceinline__ void st(u32x4* p, u32x4 v, bool nt) {
  if (nt)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}

struct StreamArgs {
  const u32x4* src[4];
  u32x4* dst[2];
  int ns, nd;
};

// One pass over n 16-byte vectors of a.ns source and a.nd destination
// streams: dst_j[i] = XOR over the sources of src[i] (or i itself with no
// source); with no destination the XOR is folded into one word per block.
// Each thread keeps U vectors of every stream in flight.  Layout: CH = false
// strides the whole grid over the buffers (a wave's U vectors are a grid
// apart); CH = true gives every block one contiguous chunk, walked U x 4 KiB
// at a time.  Tails run one vector at a time.
template <bool NT, int U, bool CH>
__global__ __launch_bounds__(kStreamThreads) void stream_kernel(StreamArgs a, int64_t n,
                                                              uint32_t* __restrict__ sink) {
  int64_t i, stride, end, ustep;
  if (CH) {
    const int64_t per = ((n + gridDim.x - 1) / gridDim.x + kStreamThreads - 1) / kStreamThreads *
                        kStreamThreads;
    i = (int64_t)blockIdx.x * per + threadIdx.x;
    end = (int64_t)(blockIdx.x + 1) * per;
    end = end < n ? end : n;
    ustep = kStreamThreads;
    stride = (int64_t)U * kStreamThreads;
  } else {
    i = (int64_t)blockIdx.x * kStreamThreads + threadIdx.x;
    end = n;
    ustep = (int64_t)gridDim.x * kStreamThreads;
    stride = (int64_t)U * ustep;
  }
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (U - 1) * ustep < end; i += stride) {
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t w = (uint32_t)(i + u * ustep);
      v[u] = u32x4{w, w, w, w};
    }
#pragma unroll
    for (int s = 0; s < 4; ++s)
      if (s < a.ns) {
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] ^= ld(a.src[s] + i + u * ustep, NT);
      }
#pragma unroll
    for (int d = 0; d < 2; ++d)
      if (d < a.nd) {
#pragma unroll
        for (int u = 0; u < U; ++u) st(a.dst[d] + i + u * ustep, v[u], NT);
      }
    if (a.nd == 0) {
#pragma unroll
      for (int u = 0; u < U; ++u) acc ^= v[u];
    }
  }
  for (; i < end; i += ustep) {
    const uint32_t w = (uint32_t)i;
    u32x4 v = {w, w, w, w};
    for (int s = 0; s < a.ns; ++s) v ^= a.src[s][i];
    for (int d = 0; d < a.nd; ++d) a.dst[d][i] = v;
    acc ^= v;
  }
  if (a.nd == 0) {
    __shared__ uint32_t red[kStreamThreads];
    red[threadIdx.x] = acc.x ^ acc.y ^ acc.z ^ acc.w;
    __syncthreads();
    for (int s = kStreamThreads / 2; s > 0; s >>= 1) {
      if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
      __syncthreads();
    }
    if (threadIdx.x == 0) sink[blockIdx.x] = red[0];
  }
}

template <bool NT, int U>
void launch_stream_u(const StreamArgs& a, int64_t n, int blocks, bool ch, uint32_t* sink,
                     hipStream_t s) {
  if (ch)
    hipLaunchKernelGGL((stream_kernel<NT, U, true>), dim3(blocks), dim3(kStreamThreads), 0, s, a, n,
                       sink);
  else
    hipLaunchKernelGGL((stream_kernel<NT, U, false>), dim3(blocks), dim3(kStreamThreads), 0, s, a, n,
                       sink);
}

template <bool NT>
void launch_stream_nt(const StreamArgs& a, int64_t n, int blocks, int u, bool ch, uint32_t* sink,
                      hipStream_t s) {
  if (u == 0)
    launch_stream_u<NT, 4>(a, n, blocks, ch, sink, s);
  else if (u == 1)
    launch_stream_u<NT, 8>(a, n, blocks, ch, sink, s);
  else
    launch_stream_u<NT, 16>(a, n, blocks, ch, sink, s);
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

extern "C" int pab_peak_stream(const void* const* src, int32_t n_src, void* const* dst,
                               int32_t n_dst, size_t bytes, int32_t blocks, int32_t variant,
                               void* sink, size_t sink_bytes, void* stream) {
  const char* fn = "pab_peak_stream";
  if (n_src < 0 || n_src > 4 || n_dst < 0 || n_dst > 2 || n_src + n_dst < 1)
    return fail(PAB_ERR_INVALID_ARG, fmt("%s: need 0 <= n_src <= 4, 0 <= n_dst <= 2, one stream", fn));
  if ((n_src && !src) || (n_dst && !dst)) return fail(PAB_ERR_INVALID_ARG, fmt("%s: NULL array", fn));
  if (bytes == 0 || bytes % 16 != 0)
    return fail(PAB_ERR_INVALID_ARG, fmt("%s: bytes must be a positive multiple of 16", fn));
  if (blocks < 1 || blocks > kMaxStreamBlocks)
    return fail(PAB_ERR_INVALID_ARG, fmt("%s: blocks must be in [1, %d]", fn, kMaxStreamBlocks));
  if (variant < 0 || variant > 15 || ((variant >> 1) & 3) == 3)
    return fail(PAB_ERR_INVALID_ARG, fmt("%s: unknown variant %d", fn, variant));
  StreamArgs a{};
  a.ns = n_src;
  a.nd = n_dst;
  const void* all[6];
  size_t nall = 0;
  for (int i = 0; i < n_src; ++i) {
    if (!aligned16(src[i])) return fail(PAB_ERR_INVALID_ARG, fmt("%s: src[%d] NULL or misaligned", fn, i));
    a.src[i] = (const u32x4*)src[i];
    all[nall++] = src[i];
  }
  for (int i = 0; i < n_dst; ++i) {
    if (!aligned16(dst[i])) return fail(PAB_ERR_INVALID_ARG, fmt("%s: dst[%d] NULL or misaligned", fn, i));
    a.dst[i] = (u32x4*)dst[i];
    all[nall++] = dst[i];
  }
  for (size_t i = 0; i < nall; ++i)
    for (size_t j = i + 1; j < nall; ++j)
      if (ranges_overlap(all[i], bytes, all[j], bytes))
        return fail(PAB_ERR_INVALID_ARG, fmt("%s: buffers overlap", fn));
  if (n_dst == 0) {
    const int st = check_sink(fn, sink, sink_bytes);
    if (st) return st;
    if ((size_t)blocks * sizeof(uint32_t) > sink_bytes)
      return fail(PAB_ERR_CAPACITY, fmt("%s: sink holds fewer words than blocks", fn));
  }
  const int64_t n = (int64_t)(bytes / 16);
  const hipStream_t s = (hipStream_t)stream;
  uint32_t* sk = (uint32_t*)sink;
  const int u = (variant >> 1) & 3;
  const bool ch = (variant >> 3) & 1;
  if (variant & 1)
    launch_stream_nt<true>(a, n, blocks, u, ch, sk, s);
  else
    launch_stream_nt<false>(a, n, blocks, u, ch, sk, s);
  return launched(fn);
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
  const size_t a = (size_t)kMaxStreamBlocks * sizeof(uint32_t);
  const size_t b = (size_t)kMfmaBlocks * kMfmaThreads * sizeof(float);
  return a > b ? a : b;
}
