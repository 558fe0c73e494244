// mse.hip -- attention difference as a mean squared error (PAB article,
// Figure 1 caption: the change of an attention output between diffusion
// steps is measured by the MSE).
//
// HBM-bound: 2*n*sizeof(dtype) bytes read, ~4 fp64 operations per element.
// Pass 1: a fixed grid (depending only on n) streams 16-byte vectors of a and
// b; every element's difference is formed and squared in fp64 and summed in
// fp64; each block writes one partial.  Pass 2: one block adds the partials in
// a fixed order and divides by n.  The reduction order depends only on n, so
// results are bitwise reproducible.
#include <atomic>

#include "device.hpp"
#include "launch.hpp"

// Device scratch of the MSE entry point that allocates nothing
// (pab_attn_diff_mse_noalloc): the per-block partial sums of pass 1, one
// double per block of the largest grid (kMaxBlocks = 4096: 32 KiB).  Every
// GPU the library runs on holds its own copy until the process ends; calls
// on one GPU share it, so calls that overlap on one GPU race.
static __device__ __align__(256) double scratch[4096];

namespace pab {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxBlocks = 4096;
constexpr int kUnroll = 4;
static_assert(sizeof(scratch) == kMaxBlocks * sizeof(double), "one partial per block");
constexpr int kMaxDevices = 64;
// The device address of `scratch` per device, looked up once per device.
std::atomic<double*> g_scratch[kMaxDevices];

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Block-wide sum in a fixed order; result valid in thread 0.
__device__ __forceinline__ double block_sum(double v) {
  __shared__ double part[kThreads / kWave];
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  if ((threadIdx.x % kWave) == 0) part[w] = v;
  __syncthreads();
  double s = 0.0;
  if (threadIdx.x == 0) {
#pragma unroll
    for (int i = 0; i < kThreads / kWave; ++i) s += part[i];
  }
  return s;
}

__device__ __forceinline__ double sq_bf16x2(uint32_t a, uint32_t b) {
  const double d0 = (double)bf16_bits_to_float(a & 0xffffu) - (double)bf16_bits_to_float(b & 0xffffu);
  const double d1 = (double)bf16_bits_to_float(a >> 16) - (double)bf16_bits_to_float(b >> 16);
  return fma(d0, d0, d1 * d1);
}

__device__ __forceinline__ double sq_f32(uint32_t a, uint32_t b) {
  const double d = (double)__builtin_bit_cast(float, a) - (double)__builtin_bit_cast(float, b);
  return d * d;
}

// One 16-byte vector of each input: 8 bf16 or 4 fp32 elements.
template <bool BF16>
__device__ __forceinline__ double sq_vec(u32x4 a, u32x4 b) {
  if (BF16) {
    return (sq_bf16x2(a.x, b.x) + sq_bf16x2(a.y, b.y)) + (sq_bf16x2(a.z, b.z) + sq_bf16x2(a.w, b.w));
  } else {
    return (sq_f32(a.x, b.x) + sq_f32(a.y, b.y)) + (sq_f32(a.z, b.z) + sq_f32(a.w, b.w));
  }
}

template <bool BF16>
__global__ __launch_bounds__(kThreads) void mse_partial_kernel(const u32x4* __restrict__ a,
                                                              const u32x4* __restrict__ b,
                                                              int64_t nvec, int64_t n,
                                                              double* __restrict__ partials) {
  constexpr int kPerVec = BF16 ? 8 : 4;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  double acc = 0.0;
  // Main loop: kUnroll independent 16-byte loads of each input in flight.
  for (; i + (kUnroll - 1) * stride < nvec; i += kUnroll * stride) {
    u32x4 va[kUnroll], vb[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      va[u] = __builtin_nontemporal_load(a + i + u * stride);
      vb[u] = __builtin_nontemporal_load(b + i + u * stride);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc += sq_vec<BF16>(va[u], vb[u]);
  }
  for (; i < nvec; i += stride) acc += sq_vec<BF16>(a[i], b[i]);
  // Ragged tail (fewer than one vector), handled by block 0.
  if (blockIdx.x == 0) {
    const int64_t e = nvec * kPerVec + threadIdx.x;
    if (e < n) {
      if (BF16) {
        const uint16_t* a16 = reinterpret_cast<const uint16_t*>(a);
        const uint16_t* b16 = reinterpret_cast<const uint16_t*>(b);
        const double d = (double)bf16_bits_to_float(a16[e]) - (double)bf16_bits_to_float(b16[e]);
        acc += d * d;
      } else {
        const float* a32 = reinterpret_cast<const float*>(a);
        const float* b32 = reinterpret_cast<const float*>(b);
        const double d = (double)a32[e] - (double)b32[e];
        acc += d * d;
      }
    }
  }
  const double s = block_sum(acc);
  if (threadIdx.x == 0) partials[blockIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void mse_final_kernel(const double* __restrict__ partials,
                                                            int nparts, int64_t n,
                                                            double* __restrict__ out) {
  // Eight loads in flight per thread; the order of the additions depends on
  // nparts alone, so the result is the same on every call.
  constexpr int U = 8;
  double acc = 0.0;
  int i = threadIdx.x;
  for (; i + (U - 1) * kThreads < nparts; i += U * kThreads) {
    double x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = partials[i + u * kThreads];
#pragma unroll
    for (int u = 0; u < U; ++u) acc += x[u];
  }
  for (; i < nparts; i += kThreads) acc += partials[i];
  const double s = block_sum(acc);
  if (threadIdx.x == 0) *out = s / (double)n;
}

}  // namespace

int mse_num_blocks(int64_t n, int dtype) {
  const int per_vec = (dtype == 0) ? 8 : 4;
  const int64_t nvec = n / per_vec;
  int64_t blocks = (nvec + (int64_t)kThreads * kUnroll * 4 - 1) / ((int64_t)kThreads * kUnroll * 4);
  if (blocks < 1) blocks = 1;
  if (blocks > kMaxBlocks) blocks = kMaxBlocks;
  return (int)blocks;
}

hipError_t launch_mse(const void* a, const void* b, int64_t n, int dtype, double* out,
                      double* partials, hipStream_t stream) {
  const int per_vec = (dtype == 0) ? 8 : 4;
  const int64_t nvec = n / per_vec;
  const int blocks = mse_num_blocks(n, dtype);
  if (dtype == 0) {
    hipLaunchKernelGGL(mse_partial_kernel<true>, dim3(blocks), dim3(kThreads), 0, stream,
                       (const u32x4*)a, (const u32x4*)b, nvec, n, partials);
  } else {
    hipLaunchKernelGGL(mse_partial_kernel<false>, dim3(blocks), dim3(kThreads), 0, stream,
                       (const u32x4*)a, (const u32x4*)b, nvec, n, partials);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mse_final_kernel, dim3(1), dim3(kThreads), 0, stream, partials, blocks, n, out);
  return hipGetLastError();
}

int mse_scratch_partials() { return kMaxBlocks; }

hipError_t mse_scratch(double** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  double* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    // With this device current: its copy of the array.  In host code the
    // array's name is only a stand-in, never a device address.
    void* addr = nullptr;
    e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    p = static_cast<double*>(addr);
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

hipError_t launch_mse_final(const double* partials, int nparts, int64_t n, double* out,
                            hipStream_t stream) {
  hipLaunchKernelGGL(mse_final_kernel, dim3(1), dim3(kThreads), 0, stream, partials, nparts, n, out);
  return hipGetLastError();
}

}  // namespace pab
