// Measurement kernels for the roofline denominators of the hot path on
// gfx950: the matrix cores' sustained dense bf16 rate with the engine clock
// it runs at, and the bandwidth of a plain device-to-device copy.  They sit
// beside the hot path so that a benchmark can report its kernels against the
// machine it actually ran on as well as against the published figures.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "vsa_internal.h"

namespace vsa {
namespace {

typedef __bf16 ev8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kChains = 4;         // independent accumulator chains per wave
constexpr int kMfmaPerIter = 16;   // v_mfma_f32_32x32x16_bf16 per loop iteration

// Every wave runs `iters` iterations of 16 MFMAs (32x32x16 bf16: 32768 flops
// each) on four independent accumulators, reading the shader-clock counter
// (s_memtime) and the constant-rate wall clock (s_memrealtime) around its
// loop.  Lane 0 of wave w writes timing[4w] = cycles, timing[4w+1] = wall
// ticks, timing[4w+2] = the bit pattern of a sum of its results (keeps the
// products live).
__global__ __launch_bounds__(256) void mfma_peak_kernel(int iters,
                                                        unsigned long long* __restrict__ timing) {
  const int lane = threadIdx.x % 64;
  ev8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = __bf16(float((lane + e) % 7) * 0.125f);
    b[e] = __bf16(float((lane * 3 + e) % 5) * 0.0625f);
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[c][j] = 0.f;
  __syncthreads();
  const unsigned long long t0 = clock64();
  const unsigned long long w0 = wall_clock64();
  __builtin_amdgcn_sched_barrier(0);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < kMfmaPerIter; ++j)
      acc[j % kChains] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j % kChains], 0, 0, 0);
  }
  __builtin_amdgcn_sched_barrier(0);
  const unsigned long long t1 = clock64();
  const unsigned long long w1 = wall_clock64();
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[c][j];
  if (lane == 0) {
    const int64_t w = int64_t(blockIdx.x) * (blockDim.x / 64) + threadIdx.x / 64;
    timing[4 * w + 0] = t1 - t0;
    timing[4 * w + 1] = w1 - w0;
    timing[4 * w + 2] = __float_as_uint(s);
    timing[4 * w + 3] = 0ull;
  }
}

// Plain copy of n 16-byte units: one unit per thread, the grid covering the
// buffer in one pass (a grid-stride loop only beyond 2^31 - 1 workgroups);
// measured faster than grid-stride loops with several units per thread.
__global__ __launch_bounds__(256) void hbm_copy_kernel(const uint4* __restrict__ src,
                                                       uint4* __restrict__ dst, int64_t n) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = src[i];
}

}  // namespace

hipError_t launch_mfma_peak(int num_workgroups, int iters, uint64_t* timing, hipStream_t s) {
  hipLaunchKernelGGL(mfma_peak_kernel, dim3(unsigned(num_workgroups)), dim3(256), 0, s, iters,
                     reinterpret_cast<unsigned long long*>(timing));
  return hipGetLastError();
}

hipError_t launch_hbm_copy(const void* src, void* dst, int64_t bytes, hipStream_t s) {
  const int64_t n = bytes / 16;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, (int64_t(1) << 31) - 1);
  hipLaunchKernelGGL(hbm_copy_kernel, dim3(unsigned(blocks)), dim3(256), 0, s,
                     static_cast<const uint4*>(src), static_cast<uint4*>(dst), n);
  return hipGetLastError();
}

}  // namespace vsa
