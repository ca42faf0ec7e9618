// Gate-compress (coarse) branch of VSA on gfx950.
//
// h3-perf-stack commit log, FastH3 example entry: the gate-compress branch
// pools per tile.  "FastVideo VSA" guide, "Checkpoint behavior": its output
// compensates the sparse branch through a learned to_gate_compress
// projection.  The pages give no formula; this computes attention among the
// per-tile pooled tokens: for every (batch, head) and query block i,
//   oc[i] = sum_j softmax_j(qbar_i . kbar_j / sqrt(D)) vbar_j
// over all nb blocks, with the standard head_size**-0.5 scale of "Verify
// routing and fallback".  The logits are the block scores of the top-k step,
// scaled.  Everything is fp32.
//
// The work is tiny (nb x nb x D per head): one wave per query-block row.
// Lane l scores keys l, l+64, ... (nb <= 1024), the row max and sum are wave
// reductions, and the probabilities go through LDS so that lane l can then
// accumulate output dimensions l and l+64 over all keys with coalesced reads
// of the pooled values.

#include "vsa_internal.h"

namespace vsa {
namespace {

constexpr int kWaves = 4;
constexpr int kMaxBlocks = 1024;

__device__ inline float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m /= 2) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m /= 2) x += __shfl_xor(x, m);
  return x;
}

// LDS written by some lanes of this wave is read by others: order them.
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ __launch_bounds__(kWaves * 64) void compress_attn_kernel(const float* __restrict__ qp,
                                                                    const float* __restrict__ kp,
                                                                    const float* __restrict__ vp,
                                                                    float* __restrict__ oc,
                                                                    VsaGeom g, float scale_log2) {
  __shared__ __align__(16) float qs[kWaves][kHeadDim];
  __shared__ float ps[kWaves][kMaxBlocks];
  const int wave = threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  const int nb = g.nb;
  const int64_t rows = int64_t(g.batch) * g.heads * nb;
  const int64_t r = int64_t(blockIdx.x) * kWaves + wave;
  if (r >= rows) return;  // no workgroup barrier below: waves only sync with themselves
  const int64_t bh = r / nb;

  qs[wave][lane] = qp[r * kHeadDim + lane];
  qs[wave][lane + 64] = qp[r * kHeadDim + lane + 64];
  wave_lds_sync();

  // logits in log2 units, one key per lane at a time
  const float4* kh = reinterpret_cast<const float4*>(kp + bh * nb * kHeadDim);
  const float4* q4 = reinterpret_cast<const float4*>(qs[wave]);
  float mx = -INFINITY;
  for (int j = lane; j < nb; j += 64) {
    float s = 0.f;
#pragma unroll 8
    for (int d4 = 0; d4 < kHeadDim / 4; ++d4) {
      const float4 kv = kh[int64_t(j) * (kHeadDim / 4) + d4];
      const float4 qv = q4[d4];
      s = fmaf(qv.x, kv.x, s);
      s = fmaf(qv.y, kv.y, s);
      s = fmaf(qv.z, kv.z, s);
      s = fmaf(qv.w, kv.w, s);
    }
    const float lg = s * scale_log2;
    ps[wave][j] = lg;
    mx = fmaxf(mx, lg);
  }
  mx = wave_max(mx);
  float sum = 0.f;
  for (int j = lane; j < nb; j += 64) {
    const float p = __builtin_amdgcn_exp2f(ps[wave][j] - mx);
    ps[wave][j] = p;
    sum += p;
  }
  sum = wave_sum(sum);
  wave_lds_sync();

  const float* vh = vp + bh * nb * kHeadDim;
  float o0 = 0.f, o1 = 0.f;
  for (int j = 0; j < nb; ++j) {
    const float p = ps[wave][j];
    o0 = fmaf(p, vh[int64_t(j) * kHeadDim + lane], o0);
    o1 = fmaf(p, vh[int64_t(j) * kHeadDim + lane + 64], o1);
  }
  const float inv = 1.f / sum;
  oc[r * kHeadDim + lane] = o0 * inv;
  oc[r * kHeadDim + lane + 64] = o1 * inv;
}

}  // namespace

hipError_t launch_compress_attn(const VsaGeom& g, const float* qp, const float* kp,
                                const float* vp, float* oc, hipStream_t s) {
  if (g.nb > kMaxBlocks) return hipErrorInvalidValue;
  const int64_t rows = int64_t(g.batch) * g.heads * g.nb;
  const float scale_log2 = 1.4426950408889634f / sqrtf(float(g.head_dim));
  hipLaunchKernelGGL(compress_attn_kernel, dim3(unsigned((rows + kWaves - 1) / kWaves)),
                     dim3(kWaves * 64), 0, s, qp, kp, vp, oc, g, scale_log2);
  return hipGetLastError();
}

}  // namespace vsa
