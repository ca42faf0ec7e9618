// Block score and per-row top-k for the VSA hot path on gfx950.
//
// "FastVideo VSA" user guide, intro: for every query block every key/value
// block is scored and attention keeps the top-k; "Choose top-k": k counts key
// blocks per query block and is at most num_blocks.  The score of (i, j) is
// the fp32 dot product of the pooled query of block i and the pooled key of
// block j; equal scores go to the lower block index.
//
// One workgroup = 4 waves = 4 query-block rows of one (batch, head), one row
// per wave (the kernel is bound by latency, so more, smaller workgroups finish
// sooner: 31 -> 18 us on the 27280-token layer against two rows per wave).
// The head's pooled keys are staged through LDS 64 blocks at a time and
// shared by the 4 rows.  Selection is exact: each row's scores become unique 64-bit
// keys (order-preserving fp32 bits, then nb-1-j so lower j ranks higher), and
// the k-th largest key is found bit by bit with wave ballots.  The selected
// ids are then written ascending.  No atomics, so results are deterministic.

#include "vsa_internal.h"

namespace vsa {
namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerWave = 1;
constexpr int kRowsPerGroup = (kThreads / 64) * kRowsPerWave;
constexpr int kMaxChunks = 16;  // nb <= 1024
constexpr int kKeyStride = kHeadDim + 4;  // floats; 528-byte rows spread float4 reads over banks

__device__ inline uint32_t ordered_bits(float f) {
  const uint32_t u = __float_as_uint(f + 0.0f);  // -0 -> +0: equal scores share one key
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(kThreads) void score_topk_kernel(const float* __restrict__ qp,
                                                              const float* __restrict__ kp,
                                                              int topk, int32_t* __restrict__ col,
                                                              float* __restrict__ scores,
                                                              VsaGeom g) {
  __shared__ __align__(16) float ks[64][kKeyStride];
  __shared__ __align__(16) float qs[kRowsPerGroup][kHeadDim];
  const int nb = g.nb;
  const int bh = blockIdx.x;
  const int i0 = blockIdx.y * kRowsPerGroup;
  const int wave = threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  const int nchunks = (nb + 63) / 64;

  for (int idx = threadIdx.x; idx < kRowsPerGroup * kHeadDim; idx += kThreads) {
    const int r = idx / kHeadDim;
    const int i = min(i0 + r, nb - 1);
    qs[r][idx % kHeadDim] = qp[(int64_t(bh) * nb + i) * kHeadDim + idx % kHeadDim];
  }

  float sc[kRowsPerWave][kMaxChunks];
#pragma unroll
  for (int c = 0; c < kMaxChunks; ++c) {
    if (c < nchunks) {
      __syncthreads();
      // stage pooled keys of blocks 64c .. 64c+63 (zeros past nb)
      for (int idx = threadIdx.x; idx < 64 * (kHeadDim / 4); idx += kThreads) {
        const int jl = idx / (kHeadDim / 4);
        const int d4 = idx % (kHeadDim / 4);
        const int j = c * 64 + jl;
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (j < nb) v = reinterpret_cast<const float4*>(kp + (int64_t(bh) * nb + j) * kHeadDim)[d4];
        *reinterpret_cast<float4*>(&ks[jl][d4 * 4]) = v;
      }
      __syncthreads();
      float a[kRowsPerWave];
#pragma unroll
      for (int rr = 0; rr < kRowsPerWave; ++rr) a[rr] = 0.f;
#pragma unroll 8
      for (int d = 0; d < kHeadDim; d += 4) {
        const float4 kv = *reinterpret_cast<const float4*>(&ks[lane][d]);
#pragma unroll
        for (int rr = 0; rr < kRowsPerWave; ++rr) {
          const float4 x = *reinterpret_cast<const float4*>(&qs[wave * kRowsPerWave + rr][d]);
          a[rr] = fmaf(x.x, kv.x, a[rr]); a[rr] = fmaf(x.y, kv.y, a[rr]);
          a[rr] = fmaf(x.z, kv.z, a[rr]); a[rr] = fmaf(x.w, kv.w, a[rr]);
        }
      }
#pragma unroll
      for (int rr = 0; rr < kRowsPerWave; ++rr) sc[rr][c] = a[rr];
    }
  }

  const int lo_bits = nb > 1 ? 32 - __clz(nb - 1) : 0;
#pragma unroll
  for (int rr = 0; rr < kRowsPerWave; ++rr) {
    const int i = i0 + wave * kRowsPerWave + rr;
    if (i >= nb) continue;  // wave-uniform
    const int64_t row = int64_t(bh) * nb + i;
    uint32_t hi[kMaxChunks], lo[kMaxChunks];
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      const int j = c * 64 + lane;
      const bool valid = c < nchunks && j < nb;
      hi[c] = valid ? ordered_bits(sc[rr][c]) : 0u;   // real keys have hi >= 0x007fffff
      lo[c] = valid ? uint32_t(nb - 1 - j) : 0u;
      if (valid && scores != nullptr) scores[row * nb + j] = sc[rr][c];
    }
    // k-th largest high word
    uint32_t thi = 0;
    for (int bit = 31; bit >= 0; --bit) {
      const uint32_t cand = thi | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c)
        if (c < nchunks) cnt += __popcll(__ballot(hi[c] >= cand));
      if (cnt >= topk) thi = cand;
    }
    int above = 0;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c)
      if (c < nchunks) above += __popcll(__ballot(hi[c] > thi));
    // among keys whose high word equals thi, the largest low words fill the rest
    uint32_t tlo = 0;
    for (int bit = lo_bits - 1; bit >= 0; --bit) {
      const uint32_t cand = tlo | (1u << bit);
      int cnt = above;
#pragma unroll
      for (int c = 0; c < kMaxChunks; ++c)
        if (c < nchunks) cnt += __popcll(__ballot(hi[c] == thi && lo[c] >= cand));
      if (cnt >= topk) tlo = cand;
    }
    // ascending compaction: chunk-major, lane-minor is ascending block id
    int base = 0;
    const uint64_t below = (uint64_t(1) << lane) - 1;
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
      if (c < nchunks) {
        const int j = c * 64 + lane;
        const bool sel = j < nb && (hi[c] > thi || (hi[c] == thi && lo[c] >= tlo));
        const uint64_t m = __ballot(sel);
        const int pos = base + __popcll(m & below);
        if (sel && pos < topk) col[row * topk + pos] = j;
        base += __popcll(m);
      }
    }
  }
}

}  // namespace

hipError_t launch_score_topk(const VsaGeom& g, const float* qp, const float* kp, int topk,
                             int32_t* col, float* scores, hipStream_t s) {
  const dim3 grid(unsigned(int64_t(g.batch) * g.heads),
                  unsigned((g.nb + kRowsPerGroup - 1) / kRowsPerGroup));
  hipLaunchKernelGGL(score_topk_kernel, grid, dim3(kThreads), 0, s, qp, kp, topk, col, scores, g);
  return hipGetLastError();
}

}  // namespace vsa
