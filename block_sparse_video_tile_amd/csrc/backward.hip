// Block-sparse attention backward (dQ, dK, dV) for the VSA path on gfx950.
//
// h3-perf-stack commit log, sm_100a route entry: the forward-only route falls
// back to the tile-64 kernels, which keep the entire gradient path; this is
// that gradient for the block-sparse forward of attention.hip.  With the
// forward's LSE the probabilities are recomputed exactly,
//   P = exp(q.k/sqrt(D) - LSE_q),  D_q = sum_d dO_q O_q,
//   dP = dO V^T,  dS = P (dP - D_q),
//   dQ = dS K / sqrt(D),  dK_j += dS^T Q / sqrt(D),  dV_j += P^T dO,
// over the valid tokens of the selected blocks (a block listed m times in a
// row counts m times, as in the forward).
//
// Kernels
//   rowdot    D_q for every blocked row.
//   transpose blocked token-major -> d-major 64-token chunks (the layout the
//             forward uses for V^T), for K, Q and dO.
//   tmap      per key block j, the query blocks i whose row lists j, with the
//             multiplicity, ascending i (one thread per column, no atomics).
//   dq        one workgroup per query block, wave w owns 32 query rows:
//             S^T = K Q^T and dP^T = V dO^T with the key rows of K and V
//             staged kappa-permuted, so dS^T comes out in exactly the register
//             layout of the B operand of dQ^T += K^T dS^T (the forward's PV
//             arrangement with K^T in place of V^T).
//   dv, dk    one workgroup per key block, wave w owns 32 keys, streaming the
//             64-query sub-tiles of the query blocks that selected the block:
//             S = Q K^T and dP = dO V^T with the query rows staged
//             kappa-permuted, so P and dS feed dV^T += dO^T P and
//             dK^T += Q^T dS as B operands.  dV and dK are separate kernels so
//             that each stays within 256 VGPRs per lane.
// dv runs the forward kernel's software pipeline (S of the next sub-tile on
// the matrix cores while this sub-tile's P is formed, 32 fenced MFMA slots per
// sub-tile).  dq and dk keep S and dP of one sub-tile at a time (their
// operands leave no room for a second set), with the sub-tile copies
// double-buffered; dk lays each sub-tile out in 48 fenced slots so that the
// dS pairs of one query tile run beside the matrix products of the next (for
// dq, with a single lse per lane, the compiler's own order measured faster).
// All three take their query block or key block from per-XCD queues at run
// time (claim_row, counters in the workspace), as the forward's balanced
// launch does; the results do not depend on which workgroup takes which.

#include <algorithm>
#include <type_traits>

#include "attn_common.h"
#include "vsa_internal.h"

namespace vsa {
namespace {

using namespace tile;

constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------------------------ helpers

// D[row] = sum_d dO[row, d] * O[row, d] over all B*NH*Npad blocked rows.
template <bool F16>
__global__ __launch_bounds__(256) void rowdot_kernel(const uint4* __restrict__ o,
                                                     const uint4* __restrict__ dout,
                                                     float* __restrict__ dsum, int64_t rows) {
  const int64_t row = int64_t(blockIdx.x) * 16 + threadIdx.x / 16;
  const int unit = threadIdx.x % 16;
  float acc = 0.f;
  if (row < rows) {
    const uint4 a = o[row * 16 + unit], b = dout[row * 16 + unit];
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float alo, ahi, blo, bhi;
      if constexpr (F16) {
        alo = float(__builtin_bit_cast(_Float16, uint16_t(aw[e] & 0xffffu)));
        ahi = float(__builtin_bit_cast(_Float16, uint16_t(aw[e] >> 16)));
        blo = float(__builtin_bit_cast(_Float16, uint16_t(bw[e] & 0xffffu)));
        bhi = float(__builtin_bit_cast(_Float16, uint16_t(bw[e] >> 16)));
      } else {
        alo = __uint_as_float(aw[e] << 16);
        ahi = __uint_as_float(aw[e] & 0xffff0000u);
        blo = __uint_as_float(bw[e] << 16);
        bhi = __uint_as_float(bw[e] & 0xffff0000u);
      }
      acc = fmaf(alo, blo, fmaf(ahi, bhi, acc));
    }
  }
#pragma unroll
  for (int m = 8; m >= 1; m /= 2) acc += __shfl_xor(acc, m, 16);
  if (row < rows && unit == 0) dsum[row] = acc;
}

// Blocked token-major [B,NH,Npad,D] -> [B,NH,Npad/64,D,64]: one workgroup per
// 64-token chunk, transposed through LDS.
__global__ __launch_bounds__(256) void transpose_kernel(const uint4* __restrict__ x,
                                                        uint4* __restrict__ xt) {
  __shared__ __align__(16) uint16_t t[64][kHeadDim + 8];
  const int64_t c = blockIdx.x;  // chunk over B*NH*Npad/64
  const uint4* src = x + c * 64 * 16;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int idx = threadIdx.x + p * 256;
    *reinterpret_cast<uint4*>(&t[idx / 16][(idx % 16) * 8]) = src[idx];
  }
  __syncthreads();
  uint4* dst = xt + c * kHeadDim * 8;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int idx = threadIdx.x + p * 256;
    const int d = idx % kHeadDim, ku = idx / kHeadDim;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = uint32_t(t[ku * 8 + 2 * e][d]) | (uint32_t(t[ku * 8 + 2 * e + 1][d]) << 16);
    dst[d * 8 + ku] = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// Bounds of CSR row r, sanitised exactly as the forward does.
__device__ inline void row_bounds(const int32_t* row_ptr, int uniform_k, int64_t nnz, int64_t r,
                                  int64_t& beg, int64_t& end) {
  if (row_ptr != nullptr) {
    beg = min(max(int64_t(row_ptr[r]), int64_t(0)), nnz);
    end = min(max(int64_t(row_ptr[r + 1]), beg), nnz);
  } else {
    beg = r * uniform_k;
    end = beg + uniform_k;
  }
}

// Transposed block map: for (bh, j), the ascending query blocks i whose row
// lists j, packed as i | min(multiplicity, 65535) << 16, and their count.
// One wave per column (b, h, j): lane t counts j in row i0 + t of each block
// of 64 rows, and a ballot places the rows that list j in ascending order.
__global__ __launch_bounds__(256) void tmap_kernel(const int32_t* __restrict__ row_ptr,
                                                   const int32_t* __restrict__ col,
                                                   int uniform_k, int64_t nnz,
                                                   int32_t* __restrict__ tlist,
                                                   int32_t* __restrict__ tcount, VsaGeom g) {
  const int nb = g.nb;
  const int64_t ncols = int64_t(g.batch) * g.heads * nb;
  const int64_t task = int64_t(blockIdx.x) * 4 + threadIdx.x / 64;  // wave-uniform
  if (task >= ncols) return;
  const int64_t bh = task / nb;
  const int j = int(task % nb);
  const int lane = threadIdx.x % 64;
  int32_t* out = tlist + task * int64_t(nb);
  int cnt = 0;
  for (int i0 = 0; i0 < nb; i0 += 64) {
    const int i = i0 + lane;
    int m = 0;
    if (i < nb) {
      int64_t beg, end;
      row_bounds(row_ptr, uniform_k, nnz, bh * nb + i, beg, end);
      for (int64_t e = beg; e < end; ++e) m += col[e] == j ? 1 : 0;
    }
    const uint64_t listed = __ballot(m > 0);
    if (m > 0) out[cnt + __popcll(listed & ((uint64_t(1) << lane) - 1))] = i | (min(m, 65535) << 16);
    cnt += __popcll(listed);
  }
  if (lane == 0) tcount[task] = cnt;
}

// Per-lane copy offsets (16-byte units inside one 64-token sub-tile) of the
// padded LDS layouts: "row" tiles (64 token rows, kappa-permuted, 17 units
// per row) and "column" tiles (128 d rows of 64 tokens, 9 units per row).
// Positions past the buffer are clamped; their copies are not issued.
__device__ inline uint32_t row_tile_off(int pos) {
  pos = min(pos, kKUnits - 1);
  const int row = pos / kKRow, unit = pos % kKRow;
  return kappa(row) * 16 + (unit < 16 ? unit : 0);
}
__device__ inline uint32_t col_tile_off(int pos) {
  pos = min(pos, kVUnits - 1);
  const int row = pos / kVRow, unit = pos % kVRow;
  return row * 8 + (unit < 8 ? unit : 0);
}

// Copy one sub-tile with all NW waves of the workgroup.
template <int NW, int CHUNKS>
__device__ inline void copy_tile(const uint4* src, uint4* dst, int wave, int lane, bool row_tile) {
#pragma unroll
  for (int x = 0; x < (CHUNKS + NW - 1) / NW; ++x) {
    const int c = wave + x * NW;
    if (c < CHUNKS) {
      const int pos = c * 64 + lane;
      wave_copy_to_lds(src, row_tile ? row_tile_off(pos) : col_tile_off(pos), dst + c * 64);
    }
  }
}

__device__ inline void wait_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Store one wave's 32 x 128 accumulator tile (acc[dt] register j holds row
// l%32, column 32dt + 8(j/4) + 4(l/32) + j%4) times `mul` as element rows.
template <bool F16>
__device__ inline void store_rows(const f32x16 (&acc)[4], float mul, uint4* rows_base, int l32,
                                  int half) {
  uint2* dst = reinterpret_cast<uint2*>(rows_base + int64_t(l32) * 16);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
      dst[(dt * 32 + 8 * jj + 4 * half) / 4] =
          make_uint2(pack2<F16>(acc[dt][4 * jj] * mul, acc[dt][4 * jj + 1] * mul),
                     pack2<F16>(acc[dt][4 * jj + 2] * mul, acc[dt][4 * jj + 3] * mul));
}

// ------------------------------------------------------------------ work lists

// Each workgroup flattens its work (the CSR row for dQ, the key block's list
// of query blocks for dK/dV) into a list of 64-token sub-tile descriptors in
// LDS, kPassEntries entries at a time:
//   (64-token chunk index within the head) << 7 | (valid tokens - 1)
// and then streams the sub-tiles double-buffered: the copies of sub-tile n+1
// are in flight while sub-tile n is computed, one wait and one barrier per
// sub-tile.
constexpr int kPassEntries = 1024;

// Exclusive scan of cnt[0..m) in place by wave 0; *total receives the sum.
__device__ inline void scan_counts(int* cnt, int m, int* total, int wave, int lane) {
  if (wave != 0) return;
  constexpr int kPer = kPassEntries / 64;
  int loc[kPer];
  int sum = 0;
#pragma unroll
  for (int x = 0; x < kPer; ++x) {
    const int e = lane * kPer + x;
    loc[x] = sum;
    sum += e < m ? cnt[e] : 0;
  }
  int incl = sum;
#pragma unroll
  for (int d = 1; d < 64; d *= 2) {
    const int up = __shfl_up(incl, d);
    if (lane >= d) incl += up;
  }
  const int base = incl - sum;
#pragma unroll
  for (int x = 0; x < kPer; ++x) {
    const int e = lane * kPer + x;
    if (e < m) cnt[e] = base + loc[x];
  }
  if (lane == 63) *total = incl;
}

// Keep the scheduler from moving work across a slot boundary, and keep a
// VALU result in the slot where it is written (as in the forward kernel).
__device__ inline void slot_fence() { __builtin_amdgcn_sched_barrier(0); }
__device__ inline void pin_v(uint32_t& x) { asm volatile("" : "+v"(x)); }

// Clears the row-queue counters of the balanced launches (claim_row).
__global__ void bwd_queue_reset_kernel(unsigned int* queues) {
  if (threadIdx.x < 9) queues[threadIdx.x] = 0u;
}

// ------------------------------------------------------------------ dQ

template <int NW, bool F16>
__global__ __launch_bounds__(NW * 64) void dq_kernel(
    const uint4* __restrict__ q, const uint4* __restrict__ k, const uint4* __restrict__ v,
    const uint4* __restrict__ kt, const uint4* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ dsum, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col, int uniform_k, int64_t nnz, uint4* __restrict__ dq,
    unsigned int* __restrict__ queues, VsaGeom g, float scale_log2, float scale) {
  constexpr int kThreads = NW * 64;
  constexpr int kPassTiles = kPassEntries * (NW / 2);  // <= vol/64 sub-tiles per block
  // two buffer sets: K rows, V rows (kappa, padded), K^T (d-major, padded)
  __shared__ __align__(16) uint4 ks0[kKUnits];
  __shared__ __align__(16) uint4 vs0[kKUnits];
  __shared__ __align__(16) uint4 kts0[kVUnits];
  __shared__ __align__(16) uint4 ks1[kKUnits];
  __shared__ __align__(16) uint4 vs1[kKUnits];
  __shared__ __align__(16) uint4 kts1[kVUnits];
  __shared__ int tl[kPassTiles];
  __shared__ int esc[kPassEntries];
  __shared__ int ntl;
  const int64_t nrows = int64_t(g.batch) * g.heads * g.nb;
  __shared__ int64_t row_sh;   // row claimed from the queues (balanced launch)
  const int64_t r = queues != nullptr ? claim_row(queues, nrows, g, &row_sh)
                                      : xcd_remap(blockIdx.x, nrows);
  if (r < 0) return;
  const int i = int(r % g.nb);
  const int64_t bh = r / g.nb;
  const int cq = block_count(g, i);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64, half = lane / 32, l32 = lane & 31;
  // Key-half waves for edge blocks, as in the forward kernel: with 8 waves and
  // 5 or 6 groups of valid query rows, waves 4 and 6 share group 4 and waves 5
  // and 7 group 5, the first of each pair taking keys 0..31 of every sub-tile
  // and the second keys 32..63; the second's partial dQ is added to the
  // first's before the store.  Waves w and w+4 share a SIMD.
  const int ngroups = (cq + 31) / 32;
  const bool split = NW == 8 && (ngroups == 5 || ngroups == 6);  // workgroup-uniform
  const int qgroup = split && wave >= 4 ? 4 + (wave & 1) : wave;
  const int khalf = split && wave >= 4 ? (wave >> 1) & 1 : -1;   // -1: all keys
  const int kh = khalf > 0 ? 1 : 0;
  const int qrow = qgroup * 32 + l32;
  const bool active = qgroup * 32 < cq;
  const bool row_valid = qrow < cq;
  const int64_t row0 = bh * g.npad + int64_t(i) * g.vol;

  ev8 qf[8], df[8];
  float lse_l2 = INFINITY, dq_row = 0.f;
  if (active) {
    const uint4* qs = q + (row0 + qrow) * 16;
    const uint4* ds = dout + (row0 + qrow) * 16;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      qf[s] = as_ev8(qs[2 * s + half]);
      df[s] = as_ev8(ds[2 * s + half]);
    }
    if (row_valid) {
      lse_l2 = lse[row0 + qrow] * kLog2e;
      dq_row = dsum[row0 + qrow];
    }
  }
  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[dt][j] = 0.f;

  const uint4* const kbase = k + bh * g.npad * 16;
  const uint4* const vbase = v + bh * g.npad * 16;
  const uint4* const ktbase = kt + bh * (g.npad / kKvChunk) * kUnits;
  const int cpb = g.vol / kKvChunk;
  const int kread = l32 * kKRow + half, ktread = l32 * kVRow + half;

  auto issue = [&](int d, uint4* ksb, uint4* vsb, uint4* ktsb) {
    const int64_t chunk = d >> 7;
    copy_tile<NW, kKChunks>(kbase + chunk * kUnits, ksb, wave, lane, true);
    copy_tile<NW, kKChunks>(vbase + chunk * kUnits, vsb, wave, lane, true);
    copy_tile<NW, kVChunks>(ktbase + chunk * kUnits, ktsb, wave, lane, false);
  };
  // key-half wave: one 32-key tile (keys 32kh..) of S^T and dP^T, dQ^T from
  // the matching two 16-key steps
  const int kread_h = kread + kh * 32 * kKRow, ktread_h = ktread + 4 * kh;
  auto compute_half = [&](int d, const uint4* ksb, const uint4* vsb, const uint4* ktsb) {
    if (!active) return;
    f32x16 s, dp;
#pragma unroll
    for (int j2 = 0; j2 < 16; ++j2) s[j2] = dp[j2] = 0.f;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      s = mfma_32x32x16<F16>(as_ev8(ksb[kread_h + 2 * st]), qf[st], s);
      dp = mfma_32x32x16<F16>(as_ev8(vsb[kread_h + 2 * st]), df[st], dp);
    }
    const int valid = (d & 127) + 1;
    uint32_t dsw[2][4];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int t = 0; t < 8; t += 2) {
        float d2[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int jj = 8 * cc + t + u;
          const int key = 32 * kh + 16 * cc + 8 * half + t + u;
          const float p = key < valid
                              ? __builtin_amdgcn_exp2f(fmaf(s[jj], scale_log2, -lse_l2))
                              : 0.f;
          d2[u] = p * (dp[jj] - dq_row);
        }
        dsw[cc][t / 2] = pack2<F16>(d2[0], d2[1]);
      }
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const ev8 b = __builtin_bit_cast(ev8, make_uint4(dsw[cc][0], dsw[cc][1], dsw[cc][2],
                                                       dsw[cc][3]));
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        acc[dt] = mfma_32x32x16<F16>(as_ev8(ktsb[ktread_h + dt * 32 * kVRow + 2 * cc]), b,
                                     acc[dt]);
    }
  };
  auto compute = [&](int d, const uint4* ksb, const uint4* vsb, const uint4* ktsb) {
    if (!active) return;
    f32x16 s[2], dp[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int j2 = 0; j2 < 16; ++j2) s[mt][j2] = dp[mt][j2] = 0.f;
#pragma unroll
    for (int st = 0; st < 8; ++st)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        s[mt] = mfma_32x32x16<F16>(as_ev8(ksb[kread + mt * 32 * kKRow + 2 * st]), qf[st], s[mt]);
        dp[mt] = mfma_32x32x16<F16>(as_ev8(vsb[kread + mt * 32 * kKRow + 2 * st]), df[st], dp[mt]);
      }
    const int valid = (d & 127) + 1;
    // dS^T pairs, grouped by 16-key step cc (keys 16cc + 8*half + 0..7)
    uint32_t dsw[4][4];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
#pragma unroll
      for (int t = 0; t < 8; t += 2) {
        float d2[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int jj = 8 * (cc % 2) + t + u;
          const int key = 16 * cc + 8 * half + t + u;
          const float p = key < valid
                              ? __builtin_amdgcn_exp2f(fmaf(s[cc / 2][jj], scale_log2, -lse_l2))
                              : 0.f;
          d2[u] = p * (dp[cc / 2][jj] - dq_row);
        }
        dsw[cc][t / 2] = pack2<F16>(d2[0], d2[1]);
      }
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const ev8 b = __builtin_bit_cast(ev8, make_uint4(dsw[cc][0], dsw[cc][1], dsw[cc][2],
                                                       dsw[cc][3]));
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        acc[dt] = mfma_32x32x16<F16>(as_ev8(ktsb[ktread + dt * 32 * kVRow + 2 * cc]), b, acc[dt]);
    }
  };

  int64_t beg, end;
  row_bounds(row_ptr, uniform_k, nnz, r, beg, end);
  // the passes are compiled twice (full and key-half waves), each with its
  // own register allocation
  auto passes = [&](auto hv) __attribute__((always_inline)) {
  constexpr bool HV = decltype(hv)::value;
  auto work = [&](int d, const uint4* ksb, const uint4* vsb, const uint4* ktsb) {
    if constexpr (HV) compute_half(d, ksb, vsb, ktsb);
    else compute(d, ksb, vsb, ktsb);
  };
  for (int64_t e0 = beg; e0 < end; e0 += kPassEntries) {
    const int m = int(min(int64_t(kPassEntries), end - e0));
    for (int x = tid; x < m; x += kThreads) {
      const int j = col[e0 + x];
      esc[x] = (j >= 0 && j < g.nb) ? (block_count(g, j) + kKvChunk - 1) / kKvChunk : 0;
    }
    __syncthreads();
    scan_counts(esc, m, &ntl, wave, lane);
    __syncthreads();
    for (int x = tid; x < m; x += kThreads) {
      const int j = col[e0 + x];
      if (j >= 0 && j < g.nb) {
        const int cj = block_count(g, j);
        for (int sub = 0; sub * kKvChunk < cj; ++sub)
          tl[esc[x] + sub] = ((j * cpb + sub) << 7) | (min(kKvChunk, cj - sub * kKvChunk) - 1);
      }
    }
    __syncthreads();
    const int T = __builtin_amdgcn_readfirstlane(ntl);
    if (T == 0) continue;
    issue(__builtin_amdgcn_readfirstlane(tl[0]), ks0, vs0, kts0);
    wait_copies();
    __syncthreads();
    for (int n = 0; n < T; n += 2) {
      const int d0 = __builtin_amdgcn_readfirstlane(tl[n]);
      const int d1 = __builtin_amdgcn_readfirstlane(tl[min(n + 1, T - 1)]);
      if (n + 1 < T) issue(d1, ks1, vs1, kts1);
      work(d0, ks0, vs0, kts0);
      wait_copies();
      __syncthreads();
      if (n + 1 >= T) break;
      if (n + 2 < T) issue(__builtin_amdgcn_readfirstlane(tl[n + 2]), ks0, vs0, kts0);
      work(d1, ks1, vs1, kts1);
      wait_copies();
      __syncthreads();
    }
  }
  };
  if (khalf >= 0) passes(std::true_type());
  else passes(std::false_type());
  // key-half pairs: the second wave's partial dQ^T (wave 6's in ks1, wave 7's
  // in vs1, both free after the last barrier) is added to the first's
  const bool own_pad = split && khalf == 1;  // waves 6, 7: their own rows are padding
  if (split) {
    float* const part = (wave & 1) == 0 ? reinterpret_cast<float*>(ks1)
                                        : reinterpret_cast<float*>(vs1);
    if (own_pad && active) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) part[(dt * 16 + j) * 64 + lane] = acc[dt][j];
    }
    __syncthreads();
    if (khalf == 0 && active) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[dt][j] += part[(dt * 16 + j) * 64 + lane];
    }
    if (own_pad) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[dt][j] = 0.f;
    }
  }
  // dQ rows (this wave's own 32 rows); pad query rows are written as zero
  store_rows<F16>(acc, row_valid && !own_pad ? scale : 0.f, dq + (row0 + wave * 32) * 16, l32,
                  half);
}

// ------------------------------------------------------------------ dV, dK

// Per 64-query sub-tile the workgroup stages lse (log2 units, +inf for pad
// query rows) and D; register jj of query tile mt holds query
// 32mt + 16(jj/8) + 8*half + jj%8 (query rows staged kappa-permuted).
__device__ inline int query_of(int mt, int jj, int half) {
  return 32 * mt + 16 * (jj / 8) + 8 * half + jj % 8;
}

template <int NW, bool F16>
__global__ __launch_bounds__(NW * 64) void dk_kernel(
    const uint4* __restrict__ q, const uint4* __restrict__ k, const uint4* __restrict__ v,
    const uint4* __restrict__ qt, const uint4* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ dsum,
    const int32_t* __restrict__ tlist, const int32_t* __restrict__ tcount,
    uint4* __restrict__ grad, unsigned int* __restrict__ queues, VsaGeom g, float scale_log2,
    float scale) {
  constexpr int kThreads = NW * 64;
  constexpr int kPassTiles = kPassEntries * (NW / 2);
  // two buffer sets.  A operand of the first product(s): query rows (Q, and
  // dO for dK); A of the accumulation: d rows (dO^T for dV, Q^T for dK)
  __shared__ __align__(16) uint4 qs0[kKUnits];
  __shared__ __align__(16) uint4 ds0[kKUnits];
  __shared__ __align__(16) uint4 ts0[kVUnits];
  __shared__ __align__(16) uint4 qs1[kKUnits];
  __shared__ __align__(16) uint4 ds1[kKUnits];
  __shared__ __align__(16) uint4 ts1[kVUnits];
  __shared__ __align__(16) float lse_sh[2][kKvChunk];
  __shared__ __align__(16) float d_sh[2][kKvChunk];
  __shared__ int tl[kPassTiles];
  __shared__ float tm[kPassTiles];  // multiplicity of each sub-tile's query block
  __shared__ int esc[kPassEntries];
  __shared__ int ntl;
  const int64_t ncols = int64_t(g.batch) * g.heads * g.nb;
  __shared__ int64_t col_sh;   // column claimed from the queues (balanced launch)
  const int64_t c = queues != nullptr ? claim_row(queues, ncols, g, &col_sh)
                                      : xcd_remap(blockIdx.x, ncols);
  if (c < 0) return;
  const int j = int(c % g.nb);
  const int64_t bh = c / g.nb;
  const int cj = block_count(g, j);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64, half = lane / 32, l32 = lane & 31;
  // Query-half waves for edge key blocks: with 8 waves and 5 or 6 groups of
  // valid keys, waves 4 and 6 share key group 4 and waves 5 and 7 group 5,
  // the first of each pair taking queries 0..31 of every query sub-tile and
  // the second queries 32..63; the second's partial dK is added to the
  // first's before the store.  Waves w and w+4 share a SIMD.
  const int ngroups = (cj + 31) / 32;
  const bool split = NW == 8 && (ngroups == 5 || ngroups == 6);  // workgroup-uniform
  const int kgroup = split && wave >= 4 ? 4 + (wave & 1) : wave;
  const int qhalf = split && wave >= 4 ? (wave >> 1) & 1 : -1;   // -1: all queries
  const int qh = qhalf > 0 ? 1 : 0;
  const int key = kgroup * 32 + l32;
  const bool active = kgroup * 32 < cj;
  const int64_t key0 = bh * g.npad + int64_t(j) * g.vol;

  ev8 kf[8], vf[8];
  if (active) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      kf[s] = as_ev8(k[(key0 + key) * 16 + 2 * s + half]);
      vf[s] = as_ev8(v[(key0 + key) * 16 + 2 * s + half]);
    }
  }
  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) acc[dt][jj] = 0.f;

  const uint4* const qbase = q + bh * g.npad * 16;
  const uint4* const dbase = dout + bh * g.npad * 16;
  const uint4* const tbase = qt + bh * (g.npad / kKvChunk) * kUnits;
  const int cpb = g.vol / kKvChunk;
  const int qread = l32 * kKRow + half, tread = l32 * kVRow + half;

  // copies of one query sub-tile and its lse / D (threads 0..63, plain loads)
  auto issue = [&](int d, uint4* qsb, uint4* dsb, uint4* tsb, int set) {
    const int64_t chunk = d >> 7;
    copy_tile<NW, kKChunks>(qbase + chunk * kUnits, qsb, wave, lane, true);
    copy_tile<NW, kKChunks>(dbase + chunk * kUnits, dsb, wave, lane, true);
    copy_tile<NW, kVChunks>(tbase + chunk * kUnits, tsb, wave, lane, false);
    if (tid < kKvChunk) {
      const int64_t row = bh * g.npad + chunk * kKvChunk + tid;
      const bool ok = tid <= (d & 127);
      lse_sh[set][tid] = ok ? lse[row] * kLog2e : INFINITY;
      d_sh[set][tid] = ok ? dsum[row] : 0.f;
    }
  };
  // One query sub-tile in 48 fenced MFMA slots: S and dP of query tile 0
  // (16), those of tile 1 (16) with the dS pairs of tile 0 on the VALU, dK^T
  // for queries 0..31 (8) with the dS pairs of tile 1, dK^T for queries
  // 32..63 (8).  Operands are read from LDS three slots ahead, the lse and D
  // of a pair two pairs ahead.
  auto compute = [&](float mult, const uint4* qsb, const uint4* dsb, const uint4* tsb, int set) {
    if (!active) return;
    f32x16 s[2], dp[2];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) s[mt][jj] = dp[mt][jj] = 0.f;
    uint32_t bw[4][4];  // dS pairs: B operands of the 4 dK^T steps
    // pad keys of this block take no part (their rows are also stored as 0):
    // their K rows are zero, so P is finite there and the factor 0 removes it
    const float mlane = key < cj ? mult : 0.f;
    // pair k (0..15): query tile mt = k/8, step cc = 2mt + (k%8)/4, queries
    // t, t+1 of it with t = 2(k%4), i.e. rows 16cc + 8*half + t (kappa-staged)
    float2 lsep[3], dp2[3];
    auto read_pair = [&](int k) {
      const int cc = 2 * (k / 8) + (k % 8) / 4, t = 2 * (k % 4);
      const int qi = 16 * cc + 8 * half + t;
      lsep[k % 3] = *reinterpret_cast<const float2*>(&lse_sh[set][qi]);
      dp2[k % 3] = *reinterpret_cast<const float2*>(&d_sh[set][qi]);
    };
    auto ds_pair = [&](int k) {
      const int mt = k / 8, cc = 2 * mt + (k % 8) / 4, t = 2 * (k % 4);
      const float2 l = lsep[k % 3], dd = dp2[k % 3];
      const int jj = 8 * (cc % 2) + t;
      const float p0 = __builtin_amdgcn_exp2f(fmaf(s[mt][jj], scale_log2, -l.x)) * mlane;
      const float p1 = __builtin_amdgcn_exp2f(fmaf(s[mt][jj + 1], scale_log2, -l.y)) * mlane;
      bw[cc][t / 2] = pack2<F16>(p0 * (dp[mt][jj] - dd.x), p1 * (dp[mt][jj + 1] - dd.y));
      pin_v(bw[cc][t / 2]);
    };
    ev8 op[4];
    auto read_op = [&](int i) {
      if (i < 32) {
        const int mt = i / 16, st = (i % 16) / 2;
        const uint4* b = (i % 2 == 0) ? qsb : dsb;
        op[i % 4] = as_ev8(b[qread + mt * 32 * kKRow + 2 * st]);
      } else {
        const int x = i - 32, cc = x / 4, dt = x % 4;
        op[i % 4] = as_ev8(tsb[tread + dt * 32 * kVRow + 2 * cc]);
      }
    };
#pragma unroll
    for (int i = 0; i < 3; ++i) read_op(i);
    read_pair(0);
    read_pair(1);
    slot_fence();
#pragma unroll
    for (int i = 0; i < 48; ++i) {
      if (i + 3 < 48) read_op(i + 3);
      if (i < 32) {
        const int mt = i / 16, st = (i % 16) / 2;
        if (i % 2 == 0) s[mt] = mfma_32x32x16<F16>(op[i % 4], kf[st], s[mt]);
        else dp[mt] = mfma_32x32x16<F16>(op[i % 4], vf[st], dp[mt]);
        if (i >= 16 && i % 2 == 1) {
          const int k = (i - 16) / 2;
          if (k + 2 < 16) read_pair(k + 2);
          ds_pair(k);
        }
      } else {
        const int x = i - 32, cc = x / 4, dt = x % 4;
        const ev8 b = __builtin_bit_cast(ev8, make_uint4(bw[cc][0], bw[cc][1], bw[cc][2],
                                                         bw[cc][3]));
        acc[dt] = mfma_32x32x16<F16>(op[i % 4], b, acc[dt]);
        if (x < 8) {
          const int k = 8 + x;
          if (k + 2 < 16) read_pair(k + 2);
          ds_pair(k);
        }
      }
      slot_fence();
    }
  };

  // query-half wave: one 32-query tile (queries 32qh..) of S and dP, dK^T
  // from the matching two 16-query steps
  const int qread_h = qread + qh * 32 * kKRow, tread_h = tread + 4 * qh;
  auto compute_half = [&](float mult, const uint4* qsb, const uint4* dsb, const uint4* tsb,
                          int set) {
    if (!active) return;
    f32x16 s1, dp1;
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) s1[jj] = dp1[jj] = 0.f;
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      s1 = mfma_32x32x16<F16>(as_ev8(qsb[qread_h + 2 * st]), kf[st], s1);
      dp1 = mfma_32x32x16<F16>(as_ev8(dsb[qread_h + 2 * st]), vf[st], dp1);
    }
    const float mlane = key < cj ? mult : 0.f;
    uint32_t bw[2][4];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      // queries 32qh + 16cc + 8*half + 0..7
      const int q0 = 32 * qh + 16 * cc + 8 * half;
      float lq[8], dq8[8];
      *reinterpret_cast<float4*>(&lq[0]) = *reinterpret_cast<const float4*>(&lse_sh[set][q0]);
      *reinterpret_cast<float4*>(&lq[4]) = *reinterpret_cast<const float4*>(&lse_sh[set][q0 + 4]);
      *reinterpret_cast<float4*>(&dq8[0]) = *reinterpret_cast<const float4*>(&d_sh[set][q0]);
      *reinterpret_cast<float4*>(&dq8[4]) = *reinterpret_cast<const float4*>(&d_sh[set][q0 + 4]);
#pragma unroll
      for (int t = 0; t < 8; t += 2) {
        float x2[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int jj = 8 * cc + t + u;
          const float p = __builtin_amdgcn_exp2f(fmaf(s1[jj], scale_log2, -lq[t + u])) * mlane;
          x2[u] = p * (dp1[jj] - dq8[t + u]);
        }
        bw[cc][t / 2] = pack2<F16>(x2[0], x2[1]);
      }
    }
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const ev8 b = __builtin_bit_cast(ev8, make_uint4(bw[cc][0], bw[cc][1], bw[cc][2],
                                                       bw[cc][3]));
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        acc[dt] = mfma_32x32x16<F16>(as_ev8(tsb[tread_h + dt * 32 * kVRow + 2 * cc]), b,
                                     acc[dt]);
    }
  };

  const int nent = tcount[c];
  const int32_t* list = tlist + c * int64_t(g.nb);
  // the passes are compiled twice (full and query-half waves), each with its
  // own register allocation
  auto passes = [&](auto hv) __attribute__((always_inline)) {
  constexpr bool HV = decltype(hv)::value;
  auto work = [&](float mult, const uint4* qsb, const uint4* dsb, const uint4* tsb, int set) {
    if constexpr (HV) compute_half(mult, qsb, dsb, tsb, set);
    else compute(mult, qsb, dsb, tsb, set);
  };
  for (int e0 = 0; e0 < nent; e0 += kPassEntries) {
    const int m = min(kPassEntries, nent - e0);
    for (int x = tid; x < m; x += kThreads)
      esc[x] = (block_count(g, list[e0 + x] & 0xffff) + kKvChunk - 1) / kKvChunk;
    __syncthreads();
    scan_counts(esc, m, &ntl, wave, lane);
    __syncthreads();
    for (int x = tid; x < m; x += kThreads) {
      const int32_t ent = list[e0 + x];
      const int qi = ent & 0xffff;
      const float mult = float(uint32_t(ent) >> 16);
      const int cq = block_count(g, qi);
      for (int sub = 0; sub * kKvChunk < cq; ++sub) {
        tl[esc[x] + sub] = ((qi * cpb + sub) << 7) | (min(kKvChunk, cq - sub * kKvChunk) - 1);
        tm[esc[x] + sub] = mult;
      }
    }
    __syncthreads();
    const int T = __builtin_amdgcn_readfirstlane(ntl);
    if (T == 0) continue;
    issue(__builtin_amdgcn_readfirstlane(tl[0]), qs0, ds0, ts0, 0);
    wait_copies();
    __syncthreads();
    for (int n = 0; n < T; n += 2) {
      const float m0 = tm[n];
      const int d1 = __builtin_amdgcn_readfirstlane(tl[min(n + 1, T - 1)]);
      const float m1 = tm[min(n + 1, T - 1)];
      if (n + 1 < T) issue(d1, qs1, ds1, ts1, 1);
      work(m0, qs0, ds0, ts0, 0);
      wait_copies();
      __syncthreads();
      if (n + 1 >= T) break;
      if (n + 2 < T) issue(__builtin_amdgcn_readfirstlane(tl[n + 2]), qs0, ds0, ts0, 0);
      work(m1, qs1, ds1, ts1, 1);
      wait_copies();
      __syncthreads();
    }
  }
  };
  if (qhalf >= 0) passes(std::true_type());
  else passes(std::false_type());
  // query-half pairs: the second wave's partial dK^T (wave 6's in qs1, wave
  // 7's in ds1, both free after the last barrier) is added to the first's
  const bool own_pad = split && qhalf == 1;  // waves 6, 7: their own rows are padding
  if (split) {
    float* const part = (wave & 1) == 0 ? reinterpret_cast<float*>(qs1)
                                        : reinterpret_cast<float*>(ds1);
    if (own_pad && active) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) part[(dt * 16 + jj) * 64 + lane] = acc[dt][jj];
    }
    __syncthreads();
    if (qhalf == 0 && active) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) acc[dt][jj] += part[(dt * 16 + jj) * 64 + lane];
    }
    if (own_pad) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) acc[dt][jj] = 0.f;
    }
  }
  // rows of this wave's own keys; pad key rows are written as zero
  store_rows<F16>(acc, key < cj && !own_pad ? scale : 0.f, grad + (key0 + wave * 32) * 16,
                  l32, half);
}

// ------------------------------------------------------------------ dV, pipelined

// dV with the forward kernel's software pipeline.  One workgroup per key
// block, wave w owns keys 32w .. 32w+31 (their K fragments stay in VGPRs).
// The 64-query sub-tiles of the query blocks whose rows list the block stream
// through LDS, Q one sub-tile ahead of dO^T, so that while
//   P_n = 2^(S_n log2(e)/sqrt(D) - lse log2(e) + log2(multiplicity))
// feeds dV^T += dO^T_n P_n the matrix cores already compute
// S_{n+1} = Q_{n+1} K^T.  32 MFMA slots per sub-tile (16 for S_{n+1}, then 16
// for dV), the 16 exponential pairs of P_n spread over them.  Pad query rows
// carry lse = +inf in LDS (P = 0); pad key rows are stored as zero.
template <int NW, bool F16>
__global__ __launch_bounds__(NW * 64) void dv_kernel(
    const uint4* __restrict__ q, const uint4* __restrict__ k, const uint4* __restrict__ dot,
    const float* __restrict__ lse, const int32_t* __restrict__ tlist,
    const int32_t* __restrict__ tcount, uint4* __restrict__ dv, unsigned int* __restrict__ queues,
    VsaGeom g, float scale_log2) {
  constexpr int kThreads = NW * 64;
  constexpr int kPassTiles = kPassEntries * (NW / 2);
  // Q sub-tiles (kappa rows, the "K" role of the forward) and dO^T sub-tiles
  // (d rows, the "V^T" role); four arrays so the compiler sees that copies in
  // flight never alias the buffers being read
  __shared__ __align__(16) uint4 kbuf0[kKUnits];
  __shared__ __align__(16) uint4 kbuf1[kKUnits];
  __shared__ __align__(16) uint4 vbuf0[kVUnits];
  __shared__ __align__(16) uint4 vbuf1[kVUnits];
  __shared__ __align__(16) float lbuf[2][kKvChunk];
  __shared__ int tl[kPassTiles];
  __shared__ float tm[kPassTiles];
  __shared__ int esc[kPassEntries];
  __shared__ int ntl;
  const int64_t ncols = int64_t(g.batch) * g.heads * g.nb;
  __shared__ int64_t col_sh;   // column claimed from the queues (balanced launch)
  const int64_t c = queues != nullptr ? claim_row(queues, ncols, g, &col_sh)
                                      : xcd_remap(blockIdx.x, ncols);
  if (c < 0) return;
  const int j = int(c % g.nb);
  const int64_t bh = c / g.nb;
  const int cj = block_count(g, j);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64, half = lane / 32, l32 = lane & 31;
  // query-half waves for edge key blocks, as in the dK kernel
  const int ngroups = (cj + 31) / 32;
  const bool split = NW == 8 && (ngroups == 5 || ngroups == 6);  // workgroup-uniform
  const int kgroup = split && wave >= 4 ? 4 + (wave & 1) : wave;
  const int qhalf = split && wave >= 4 ? (wave >> 1) & 1 : -1;   // -1: all queries
  const int qh = qhalf > 0 ? 1 : 0;
  const int key = kgroup * 32 + l32;
  const bool active = kgroup * 32 < cj;
  const int64_t key0 = bh * g.npad + int64_t(j) * g.vol;

  ev8 kf[8];
  if (active) {
#pragma unroll
    for (int s = 0; s < 8; ++s) kf[s] = as_ev8(k[(key0 + key) * 16 + 2 * s + half]);
  }
  f32x16 acc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) acc[dt][jj] = 0.f;

  const uint4* const qbase = q + bh * g.npad * 16;
  const uint4* const tbase = dot + bh * (g.npad / kKvChunk) * kUnits;
  const float* const lbase = lse + bh * g.npad;
  const int cpb = g.vol / kKvChunk;
  constexpr int kMaxK = (kKChunks + NW - 1) / NW, kMaxV = (kVChunks + NW - 1) / NW;
  constexpr bool kSlotCopies = kMaxK + kMaxV <= 6;
  uint32_t koff[kMaxK], voff[kMaxV];
#pragma unroll
  for (int x = 0; x < kMaxK; ++x) koff[x] = row_tile_off((wave + x * NW) * 64 + lane);
#pragma unroll
  for (int x = 0; x < kMaxV; ++x) voff[x] = col_tile_off((wave + x * NW) * 64 + lane);
  auto src_of = [](const uint4* base, int d) { return base + int64_t(d >> 7) * kUnits; };
  auto copy_k = [&](const uint4* src, int x, uint4* dst) {
    if (tid / 64 + x * NW < kKChunks) wave_copy_to_lds(src, koff[x], dst + (wave + x * NW) * 64);
  };
  auto copy_v = [&](const uint4* src, int x, uint4* dst) {
    if (tid / 64 + x * NW < kVChunks) wave_copy_to_lds(src, voff[x], dst + (wave + x * NW) * 64);
  };
  auto load_k = [&](int d, uint4* dst) {
#pragma unroll
    for (int x = 0; x < kMaxK; ++x) copy_k(src_of(qbase, d), x, dst);
  };
  auto load_v = [&](int d, uint4* dst) {
#pragma unroll
    for (int x = 0; x < kMaxV; ++x) copy_v(src_of(tbase, d), x, dst);
  };
  // lse of the 64 query rows of sub-tile d, staged by wave 0: a plain load
  // issued early, the LDS write late
  auto lse_raw = [&](int d) { return wave == 0 ? lbase[int64_t(d >> 7) * kKvChunk + lane] : 0.f; };
  auto lse_put = [&](float raw, int d, float mult, float* dst) {
    if (wave == 0) dst[lane] = lane <= (d & 127) ? raw * kLog2e - __log2f(mult) : INFINITY;
  };
  const int kread = l32 * kKRow + half;
  const int vread = l32 * kVRow + half;
  // operand bases of a query-half wave: queries 32qh .. 32qh+31 of each sub-tile
  const int kread_h = kread + qh * 32 * kKRow, vread_h = vread + 4 * qh;

  const int nent = tcount[c];
  const int32_t* list = tlist + c * int64_t(g.nb);
  // the passes are compiled twice (full and query-half waves), each with its
  // own register allocation
  auto passes = [&](auto hv) __attribute__((always_inline)) {
  constexpr bool HV = decltype(hv)::value;
  f32x16 sa[2], sb[2];
  for (int e0 = 0; e0 < nent; e0 += kPassEntries) {
    const int m = min(kPassEntries, nent - e0);
    for (int x = tid; x < m; x += kThreads)
      esc[x] = (block_count(g, list[e0 + x] & 0xffff) + kKvChunk - 1) / kKvChunk;
    __syncthreads();
    scan_counts(esc, m, &ntl, wave, lane);
    __syncthreads();
    for (int x = tid; x < m; x += kThreads) {
      const int32_t ent = list[e0 + x];
      const int qi = ent & 0xffff;
      const float mult = float(uint32_t(ent) >> 16);
      const int cq = block_count(g, qi);
      for (int sub = 0; sub * kKvChunk < cq; ++sub) {
        tl[esc[x] + sub] = ((qi * cpb + sub) << 7) | (min(kKvChunk, cq - sub * kKvChunk) - 1);
        tm[esc[x] + sub] = mult;
      }
    }
    __syncthreads();
    const int T = __builtin_amdgcn_readfirstlane(ntl);
    if (T == 0) continue;
    // descriptor / multiplicity of sub-tile n; past the end the last one
    // repeats (its copies land in buffers that are not read again)
    auto desc_at = [&](int n) { return tl[min(n, T - 1)]; };
    auto mult_at = [&](int n) { return tm[min(n, T - 1)]; };

    int n = 0;
    int d0 = __builtin_amdgcn_readfirstlane(desc_at(0));
    int d1 = __builtin_amdgcn_readfirstlane(desc_at(1));
    int d2 = __builtin_amdgcn_readfirstlane(desc_at(2));
    load_k(d0, kbuf0);
    load_v(d0, vbuf0);
    load_k(d1, kbuf1);
    {
      const float raw = lse_raw(d0);
      wait_copies();
      lse_put(raw, d0, mult_at(0), lbuf[0]);
    }
    __syncthreads();
    if (active && !HV) {
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) sa[mt][jj] = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          sa[mt] = mfma_32x32x16<F16>(as_ev8(kbuf0[kread + mt * 32 * kKRow + 2 * s]), kf[s],
                                      sa[mt]);
    } else if (active) {
#pragma unroll
      for (int jj = 0; jj < 16; ++jj) sa[0][jj] = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s)
        sa[0] = mfma_32x32x16<F16>(as_ev8(kbuf0[kread_h + 2 * s]), kf[s], sa[0]);
    }
    // the first step copies Q_2 into kbuf0: every wave must be done with Q_0
    __syncthreads();

    // Finish sub-tile n (S_n in `cur`, lse_n in lcur) and compute S_{n+1}
    // into `nxt`.  kn: Q_{n+1}; kw receives Q_{n+2}; vn: dO^T_n; vw receives
    // dO^T_{n+1}; lnx receives lse_{n+1}.
    auto step = [&](f32x16 (&cur)[2], f32x16 (&nxt)[2], const uint4* kn, uint4* kw,
                    const uint4* vn, uint4* vw, const float* lcur, float* lnx) {
      const uint4* const sk = src_of(qbase, d2);
      const uint4* const sv = src_of(tbase, d1);
      const int d3 = desc_at(n + 3);  // LDS read; made uniform after the barrier
      const float m1 = mult_at(n + 1);
      const float raw = lse_raw(d1);
      if constexpr (!kSlotCopies) {
        load_k(d2, kw);
        load_v(d1, vw);
      }
      if (HV && active) {
        // query-half wave: one 32-query S tile, 8 + 8 MFMA slots
        uint32_t pw[2][4];
        ev8 opk[8], opv[8];
        float4 lq[2][2];
        auto read_k = [&](int u) { opk[u % 8] = as_ev8(kn[kread_h + 2 * u]); };
        auto read_v = [&](int w) {
          opv[w % 8] = as_ev8(vn[vread_h + (w % 4) * 32 * kVRow + 2 * (w / 4)]);
        };
        auto read_l = [&](int cc) {  // queries 32qh + 16cc + 8*half + 0..7
          lq[cc][0] = *reinterpret_cast<const float4*>(lcur + 32 * qh + 16 * cc + 8 * half);
          lq[cc][1] = *reinterpret_cast<const float4*>(lcur + 32 * qh + 16 * cc + 8 * half + 4);
        };
        read_l(0);
#pragma unroll
        for (int u = 0; u < 4; ++u) read_k(u);
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) nxt[0][jj] = 0.f;
        slot_fence();
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          if constexpr (kSlotCopies) {
#pragma unroll
            for (int x = 0; x < kMaxK; ++x)
              if (u == 1 + (x * 8) / kMaxK) copy_k(sk, x, kw);
#pragma unroll
            for (int x = 0; x < kMaxV; ++x)
              if (u == 9 + (x * 8) / kMaxV) copy_v(sv, x, vw);
          }
          if (u == 1) read_l(1);
          if (u < 8) {
            if (u % 4 == 0) {
#pragma unroll
              for (int x = 0; x < 4; ++x) {
                if (u + 4 < 8) read_k(u + 4 + x);
                else read_v(x);
              }
            }
            nxt[0] = mfma_32x32x16<F16>(opk[u % 8], kf[u], nxt[0]);
            // exponential pair u: queries t, t+1 of step u/4
            const int cc = u / 4, t = 2 * (u % 4);
            const float4 l4 = lq[cc][t / 4];
            const float la = (t % 4 == 0) ? l4.x : l4.z;
            const float lb = (t % 4 == 0) ? l4.y : l4.w;
            const float p0 = __builtin_amdgcn_exp2f(fmaf(cur[0][8 * cc + t], scale_log2, -la));
            const float p1 =
                __builtin_amdgcn_exp2f(fmaf(cur[0][8 * cc + t + 1], scale_log2, -lb));
            pw[cc][t / 2] = pack2<F16>(p0, p1);
            pin_v(pw[cc][t / 2]);
          } else {
            const int w = u - 8, cc = w / 4, dt = w % 4;
            if (w == 0) {
#pragma unroll
              for (int x = 0; x < 4; ++x) read_v(4 + x);
            }
            const ev8 pb = __builtin_bit_cast(
                ev8, make_uint4(pw[cc][0], pw[cc][1], pw[cc][2], pw[cc][3]));
            acc[dt] = mfma_32x32x16<F16>(opv[w % 8], pb, acc[dt]);
          }
          slot_fence();
        }
      } else if (!HV && active) {
        uint32_t pw[4][4];  // bf16 pairs of P: B operands of the 4 dV steps
        ev8 opk[8], opv[8];
        float4 lq[4][2];    // lse of the 8 queries of each dV step
        auto read_k = [&](int u) {
          opk[u % 8] = as_ev8(kn[kread + (u % 2) * 32 * kKRow + 2 * (u / 2)]);
        };
        auto read_v = [&](int w) {
          opv[w % 8] = as_ev8(vn[vread + (w % 4) * 32 * kVRow + 2 * (w / 4)]);
        };
        // queries of step cc: 16cc + 8*half + 0..7 (kappa-staged rows)
        auto read_l = [&](int cc) {
          lq[cc][0] = *reinterpret_cast<const float4*>(lcur + 16 * cc + 8 * half);
          lq[cc][1] = *reinterpret_cast<const float4*>(lcur + 16 * cc + 8 * half + 4);
        };
        read_l(0);
#pragma unroll
        for (int u = 0; u < 4; ++u) read_k(u);
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int jj = 0; jj < 16; ++jj) nxt[mt][jj] = 0.f;
        slot_fence();
#pragma unroll
        for (int u = 0; u < 32; ++u) {
          if constexpr (kSlotCopies) {
#pragma unroll
            for (int x = 0; x < kMaxK; ++x)
              if (u == 1 + (x * 16) / kMaxK) copy_k(sk, x, kw);
#pragma unroll
            for (int x = 0; x < kMaxV; ++x)
              if (u == 17 + (x * 16) / kMaxV) copy_v(sv, x, vw);
          }
          // lse of dV step cc read two steps' worth of slots ahead of its pairs
          if (u == 2) read_l(1);
          if (u == 10) read_l(2);
          if (u == 18) read_l(3);
          if (u < 16) {
            const int s = u / 2, mt = u % 2;
            if (u % 4 == 0) {
#pragma unroll
              for (int x = 0; x < 4; ++x) {
                if (u + 4 < 16) read_k(u + 4 + x);
                else read_v(x);
              }
            }
            nxt[mt] = mfma_32x32x16<F16>(opk[u % 8], kf[s], nxt[mt]);
          } else {
            const int w = u - 16, cc = w / 4, dt = w % 4;
            if (w % 4 == 0 && w + 4 < 16) {
#pragma unroll
              for (int x = 0; x < 4; ++x) read_v(w + 4 + x);
            }
            const ev8 pb = __builtin_bit_cast(
                ev8, make_uint4(pw[cc][0], pw[cc][1], pw[cc][2], pw[cc][3]));
            acc[dt] = mfma_32x32x16<F16>(opv[w % 8], pb, acc[dt]);
          }
          // exponential pair e (queries 2e%8, +1 of step e/4): pairs 0..11 in
          // even slots 0..22, pairs 12..15 in slots 24..27
          const int e = (u < 24) ? ((u % 2 == 0) ? u / 2 : -1) : ((u < 28) ? u - 12 : -1);
          if (e >= 0) {
            const int cc = e / 4, t = 2 * (e % 4);
            const float4 l4 = lq[cc][t / 4];
            const float la = (t % 4 == 0) ? l4.x : l4.z;
            const float lb = (t % 4 == 0) ? l4.y : l4.w;
            const float p0 =
                __builtin_amdgcn_exp2f(fmaf(cur[cc / 2][8 * (cc % 2) + t], scale_log2, -la));
            const float p1 =
                __builtin_amdgcn_exp2f(fmaf(cur[cc / 2][8 * (cc % 2) + t + 1], scale_log2, -lb));
            pw[cc][t / 2] = pack2<F16>(p0, p1);
            pin_v(pw[cc][t / 2]);
          }
          slot_fence();
        }
      } else if constexpr (kSlotCopies) {
#pragma unroll
        for (int x = 0; x < kMaxK; ++x) copy_k(sk, x, kw);
#pragma unroll
        for (int x = 0; x < kMaxV; ++x) copy_v(sv, x, vw);
      }
      wait_copies();
      lse_put(raw, d1, m1, lnx);
      __syncthreads();
      ++n;
      d0 = d1;
      d1 = d2;
      d2 = __builtin_amdgcn_readfirstlane(d3);
    };

    while (true) {
      step(sa, sb, kbuf1, kbuf0, vbuf0, vbuf1, lbuf[0], lbuf[1]);
      if (n >= T) break;
      step(sb, sa, kbuf0, kbuf1, vbuf1, vbuf0, lbuf[1], lbuf[0]);
      if (n >= T) break;
    }
  }
  };
  if (qhalf >= 0) passes(std::true_type());
  else passes(std::false_type());
  // query-half pairs: the second wave's partial dV^T (wave 6's in kbuf1, wave
  // 7's in vbuf1, both free after the last barrier) is added to the first's
  const bool own_pad = split && qhalf == 1;  // waves 6, 7: their own rows are padding
  if (split) {
    float* const part = (wave & 1) == 0 ? reinterpret_cast<float*>(kbuf1)
                                        : reinterpret_cast<float*>(vbuf1);
    if (own_pad && active) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) part[(dt * 16 + jj) * 64 + lane] = acc[dt][jj];
    }
    __syncthreads();
    if (qhalf == 0 && active) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) acc[dt][jj] += part[(dt * 16 + jj) * 64 + lane];
    }
    if (own_pad) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) acc[dt][jj] = 0.f;
    }
  }
  // rows of this wave's own keys; pad key rows are written as zero
  store_rows<F16>(acc, key < cj && !own_pad ? 1.f : 0.f, dv + (key0 + wave * 32) * 16, l32,
                  half);
}

template <int NW, bool F16>
hipError_t launch_bwd_nw(const VsaGeom& g, const BwdArgs& a, hipStream_t s) {
  const int64_t rows = int64_t(g.batch) * g.heads * g.nb;
  const float scale = 1.0f / sqrtf(float(g.head_dim));
  const float scale_log2 = scale * kLog2e;
  // Balanced launches (claim_row): a quarter more workgroups than rows or
  // columns, the queue counters cleared before each of the three kernels
  // (they run one after another on `s`, so one counter block serves all).
  const unsigned grid = unsigned(rows + std::max<int64_t>(8, rows / 4));
  auto reset = [&] {
    hipLaunchKernelGGL(bwd_queue_reset_kernel, dim3(1), dim3(64), 0, s, a.queues);
    return hipGetLastError();
  };
  hipError_t e = reset();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((dq_kernel<NW, F16>), dim3(grid), dim3(NW * 64), 0, s,
                     static_cast<const uint4*>(a.q), static_cast<const uint4*>(a.k),
                     static_cast<const uint4*>(a.v), static_cast<const uint4*>(a.kt),
                     static_cast<const uint4*>(a.dout), a.lse, a.dsum, a.row_ptr, a.col,
                     a.uniform_k, a.nnz, static_cast<uint4*>(a.dq), a.queues, g, scale_log2,
                     scale);
  if ((e = hipGetLastError()) != hipSuccess || (e = reset()) != hipSuccess) return e;
  hipLaunchKernelGGL((dv_kernel<NW, F16>), dim3(grid), dim3(NW * 64), 0, s,
                     static_cast<const uint4*>(a.q), static_cast<const uint4*>(a.k),
                     static_cast<const uint4*>(a.dot), a.lse, a.tlist, a.tcount,
                     static_cast<uint4*>(a.dv), a.queues, g, scale_log2);
  if ((e = hipGetLastError()) != hipSuccess || (e = reset()) != hipSuccess) return e;
  hipLaunchKernelGGL((dk_kernel<NW, F16>), dim3(grid), dim3(NW * 64), 0, s,
                     static_cast<const uint4*>(a.q), static_cast<const uint4*>(a.k),
                     static_cast<const uint4*>(a.v), static_cast<const uint4*>(a.qt),
                     static_cast<const uint4*>(a.dout), a.lse, a.dsum, a.tlist, a.tcount,
                     static_cast<uint4*>(a.dk), a.queues, g, scale_log2, scale);
  return hipGetLastError();
}

template <int NW>
hipError_t launch_bwd_typed(const VsaGeom& g, const BwdArgs& a, hipStream_t s) {
  return g.dtype == VSA_DTYPE_FP16 ? launch_bwd_nw<NW, true>(g, a, s)
                                   : launch_bwd_nw<NW, false>(g, a, s);
}

}  // namespace

hipError_t launch_attn_bwd(const VsaGeom& g, const BwdArgs& a, hipStream_t s) {
  const int64_t blocked_rows = int64_t(g.batch) * g.heads * g.npad;
  hipError_t e;
  if (g.dtype == VSA_DTYPE_FP16)
    hipLaunchKernelGGL(rowdot_kernel<true>, dim3(unsigned((blocked_rows + 15) / 16)), dim3(256),
                       0, s, static_cast<const uint4*>(a.o), static_cast<const uint4*>(a.dout),
                       a.dsum, blocked_rows);
  else
    hipLaunchKernelGGL(rowdot_kernel<false>, dim3(unsigned((blocked_rows + 15) / 16)), dim3(256),
                       0, s, static_cast<const uint4*>(a.o), static_cast<const uint4*>(a.dout),
                       a.dsum, blocked_rows);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const unsigned chunks = unsigned(blocked_rows / kKvChunk);
  const void* srcs[3] = {a.k, a.q, a.dout};
  void* dsts[3] = {a.kt, a.qt, a.dot};
  for (int t = 0; t < 3; ++t) {
    hipLaunchKernelGGL(transpose_kernel, dim3(chunks), dim3(256), 0, s,
                       static_cast<const uint4*>(srcs[t]), static_cast<uint4*>(dsts[t]));
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(tmap_kernel, dim3(unsigned((int64_t(g.batch) * g.heads * g.nb + 3) / 4)),
                     dim3(256), 0, s, a.row_ptr, a.col, a.uniform_k, a.nnz, a.tlist, a.tcount, g);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  switch (g.vol / 32) {
    case 2: return launch_bwd_typed<2>(g, a, s);
    case 4: return launch_bwd_typed<4>(g, a, s);
    case 6: return launch_bwd_typed<6>(g, a, s);
    case 8: return launch_bwd_typed<8>(g, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vsa
