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
//   tmap      per key block j, the query blocks i whose row lists j, with the
//             multiplicity, ascending i (one thread per column, no atomics).
//   dq        one workgroup per query block, wave w owns 32 query rows:
//             S^T = K Q^T and dP^T = V dO^T with the key rows of K and V
//             staged kappa-permuted, so dS^T comes out in exactly the register
//             layout of the B operand of dQ^T += K^T dS^T (the forward's PV
//             arrangement with K^T in place of V^T); K^T is read from the K
//             rows with the transposing LDS read.
//   dkv       one workgroup per key block, wave w owns 32 keys, streaming the
//             64-query sub-tiles of the query blocks that selected the block:
//             S = Q K^T and dP = dO V^T with the query rows staged
//             kappa-permuted, so P and dS feed dV^T += dO^T P and
//             dK^T += Q^T dS as B operands; the A operands Q^T and dO^T are
//             read from the same row-major tiles with the transposing LDS
//             read.  S and dP are formed once for both gradients.
// dq keeps S and dP of one sub-tile at a time, with the sub-tile copies
// double-buffered (for dq, with a single lse per lane, the compiler's own
// order measured faster than fenced slots); dkv lays each 32-query half of a
// sub-tile out in 32 fenced MFMA slots.  Both take their query block or key
// block from per-XCD queues at run time (claim_row, counters in the
// workspace), as the forward's balanced launch does; the results do not
// depend on which workgroup takes which.

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

// Per-lane copy offset (16-byte units inside one 64-token sub-tile) of the
// padded row tiles: 64 token rows, kappa-permuted, 17 units per row (the pad
// unit re-reads unit 0).  Positions past the buffer are clamped; their copies
// are not issued.
__device__ inline uint32_t row_tile_off(int pos) {
  pos = min(pos, kKUnits - 1);
  const int row = pos / kKRow, unit = pos % kKRow;
  return kappa(row) * 16 + (unit < 16 ? unit : 0);
}

// Copy one row tile with all NW waves of the workgroup.
template <int NW>
__device__ inline void copy_tile(const uint4* src, uint4* dst, int wave, int lane) {
#pragma unroll
  for (int x = 0; x < (kKChunks + NW - 1) / NW; ++x) {
    const int c = wave + x * NW;
    if (c < kKChunks) wave_copy_to_lds(src, row_tile_off(c * 64 + lane), dst + c * 64);
  }
}

__device__ inline void wait_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ------------------------------------------------------------------ work lists

// Each workgroup flattens its work (the CSR row for dQ, the key block's list
// of query blocks for dK/dV) into a list of 64-token sub-tile descriptors in
// LDS, kPassEntries entries at a time (half as many in dkv, whose LDS holds
// the key block's V rows as well):
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

// Clears the row-queue counters and the tail-split counters of the balanced
// launches (claim_row).
__global__ void bwd_queue_reset_kernel(unsigned int* queues, unsigned int* flags, int nflags) {
  if (threadIdx.x < 9) queues[threadIdx.x] = 0u;
  for (int x = threadIdx.x; x < nflags; x += blockDim.x) flags[x] = 0u;
}

// Tail split of the balanced launches (the rule of the forward's, TailSplit):
// with at most 256 rows per queue, the last rows of each queue are handed out
// as two halves of their entries, so that the kernel's last round is made of
// half rows.  A gradient row is a plain sum over the entries, so the halves
// merge by addition: each half stores its accumulators (NT = 4 or 8 tiles
// per lane of every wave holding rows) with device-coherent stores (relaxed
// agent-scope atomics, past the XCD's non-coherent L2; a fence would write
// back or invalidate the whole L2 under the other workgroups), drains them,
// and counts itself done; the half that counts second adds the other's
// partial, a + b (the same bits whichever half adds), and writes the rows.
// Returns false for the half that finished first, which then leaves.
template <int NW, bool TWO>
__device__ __attribute__((always_inline)) inline bool bwd_tail_merge(
    unsigned int* flags, int32_t* ids, float* parts, int part, int wave, int lane, bool holds,
    f32x16 (&a)[4], f32x16 (&b)[4], int64_t id, unsigned int* done_sh) {
  const int slot = part >> 1, hf = part & 1;
  float* const mine = parts + (size_t(2 * slot + hf) * NW + wave) * kBwdSplitHalfFloatsPerWave;
  if (holds) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        __hip_atomic_store(mine + (dt * 16 + j) * 64 + lane, a[dt][j], __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        if constexpr (TWO)
          __hip_atomic_store(mine + (64 + dt * 16 + j) * 64 + lane, b[dt][j], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) *done_sh = atomicAdd(&flags[slot], 1u);
  __syncthreads();
  if (*done_sh == 0) return false;
  if (threadIdx.x == 0) ids[slot] = int32_t(id);
  float* const other =
      parts + (size_t(2 * slot + (1 - hf)) * NW + wave) * kBwdSplitHalfFloatsPerWave;
  if (holds) {
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        a[dt][j] += __hip_atomic_load(other + (dt * 16 + j) * 64 + lane, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
        if constexpr (TWO)
          b[dt][j] += __hip_atomic_load(other + (64 + dt * 16 + j) * 64 + lane,
                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
  }
  return true;
}

typedef short v4i16 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// i%4 of the 8-byte segments addressed by lanes 4e + i/4, e = 0..3.
__device__ inline v4i16 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(const_cast<void*>(p)));
}

// Store a 32 x 128 accumulator tile whose MFMA row m of tile dt holds column
// d = 64(m/16) + 8dt + 32((m%16)/8) + 4((m/4)%2) + m%4 (the order the
// transposing reads produce), times `mul`, as element rows: register j of
// lane l holds key l%32 and d = 64(j/8) + 8dt + 32((j/4)%2) + 4(l/32) + j%4.
template <bool F16>
__device__ inline void store_rows_perm(const f32x16 (&acc)[4], float mul, uint4* rows_base,
                                       int l32, int half) {
  uint2* dst = reinterpret_cast<uint2*>(rows_base + int64_t(l32) * 16);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int d0 = 64 * (jj / 2) + 8 * dt + 32 * (jj % 2) + 4 * half;
      dst[d0 / 4] = make_uint2(pack2<F16>(acc[dt][4 * jj] * mul, acc[dt][4 * jj + 1] * mul),
                               pack2<F16>(acc[dt][4 * jj + 2] * mul, acc[dt][4 * jj + 3] * mul));
    }
}

// Column operand of a kappa-permuted 64-row tile of 17-unit rows (the K
// tiles of dq, the Q and dO tiles of dkv), read with two transposing reads:
// lane l gets the 8 consecutive rows' (keys' or queries') elements of one
// column for the 16-row step starting at the tile byte offset `base`; `trb`
// is the lane's part of the address (tr_lane_base), dt selects the d tile.
// Within a group of 16 lanes the reads address 4 rows (68 dwords apart) and 4
// segments of 8 bytes at byte offsets 0, 8, 64, 72 of a 128-byte window, so
// the 16 two-dword spans 4e + {0, 2, 16, 18} (mod 32) cover every bank once.
// MFMA row m of the product then holds column
// d = 64(m/16) + 8dt + 32((m%16)/8) + 4((m/4)%2) + m%4 (store_rows_perm).
__device__ inline int tr_lane_base(int lane) {
  const int half = lane / 32;
  return (4 * half + (lane & 15) / 4) * (kKRow * 16) + 128 * ((lane >> 4) & 1) +
         64 * ((lane & 3) >> 1) + 8 * (lane & 1);
}
// The operand at tile byte offset trb + base + 16dt: the first read takes rows
// 8*half + 0..3 of the step, the second 4..7 (kappa places them 8 rows on).
__device__ inline ev8 tr_operand(const uint4* tile, int off) {
  const char* p = reinterpret_cast<const char*>(tile) + off;
  const v4i16 lo = lds_read_tr16(p);
  const v4i16 hi = lds_read_tr16(p + 8 * (kKRow * 16));
  return __builtin_bit_cast(ev8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// ------------------------------------------------------------------ dQ

template <int NW, bool F16, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void dq_kernel(
    const uint4* __restrict__ q, const uint4* __restrict__ k, const uint4* __restrict__ v,
    const uint4* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ dsum, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col, int uniform_k, int64_t nnz, uint4* __restrict__ dq,
    unsigned int* __restrict__ queues, VsaGeom g, float scale_log2, float scale,
    unsigned int* __restrict__ split_flags, int32_t* __restrict__ split_ids,
    float* __restrict__ split_part, int tail_split) {
  constexpr int kThreads = NW * 64;
  constexpr int kPassTiles = kPassEntries * (NW / 2);  // <= vol/64 sub-tiles per block
  // two buffer sets: K rows and V rows (kappa, padded); K^T is read from the
  // K rows with the transposing read
  __shared__ __align__(16) uint4 ks0[kKUnits];
  __shared__ __align__(16) uint4 vs0[kKUnits];
  __shared__ __align__(16) uint4 ks1[kKUnits];
  __shared__ __align__(16) uint4 vs1[kKUnits];
  __shared__ int tl[kPassTiles];
  __shared__ int esc[kPassEntries];
  __shared__ int ntl;
  const int64_t nrows = int64_t(g.batch) * g.heads * g.nb;
  __shared__ int64_t row_sh;   // row claimed from the queues (balanced launch)
  __shared__ int part_sh;      // -1, or 2 * split slot + half
  __shared__ unsigned int done_sh;
  const int64_t r = queues != nullptr
                        ? claim_row(queues, nrows, g, &row_sh, nullptr, SPLIT ? uint32_t(tail_split) : 0u,
                                    SPLIT ? &part_sh : nullptr)
                        : xcd_remap(blockIdx.x, nrows);
  if (r < 0) return;
  // -1 (whole), or 2 * split slot + half; SPLIT: the launch splits rows
  const int part = SPLIT && queues != nullptr ? part_sh : -1;  // workgroup-uniform
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
  const int cpb = g.vol / kKvChunk;
  const int kread = l32 * kKRow + half, trb = tr_lane_base(lane);

  auto issue = [&](int d, uint4* ksb, uint4* vsb) {
    const int64_t chunk = d >> 7;
    copy_tile<NW>(kbase + chunk * kUnits, ksb, wave, lane);
    copy_tile<NW>(vbase + chunk * kUnits, vsb, wave, lane);
  };
  // key-half wave: one 32-key tile (keys 32kh..) of S^T and dP^T, dQ^T from
  // the matching two 16-key steps
  const int kread_h = kread + kh * 32 * kKRow, trb_h = trb + kh * 32 * (kKRow * 16);
  auto compute_half = [&](int d, const uint4* ksb, const uint4* vsb) {
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
    auto pairs = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int t = 0; t < 8; t += 2) {
          float d2[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int jj = 8 * cc + t + u;
            const int key = 32 * kh + 16 * cc + 8 * half + t + u;
            float p = __builtin_amdgcn_exp2f(fmaf(s[jj], scale_log2, -lse_l2));
            if constexpr (decltype(masked)::value) p = key < valid ? p : 0.f;
            d2[u] = p * (dp[jj] - dq_row);
          }
          dsw[cc][t / 2] = pack2<F16>(d2[0], d2[1]);
        }
    };
    if (valid == kKvChunk) pairs(std::false_type());
    else pairs(std::true_type());
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      const ev8 b = __builtin_bit_cast(ev8, make_uint4(dsw[cc][0], dsw[cc][1], dsw[cc][2],
                                                       dsw[cc][3]));
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        acc[dt] = mfma_32x32x16<F16>(tr_operand(ksb, trb_h + cc * 16 * (kKRow * 16) + 16 * dt),
                                     b, acc[dt]);
    }
  };
  auto compute = [&](int d, const uint4* ksb, const uint4* vsb) {
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
    // dS^T pairs, grouped by 16-key step cc (keys 16cc + 8*half + 0..7); the
    // comparison with the valid count only for a partial sub-tile
    uint32_t dsw[4][4];
    auto pairs = [&](auto masked) __attribute__((always_inline)) {
#pragma unroll
      for (int cc = 0; cc < 4; ++cc)
#pragma unroll
        for (int t = 0; t < 8; t += 2) {
          float d2[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int jj = 8 * (cc % 2) + t + u;
            const int key = 16 * cc + 8 * half + t + u;
            float p = __builtin_amdgcn_exp2f(fmaf(s[cc / 2][jj], scale_log2, -lse_l2));
            if constexpr (decltype(masked)::value) p = key < valid ? p : 0.f;
            d2[u] = p * (dp[cc / 2][jj] - dq_row);
          }
          dsw[cc][t / 2] = pack2<F16>(d2[0], d2[1]);
        }
    };
    if (valid == kKvChunk) pairs(std::false_type());
    else pairs(std::true_type());
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const ev8 b = __builtin_bit_cast(ev8, make_uint4(dsw[cc][0], dsw[cc][1], dsw[cc][2],
                                                       dsw[cc][3]));
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        acc[dt] = mfma_32x32x16<F16>(tr_operand(ksb, trb + cc * 16 * (kKRow * 16) + 16 * dt), b,
                                     acc[dt]);
    }
  };

  int64_t beg, end;
  row_bounds(row_ptr, uniform_k, nnz, r, beg, end);
  if (part >= 0) {
    // a half of a split row: the first or the second half of its entries
    const int64_t mid = beg + (end - beg) / 2;
    if (part & 1) beg = mid;
    else end = mid;
  }
  // the passes are compiled twice (full and key-half waves), each with its
  // own register allocation
  auto passes = [&](auto hv) __attribute__((always_inline)) {
  constexpr bool HV = decltype(hv)::value;
  auto work = [&](int d, const uint4* ksb, const uint4* vsb) {
    if constexpr (HV) compute_half(d, ksb, vsb);
    else compute(d, ksb, vsb);
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
    issue(__builtin_amdgcn_readfirstlane(tl[0]), ks0, vs0);
    wait_copies();
    __syncthreads();
    for (int n = 0; n < T; n += 2) {
      const int d0 = __builtin_amdgcn_readfirstlane(tl[n]);
      const int d1 = __builtin_amdgcn_readfirstlane(tl[min(n + 1, T - 1)]);
      if (n + 1 < T) issue(d1, ks1, vs1);
      work(d0, ks0, vs0);
      wait_copies();
      __syncthreads();
      if (n + 1 >= T) break;
      if (n + 2 < T) issue(__builtin_amdgcn_readfirstlane(tl[n + 2]), ks0, vs0);
      work(d1, ks1, vs1);
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
  if (SPLIT && part >= 0 && !bwd_tail_merge<NW, false>(split_flags, split_ids, split_part, part, wave,
                                                lane, active && !own_pad, acc, acc, r, &done_sh))
    return;
  // dQ rows (this wave's own 32 rows); pad query rows are written as zero
  store_rows_perm<F16>(acc, row_valid && !own_pad ? scale : 0.f, dq + (row0 + wave * 32) * 16, l32,
                  half);
}

// ------------------------------------------------------------------ dK and dV together

// Query sub-tiles of the fused dK/dV kernel: 64 query rows, kappa-permuted,
// of 16 data units and 1 pad unit (272 B), as the forward's K tiles.  They
// are read as rows (ds_read_b128: the A operands of S = Q K^T and
// dP = dO V^T; 8 consecutive rows at the same unit fall on distinct banks)
// and as columns (tr_operand: the A operands of dK^T += Q^T dS and
// dV^T += dO^T P).
constexpr int kQRow = kKRow;
constexpr int kQUnits = 64 * kQRow;    // 1088 16-byte units (17 KB)
constexpr int kQChunks = kQUnits / 64;  // 17 wave-loads of 1 KB

// Source unit (within a 64-token sub-tile) of LDS position pos of a query
// sub-tile; the pad unit re-reads unit 0 of its row.
__device__ inline uint32_t qtile_off(int pos) {
  const int row = pos / kQRow, unit = pos % kQRow;
  return kappa(row) * 16 + (unit < 16 ? unit : 0);
}

// dK and dV of one key block in one pass over the query sub-tiles that
// selected it.  One workgroup per key block, wave w owns keys 32w .. 32w+31:
// their K fragments stay in VGPRs, the block's V rows are staged in LDS once.
// Each 64-query sub-tile (Q and dO rows, kappa-permuted, and the queries' lse
// and D) is copied into LDS once, double-buffered, and every wave takes it in
// two 32-query halves of 32 fenced MFMA slots:
//   slots  0.. 7  S   = Q K^T    (A: Q rows, B: K fragments)
//   slots  8..15  dP  = dO V^T   (A: dO rows, B: V rows), with the 8
//                 exponential pairs P = 2^(S log2(e)/sqrt(D) - lse log2(e) +
//                 log2(multiplicity)) in slots 10..17
//   slots 16..23  dV^T += dO^T P (A: dO columns), with the 8 pairs
//                 dS = P (dP - D) in slots 18..25
//   slots 24..31  dK^T += Q^T dS (A: Q columns)
// so S and dP are formed once for both gradients.  The registers of S, dP,
// P and dS of one half, the two accumulator sets and the K fragments fit the
// 256 of two waves per SIMD; V, the largest operand held per wave otherwise,
// is read from LDS.  Pad query rows carry lse = +inf (P = 0) and D = 0.  A
// pad key's P and dS reach only that key's own columns of dV^T and dK^T
// (each column of these products is one key), and those rows are stored as
// 0, so pad keys need no masking.
// Edge key blocks of 5 or 6 key groups split waves 4..7 by query halves, as
// the separate kernels did.
template <int NW, bool F16, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void dkv_kernel(
    const uint4* __restrict__ q, const uint4* __restrict__ k, const uint4* __restrict__ v,
    const uint4* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ dsum, const int32_t* __restrict__ tlist,
    const int32_t* __restrict__ tcount, uint4* __restrict__ dk, uint4* __restrict__ dv,
    unsigned int* __restrict__ queues, VsaGeom g, float scale_log2, float scale,
    unsigned int* __restrict__ split_flags, int32_t* __restrict__ split_ids,
    float* __restrict__ split_part, int tail_split) {
  constexpr int kThreads = NW * 64;
  constexpr int kEntries = kPassEntries / 2;       // query blocks per pass
  constexpr int kTiles = kEntries * (NW / 2);      // <= vol/64 sub-tiles per query block
  constexpr int kVRows = NW * 32 * kKRow;          // the key block's V rows, padded
  __shared__ __align__(16) uint4 vrows[kVRows];
  __shared__ __align__(16) uint4 qs0[kQUnits];
  __shared__ __align__(16) uint4 ds0[kQUnits];
  __shared__ __align__(16) uint4 qs1[kQUnits];
  __shared__ __align__(16) uint4 ds1[kQUnits];
  __shared__ __align__(16) float lse_sh[2][kKvChunk];
  __shared__ __align__(16) float d_sh[2][kKvChunk];
  __shared__ int tl[kTiles];
  __shared__ uint16_t tm[kTiles];  // multiplicity of each sub-tile's query block
  __shared__ int esc[kEntries];
  __shared__ int ntl;
  static_assert(kVRows * 16 + 4 * kQUnits * 16 + 4 * kKvChunk * 4 + kTiles * 6 + kEntries * 4 +
                        64 <= 160 * 1024,
                "the fused kernel's LDS must fit one CU");
  const int64_t ncols = int64_t(g.batch) * g.heads * g.nb;
  __shared__ int64_t col_sh;  // column claimed from the queues (balanced launch)
  __shared__ int part_sh;     // -1, or 2 * split slot + half
  __shared__ unsigned int done_sh;
  const int64_t c = queues != nullptr
                        ? claim_row(queues, ncols, g, &col_sh, nullptr, SPLIT ? uint32_t(tail_split) : 0u,
                                    SPLIT ? &part_sh : nullptr)
                        : xcd_remap(blockIdx.x, ncols);
  if (c < 0) return;
  // -1 (whole), or 2 * split slot + half; SPLIT: the launch splits rows
  const int part = SPLIT && queues != nullptr ? part_sh : -1;  // workgroup-uniform
  const int j = int(c % g.nb);
  const int64_t bh = c / g.nb;
  const int cj = block_count(g, j);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const int lane = tid % 64, half = lane / 32, l32 = lane & 31;
  const int ngroups = (cj + 31) / 32;
  const bool split = NW == 8 && (ngroups == 5 || ngroups == 6);  // workgroup-uniform
  const int kgroup = split && wave >= 4 ? 4 + (wave & 1) : wave;
  const int qhalf = split && wave >= 4 ? (wave >> 1) & 1 : -1;   // -1: all queries
  const int key = kgroup * 32 + l32;
  const bool active = kgroup * 32 < cj;
  const int64_t key0 = bh * g.npad + int64_t(j) * g.vol;
  // 32-query halves of every sub-tile this wave takes (wave-uniform)
  const int hs_lo = qhalf > 0 ? 1 : 0, hs_hi = qhalf == 0 ? 0 : 1;

  // the key block's V rows (keys in order, 17-unit rows), all waves
#pragma unroll
  for (int x = 0; x < (kVRows / 64 + NW - 1) / NW; ++x) {
    const int ch = wave + x * NW;
    if (ch < kVRows / 64) {
      const int pos = ch * 64 + lane;
      const int row = pos / kKRow, unit = pos % kKRow;
      wave_copy_to_lds(v + key0 * 16, uint32_t(row * 16 + (unit < 16 ? unit : 0)),
                       vrows + ch * 64);
    }
  }
  ev8 kf[8];
  if (active) {
#pragma unroll
    for (int s = 0; s < 8; ++s) kf[s] = as_ev8(k[(key0 + key) * 16 + 2 * s + half]);
  }
  f32x16 accv[4], acck[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) accv[dt][jj] = acck[dt][jj] = 0.f;

  const uint4* const qbase = q + bh * g.npad * 16;
  const uint4* const dbase = dout + bh * g.npad * 16;
  const float* const lbase = lse + bh * g.npad;
  const float* const dsbase = dsum + bh * g.npad;
  const int cpb = g.vol / kKvChunk;
  constexpr int kMaxC = (kQChunks + NW - 1) / NW;
  uint32_t qoff[kMaxC];
#pragma unroll
  for (int x = 0; x < kMaxC; ++x) qoff[x] = qtile_off(min((wave + x * NW) * 64 + lane, kQUnits - 1));
  // copies of query sub-tile d (Q and dO rows) into one buffer set
  auto issue = [&](int d, uint4* qsb, uint4* dsb) {
    const int64_t chunk = d >> 7;
#pragma unroll
    for (int x = 0; x < kMaxC; ++x)
      if (wave + x * NW < kQChunks) {
        wave_copy_to_lds(qbase + chunk * kUnits, qoff[x], qsb + (wave + x * NW) * 64);
        wave_copy_to_lds(dbase + chunk * kUnits, qoff[x], dsb + (wave + x * NW) * 64);
      }
  };
  // lse (log2 units) and D of the sub-tile's 64 queries, staged by wave 0:
  // plain loads issued early, the LDS writes after the copies' wait
  struct Raw { float l, d; };
  auto raw_of = [&](int d) -> Raw {
    if (wave != 0) return {0.f, 0.f};
    const int64_t row = int64_t(d >> 7) * kKvChunk + lane;
    return {lbase[row], dsbase[row]};
  };
  // the sub-tile's query block is listed `mult` times: P carries that factor
  // as -log2(mult) in the staged lse
  auto put = [&](Raw r, int d, int set, float mult) {
    if (wave == 0) {
      const bool ok = lane <= (d & 127);
      lse_sh[set][lane] = ok ? r.l * kLog2e - __log2f(mult) : INFINITY;
      d_sh[set][lane] = ok ? r.d : 0.f;
    }
  };

  // per-lane operand bases: row reads (query row l32, unit half), V row of
  // this lane's key, and the byte offset of the transposing reads (query row
  // 4*half + (lane%16)/4 of a 16-query step, kappa-placed; the segment of d
  // columns 64*((lane/16)%2) + 32*((lane%4)/2) + 4*(lane%2) .. +3, plus 8dt)
  const int qread = l32 * kQRow + half;
  const int vread = key * kKRow + half;
  const int trb = tr_lane_base(lane);

  // one 32-query half hs of a sub-tile held in (qsb, dsb), lse / D in set
  auto half_tile = [&](int hs, const uint4* qsb, const uint4* dsb, int set)
      __attribute__((always_inline)) {
    f32x16 s, dp;
#pragma unroll
    for (int jj = 0; jj < 16; ++jj) s[jj] = dp[jj] = 0.f;
    uint32_t pw[2][4], dsw[2][4];
    const int rbase = qread + hs * 32 * kQRow;
    const int hsoff = hs * 32 * (kQRow * 16);
    // A operand of a transposed product, 16-query step cc, d tile dt
    auto tr_op = [&](const uint4* tile, int hsoff, int cc, int dt) -> ev8 {
      return tr_operand(tile, trb + hsoff + cc * 16 * (kQRow * 16) + 16 * dt);
    };
    // A operand of slot i, read 2 slots ahead, and the V operand of slots
    // 8..15 one slot ahead (longer leads spill at 256 registers)
    ev8 opa[3], opv[2];
    auto read_op = [&](int i) {
      if (i < 8) {
        opa[i % 3] = as_ev8(qsb[rbase + 2 * i]);
      } else if (i < 16) {
        opa[i % 3] = as_ev8(dsb[rbase + 2 * (i - 8)]);
      } else if (i < 24) {
        const int x = i - 16;
        opa[i % 3] = tr_op(dsb, hsoff, x / 4, x % 4);
      } else {
        const int x = i - 24;
        opa[i % 3] = tr_op(qsb, hsoff, x / 4, x % 4);
      }
    };
    // pair e holds registers 2e, 2e+1: queries 32hs + 16(e/4) + 8*half +
    // 2(e%4) and the next one; lse of the pairs two ahead of the
    // exponentials, D two ahead of the dS pairs
    float2 lq[3], dq2[3];
    auto q_of = [&](int e) { return 32 * hs + 16 * (e / 4) + 8 * half + 2 * (e % 4); };
    auto read_l = [&](int e) {
      lq[e % 3] = *reinterpret_cast<const float2*>(&lse_sh[set][q_of(e)]);
    };
    auto read_d = [&](int e) {
      dq2[e % 3] = *reinterpret_cast<const float2*>(&d_sh[set][q_of(e)]);
    };
#pragma unroll
    for (int i = 0; i < 2; ++i) read_op(i);
    slot_fence();
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if (i + 2 < 32) read_op(i + 2);
      if (i >= 7 && i < 15) opv[(i + 1) % 2] = as_ev8(vrows[vread + 2 * (i + 1 - 8)]);
      if (i == 6) read_l(0);
      if (i == 7) read_l(1);
      if (i == 14) read_d(0);
      if (i == 15) read_d(1);
      if (i < 8) {
        s = mfma_32x32x16<F16>(opa[i % 3], kf[i], s);
      } else if (i < 16) {
        dp = mfma_32x32x16<F16>(opa[i % 3], opv[i % 2], dp);
      } else if (i < 24) {
        const int x = i - 16, cc = x / 4, dt = x % 4;
        const ev8 b = __builtin_bit_cast(ev8, make_uint4(pw[cc][0], pw[cc][1], pw[cc][2],
                                                         pw[cc][3]));
        accv[dt] = mfma_32x32x16<F16>(opa[i % 3], b, accv[dt]);
      } else {
        const int x = i - 24, cc = x / 4, dt = x % 4;
        const ev8 b = __builtin_bit_cast(ev8, make_uint4(dsw[cc][0], dsw[cc][1], dsw[cc][2],
                                                         dsw[cc][3]));
        acck[dt] = mfma_32x32x16<F16>(opa[i % 3], b, acck[dt]);
      }
      if (i >= 10 && i < 18) {  // exponential pair e: P, kept in fp32 in s
        const int e = i - 10, jj = 2 * e;
        const float2 l = lq[e % 3];
        if (e + 2 < 8) read_l(e + 2);
        s[jj] = __builtin_amdgcn_exp2f(fmaf(s[jj], scale_log2, -l.x));
        s[jj + 1] = __builtin_amdgcn_exp2f(fmaf(s[jj + 1], scale_log2, -l.y));
        pw[e / 4][e % 4] = pack2<F16>(s[jj], s[jj + 1]);
        pin_v(pw[e / 4][e % 4]);
      }
      if (i >= 18 && i < 26) {  // dS pair e
        const int e = i - 18, jj = 2 * e;
        const float2 dd = dq2[e % 3];
        if (e + 2 < 8) read_d(e + 2);
        dsw[e / 4][e % 4] = pack2<F16>(s[jj] * (dp[jj] - dd.x), s[jj + 1] * (dp[jj + 1] - dd.y));
        pin_v(dsw[e / 4][e % 4]);
      }
      slot_fence();
    }
  };
  auto work = [&](const uint4* qsb, const uint4* dsb, int set) {
    if (!active) return;
    for (int hs = hs_lo; hs <= hs_hi; ++hs) half_tile(hs, qsb, dsb, set);
  };

  // the column's query blocks (a half of a split column: the first or the
  // second half of them)
  int e_lo = 0, e_hi = tcount[c];
  if (part >= 0) {
    const int mid = e_hi / 2;
    if (part & 1) e_lo = mid;
    else e_hi = mid;
  }
  const int32_t* list = tlist + c * int64_t(g.nb);
  for (int e0 = e_lo; e0 < e_hi; e0 += kEntries) {
    const int m = min(kEntries, e_hi - e0);
    for (int x = tid; x < m; x += kThreads)
      esc[x] = (block_count(g, list[e0 + x] & 0xffff) + kKvChunk - 1) / kKvChunk;
    __syncthreads();
    scan_counts(esc, m, &ntl, wave, lane);
    __syncthreads();
    for (int x = tid; x < m; x += kThreads) {
      const int32_t ent = list[e0 + x];
      const int qi = ent & 0xffff;
      const int cq = block_count(g, qi);
      for (int sub = 0; sub * kKvChunk < cq; ++sub) {
        tl[esc[x] + sub] = ((qi * cpb + sub) << 7) | (min(kKvChunk, cq - sub * kKvChunk) - 1);
        tm[esc[x] + sub] = uint16_t(uint32_t(ent) >> 16);
      }
    }
    __syncthreads();
    const int T = __builtin_amdgcn_readfirstlane(ntl);
    if (T == 0) continue;
    {
      const int d0 = __builtin_amdgcn_readfirstlane(tl[0]);
      issue(d0, qs0, ds0);
      const Raw r0 = raw_of(d0);
      wait_copies();  // also the V rows of the first pass
      put(r0, d0, 0, float(tm[0]));
    }
    __syncthreads();
    for (int n = 0; n < T; n += 2) {
      const int d1 = __builtin_amdgcn_readfirstlane(tl[min(n + 1, T - 1)]);
      const float m1 = float(tm[min(n + 1, T - 1)]);
      Raw r1 = {0.f, 0.f};
      if (n + 1 < T) {
        issue(d1, qs1, ds1);
        r1 = raw_of(d1);
      }
      work(qs0, ds0, 0);
      wait_copies();
      if (n + 1 < T) put(r1, d1, 1, m1);
      __syncthreads();
      if (n + 1 >= T) break;
      const int d2 = __builtin_amdgcn_readfirstlane(tl[min(n + 2, T - 1)]);
      const float m2 = float(tm[min(n + 2, T - 1)]);
      Raw r2 = {0.f, 0.f};
      if (n + 2 < T) {
        issue(d2, qs0, ds0);
        r2 = raw_of(d2);
      }
      work(qs1, ds1, 1);
      wait_copies();
      if (n + 2 < T) put(r2, d2, 0, m2);
      __syncthreads();
    }
  }
  wait_copies();  // the V rows, when no pass ran
  __syncthreads();
  // query-half pairs: the second wave's partial dV^T and dK^T (wave 6's in
  // qs0/qs1, wave 7's in ds0/ds1, free after the last barrier) are added to
  // the first's
  const bool own_pad = split && qhalf == 1;  // waves 6, 7: their own rows are padding
  if (split) {
    float* const pv = reinterpret_cast<float*>((wave & 1) == 0 ? qs0 : ds0);
    float* const pk = reinterpret_cast<float*>((wave & 1) == 0 ? qs1 : ds1);
    if (own_pad && active) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          pv[(dt * 16 + jj) * 64 + lane] = accv[dt][jj];
          pk[(dt * 16 + jj) * 64 + lane] = acck[dt][jj];
        }
    }
    __syncthreads();
    if (qhalf == 0 && active) {
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int jj = 0; jj < 16; ++jj) {
          accv[dt][jj] += pv[(dt * 16 + jj) * 64 + lane];
          acck[dt][jj] += pk[(dt * 16 + jj) * 64 + lane];
        }
    }
  }
  if (SPLIT && part >= 0 && !bwd_tail_merge<NW, true>(split_flags, split_ids, split_part, part, wave,
                                               lane, active && !own_pad, accv, acck, c, &done_sh))
    return;
  // rows of this wave's own keys; pad key rows (and waves 6, 7) write zeros
  const bool keep = key < cj && !own_pad;
  store_rows_perm<F16>(accv, keep ? 1.f : 0.f, dv + (key0 + wave * 32) * 16, l32, half);
  store_rows_perm<F16>(acck, keep ? scale : 0.f, dk + (key0 + wave * 32) * 16, l32, half);
}

template <int NW, bool F16>
hipError_t launch_bwd_nw(const VsaGeom& g, const BwdArgs& a, hipStream_t s) {
  const int64_t rows = int64_t(g.batch) * g.heads * g.nb;
  const float scale = 1.0f / sqrtf(float(g.head_dim));
  const float scale_log2 = scale * kLog2e;
  // Balanced launches (claim_row): a quarter more workgroups than rows or
  // columns (plus one per split row), the queue and split counters cleared
  // before each kernel (they run one after another on `s`, so one counter
  // block and one split region serve both).  The tail split applies when no
  // queue holds more than kSplitMaxQueueRows rows.
  const int split =
      a.split_flags != nullptr && (rows + 7) / 8 <= kSplitMaxQueueRows ? kSplitPerQueue : 0;
  const int nflags = int(split_slots(rows, split));
  const int64_t items = rows + nflags;
  const unsigned grid = unsigned(items + std::max<int64_t>(8, items / 4));
  auto reset = [&] {
    hipLaunchKernelGGL(bwd_queue_reset_kernel, dim3(1), dim3(256), 0, s, a.queues, a.split_flags,
                       nflags);
    return hipGetLastError();
  };
  hipError_t e = reset();
  if (e != hipSuccess) return e;
  // launches that split no rows run instantiations without the merge code
  auto run = [&](auto split_t) {
    constexpr bool SPLIT = decltype(split_t)::value;
    hipLaunchKernelGGL((dq_kernel<NW, F16, SPLIT>), dim3(grid), dim3(NW * 64), 0, s,
                       static_cast<const uint4*>(a.q), static_cast<const uint4*>(a.k),
                       static_cast<const uint4*>(a.v), static_cast<const uint4*>(a.dout), a.lse,
                       a.dsum, a.row_ptr, a.col, a.uniform_k, a.nnz, static_cast<uint4*>(a.dq),
                       a.queues, g, scale_log2, scale, a.split_flags, a.split_rows,
                       a.split_part, split);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || (err = reset()) != hipSuccess) return err;
    hipLaunchKernelGGL((dkv_kernel<NW, F16, SPLIT>), dim3(grid), dim3(NW * 64), 0, s,
                       static_cast<const uint4*>(a.q), static_cast<const uint4*>(a.k),
                       static_cast<const uint4*>(a.v), static_cast<const uint4*>(a.dout), a.lse,
                       a.dsum, a.tlist, a.tcount, static_cast<uint4*>(a.dk),
                       static_cast<uint4*>(a.dv), a.queues, g, scale_log2, scale,
                       a.split_flags, a.split_rows, a.split_part, split);
    return hipGetLastError();
  };
  return split > 0 ? run(std::true_type()) : run(std::false_type());
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
