// Block-sparse flash-attention forward for the VSA hot path on gfx950 (CDNA4).
//
// "FastVideo VSA" user guide, intro: exact attention runs only against the
// selected key/value blocks of each query block; "Verify routing and
// fallback": non-causal, equal Q/KV lengths, scale head_size**-0.5, equal
// head counts, no mask.  FastVideo h3-perf-stack commit log, sm_100a tile-64
// route entry: rows of a compacted block map may hold different numbers of
// blocks, including none.
//
// Work decomposition
//   One workgroup per CSR row r = (b*NH + h)*nb + i, i.e. one query block of
//   V = 32*NW tokens; wave w owns query rows 32w .. 32w+31.  Row ids are
//   remapped so that each of the 8 XCDs (workgroups are dispatched to XCDs
//   round-robin) works through a contiguous range of rows, i.e. the same
//   heads, and its L2 serves their shared key/value blocks.
//   The row's key blocks are streamed in 64-key sub-tiles (a block with c
//   valid tokens has ceil(c/64) of them; trailing all-pad sub-tiles are never
//   loaded).  K (64 x 128) and V^T (128 x 64) sub-tiles are copied HBM/L2 ->
//   LDS directly (global_load_lds_dwordx4, no VGPR staging), double-buffered,
//   one barrier per sub-tile.  K runs one sub-tile ahead of V so that the
//   next sub-tile's QK^T can run on the matrix cores while this sub-tile's
//   softmax runs on the VALU (software pipeline inside each wave).
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16, D[m][n] += A[m][k] B[k][n];
// lane l holds A row m = l%32, B column n = l%32, and accumulator register
// j holds row m = 8*(j/4) + 4*(l/32) + j%4 of column n = l%32):
//   S^T = K Q^T :  A = K sub-tile rows (keys) from LDS, B = Q^T fragments
//                  kept in VGPRs for the whole row.  Each lane then holds 32
//                  scores of ONE query (column n), so the softmax max and sum
//                  are in-lane plus one exchange between lanes l and l^32.
//   O^T += V^T P^T: A = V^T rows (d) from LDS, B = P^T taken straight from the
//                  S^T accumulators after exp2 and bf16 rounding.
//   For the second product the 8 keys a lane feeds at k-slot (l/32, t) must be
//   the 8 keys its S^T accumulator holds.  Staging K row `key` into LDS row
//   kappa(key) (kappa swaps bits 2 and 3 of the row index) makes accumulator
//   register j of a 32-key S^T tile hold key 16*(j/8) + 8*(l/32) + j%8, so
//   the keys of PV step c are the contiguous run 16c + 8*(l/32) + 0..7 and the
//   matching V^T operand is one 16-byte LDS read.
//
// Online softmax (exact up to rounding): running reference max m and sum l per
// query in fp32, p = exp2(s*log2(e)/sqrt(D) - m*log2(e)/sqrt(D)) on the
// transcendental unit, l summed from the fp32 p, P rounded to bf16 for the PV
// product, O rescaled by exp2 of the max change only when the max grows by
// more than 2^8 (so p <= 256).  Padded keys of a partial sub-tile are masked
// to -inf.  A row without blocks leaves l = 0 and writes O = 0, LSE = -inf.

#include "vsa_internal.h"

namespace vsa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kUnits = 1024;  // 16-byte units in one 64 x 128 bf16 sub-tile (16 KB)

__device__ inline bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Dispatch is round-robin over the 8 XCDs; give each XCD a contiguous run of rows.
__device__ inline int64_t xcd_remap(int64_t wg, int64_t n) {
  const int64_t per = n / 8, rem = n % 8;
  const int64_t x = wg % 8, loc = wg / 8;
  return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + loc;
}

// LDS row holding key `key` of a K sub-tile: swap bits 2 and 3.
__device__ inline int kappa(int key) {
  return (key & ~0xc) | ((key & 4) << 1) | ((key & 8) >> 1);
}

// LDS tiles use padded rows so that every MFMA operand read is one base
// register plus an immediate offset and the 16-byte reads of 8 (or 16)
// consecutive lanes fall on distinct banks:
//   K   : 64 rows (keys, kappa-permuted) x (16 + 1) 16-byte units = 17 KB
//   V^T : 128 rows (d) x (8 + 1) units = 18 KB
// The pad unit of each row is filled with a copy of the row's first unit.
constexpr int kKRow = 17, kVRow = 9;
constexpr int kKUnits = 64 * kKRow;    // 1088
constexpr int kVUnits = 128 * kVRow;   // 1152
constexpr int kKChunks = kKUnits / 64;  // 17 wave-loads of 1 KB
constexpr int kVChunks = kVUnits / 64;  // 18
constexpr int kORow = 17;               // epilogue O staging row: 272 B

struct TileCursor {
  int e;    // CSR entry, relative to the row start
  int sub;  // 64-key sub-tile inside the block
  int j;    // key block id
  int cj;   // its valid-token count
};

// Move to the first sub-tile of the next valid CSR entry after `c.e`.
__device__ inline bool next_entry(TileCursor& c, int len, const int32_t* __restrict__ col,
                                  const VsaGeom& g) {
  for (++c.e; c.e < len; ++c.e) {
    const int j = col[c.e];
    if (j >= 0 && j < g.nb) {
      c.j = j;
      c.sub = 0;
      c.cj = block_count(g, j);
      return true;
    }
  }
  return false;
}

__device__ inline bool next_tile(TileCursor& c, int len, const int32_t* __restrict__ col,
                                 const VsaGeom& g) {
  if ((c.sub + 1) * kKvChunk < c.cj) {
    ++c.sub;
    return true;
  }
  return next_entry(c, len, col, g);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// One wave copies 64 x 16 bytes from global memory straight into LDS: lane l
// reads `src + off` and its 16 bytes land at `dst + 16*l`.
__device__ inline void wave_copy_to_lds(const uint4* src, uint32_t off, uint4* dst) {
  __builtin_amdgcn_global_load_lds(static_cast<const void*>(src + off),
                                   (lds_ptr_t)(dst), 16, 0, 0);
}

// S^T (2 tiles of 32 keys x 32 queries) = K sub-tile (LDS) x Q^T (VGPRs).
__device__ inline void qk_tile(const uint4* __restrict__ kl, const bf16x8 (&qf)[8],
                               f32x16 (&st)[2]) {
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int j = 0; j < 16; ++j) st[mt][j] = 0.f;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const bf16x8 a = as_bf16x8(kl[mt * 32 * kKRow + 2 * s]);
      st[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], st[mt], 0, 0, 0);
    }
  }
}

// p = exp2(s*c - mb) for the 32 scores of this lane: fp32 partial sums for l,
// bf16 values grouped as the B operands of the 4 PV steps (16 keys each).
__device__ inline void exp_tile(const f32x16 (&st)[2], float c, float mb, bf16x8 (&pb)[4],
                                float& rs0, float& rs1) {
#pragma unroll
  for (int cc = 0; cc < 4; ++cc)
#pragma unroll
    for (int t = 0; t < 8; t += 2) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(st[cc / 2][8 * (cc % 2) + t], c, -mb));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(st[cc / 2][8 * (cc % 2) + t + 1], c, -mb));
      rs0 += p0;
      rs1 += p1;
      pb[cc][t] = __bf16(p0);
      pb[cc][t + 1] = __bf16(p1);
    }
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(
    const uint4* __restrict__ q, const uint4* __restrict__ k, const uint4* __restrict__ vt,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col, int uniform_k,
    int64_t nnz, uint4* __restrict__ o, float* __restrict__ lse, VsaGeom g, float scale_log2,
    float scale) {
  static_assert(2 * (kKUnits + kVUnits) >= NW * 32 * kORow, "O staging must fit in LDS");
  const float rescale_thr = 8.0f / scale_log2;  // raw-score growth that triggers a rescale
  // K runs one sub-tile ahead of V: while sub-tile n is finished, K buffer
  // n^1 holds K_{n+1} (read) and buffer n receives K_{n+2}; V buffer n holds
  // V_n (read) and buffer n^1 receives V_{n+1}.
  __shared__ __align__(16) uint4 smem[2 * kKUnits + 2 * kVUnits];
  uint4* const kbuf0 = smem;
  uint4* const vbuf0 = smem + 2 * kKUnits;

  const int64_t nrows = int64_t(g.batch) * g.heads * g.nb;
  const int64_t r = xcd_remap(blockIdx.x, nrows);
  const int i = int(r % g.nb);
  const int64_t bh = r / g.nb;
  const int cq = block_count(g, i);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / 64);  // uniform: lives in an SGPR
  const int lane = tid % 64;
  const int half = lane / 32;
  const int l32 = lane & 31;
  const int qrow = wave * 32 + l32;      // this lane's query row inside the block
  const bool active = wave * 32 < cq;    // wave-uniform

  int64_t beg, end;
  if (row_ptr != nullptr) {
    beg = min(max(int64_t(row_ptr[r]), int64_t(0)), nnz);
    end = min(max(int64_t(row_ptr[r + 1]), beg), nnz);
  } else {
    beg = r * uniform_k;
    end = beg + uniform_k;
  }
  const int32_t* rcol = col + beg;
  const int len = int(end - beg);

  const int64_t qk_row0 = bh * g.npad + int64_t(i) * g.vol;  // first token row of block i
  bf16x8 qf[8];
  if (active) {
    const uint4* qsrc = q + (qk_row0 + qrow) * 16;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = as_bf16x8(qsrc[2 * s + half]);
  }

  f32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int j = 0; j < 16; ++j) oacc[dt][j] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  const uint4* const kbase = k + bh * g.npad * 16;
  const uint4* const vbase = vt + bh * (g.npad / kKvChunk) * kUnits;
  const int chunks_per_block = g.vol / kKvChunk;
  // per-lane source offsets (16-byte units inside a sub-tile) of this wave's
  // chunk loads; the same for every sub-tile
  constexpr int kMaxK = (kKChunks + NW - 1) / NW, kMaxV = (kVChunks + NW - 1) / NW;
  uint32_t koff[kMaxK], voff[kMaxV];
#pragma unroll
  for (int u = 0; u < kMaxK; ++u) {
    const int pos = (wave + u * NW) * 64 + lane;
    const int row = pos / kKRow, unit = pos % kKRow;
    koff[u] = kappa(row) * 16 + (unit < 16 ? unit : 0);
  }
#pragma unroll
  for (int u = 0; u < kMaxV; ++u) {
    const int pos = (wave + u * NW) * 64 + lane;
    const int row = pos / kVRow, unit = pos % kVRow;
    voff[u] = row * 8 + (unit < 8 ? unit : 0);
  }
  auto load_k = [&](const TileCursor& c, int b) {
    const uint4* src = kbase + (int64_t(c.j) * g.vol + c.sub * kKvChunk) * 16;
#pragma unroll
    for (int u = 0; u < kMaxK; ++u)
      if (wave + u * NW < kKChunks)
        wave_copy_to_lds(src, koff[u], kbuf0 + b * kKUnits + (wave + u * NW) * 64);
  };
  auto load_v = [&](const TileCursor& c, int b) {
    const uint4* src = vbase + (int64_t(c.j) * chunks_per_block + c.sub) * kUnits;
#pragma unroll
    for (int u = 0; u < kMaxV; ++u)
      if (wave + u * NW < kVChunks)
        wave_copy_to_lds(src, voff[u], vbuf0 + b * kVUnits + (wave + u * NW) * 64);
  };
  auto wait_loads = [] { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

  // cursors of sub-tiles n, n+1, n+2
  TileCursor c0, c1, c2;
  c0.e = -1;
  bool h0 = next_entry(c0, len, rcol, g);
  c1 = c0;
  bool h1 = h0 && next_tile(c1, len, rcol, g);
  c2 = c1;
  bool h2 = h1 && next_tile(c2, len, rcol, g);
  if (h0) {
    load_k(c0, 0);
    load_v(c0, 0);
  }
  if (h1) load_k(c1, 1);
  wait_loads();
  __syncthreads();

  // per-lane operand bases: K row l32 (+ half unit), V^T row l32 (+ half unit)
  const int kread = l32 * kKRow + half;
  const int vread = l32 * kVRow + half;

  f32x16 sa[2], sb[2];
  if (h0 && active) qk_tile(kbuf0 + kread, qf, sa);

  // Finish sub-tile n (scores in `cur`) and compute the scores of n+1 into `nxt`.
  auto step = [&](f32x16 (&cur)[2], f32x16 (&nxt)[2], const int n) {
    if (h2) load_k(c2, n);      // K_{n+2} replaces K_n
    if (h1) load_v(c1, n ^ 1);  // V_{n+1} replaces V_{n-1}
    if (active) {
      // mask keys past the block's valid count (only in its last sub-tile)
      const int valid = c0.cj - c0.sub * kKvChunk;
      if (valid < kKvChunk) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = mt * 32 + 16 * (j / 8) + 8 * half + (j % 8);
            if (key >= valid) cur[mt][j] = -INFINITY;
          }
      }
      // row max over this lane's 32 keys and the partner lane's (l ^ 32)
      float mx = cur[0][0];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, cur[mt][j]);
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                         false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      // Lazy rescale: the reference max m_run only moves (and O, l are only
      // rescaled) when a score exceeds it by more than 8 in log2 units, so
      // every p = exp2((s - m_run) * scale * log2 e) stays <= 2^8.  The final
      // O / l is the same softmax whichever reference max was used.
      if (__ballot(mx > m_run + rescale_thr) != 0) {  // wave-uniform branch
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
        m_run = m_new;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int j = 0; j < 16; ++j) oacc[dt][j] *= alpha;
      }
      const float mb = m_run * scale_log2;
      bf16x8 pb[4];
      float rs0 = 0.f, rs1 = 0.f;
      if (h1) {
        // next sub-tile's QK^T on the matrix cores, interleaved with this
        // sub-tile's exponentials on the VALU
        qk_tile(kbuf0 + (n ^ 1) * kKUnits + kread, qf, nxt);
        exp_tile(cur, scale_log2, mb, pb, rs0, rs1);
        // K operand reads run 4 ahead of the MFMAs that consume them; every
        // MFMA is followed by 7 VALU instructions of the softmax
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (u < 12) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);
        }
      } else {
        exp_tile(cur, scale_log2, mb, pb, rs0, rs1);
      }
      l_run += rs0 + rs1;
      // O^T += V^T P^T, 4 steps of 16 keys
      const uint4* vl = vbuf0 + n * kVUnits + vread;
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const bf16x8 a = as_bf16x8(vl[dt * 32 * kVRow + 2 * cc]);
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[cc], oacc[dt], 0, 0, 0);
        }
      }
      // V operand reads run 2 ahead of the MFMAs that consume them
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        if (u < 14) __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
      }
    }
    wait_loads();
    __syncthreads();
    TileCursor c3 = c2;
    const bool h3 = h2 && next_tile(c3, len, rcol, g);
    c0 = c1;
    h0 = h1;
    c1 = c2;
    h1 = h2;
    c2 = c3;
    h2 = h3;
  };

  while (h0) {
    step(sa, sb, 0);
    if (!h0) break;
    step(sb, sa, 1);
  }

  // ---- epilogue: combine the two lane halves' partial sums, normalise, and
  // store O through LDS so that every global store is a full 256-byte row.
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run),
                                                     __float_as_uint(l_run), false, false);
    l_run = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  const bool row_valid = active && qrow < cq;
  const float inv = (row_valid && l_run > 0.f) ? 1.f / l_run : 0.f;
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  uint2* const ostage = reinterpret_cast<uint2*>(smem + wave * 32 * kORow);  // 32 rows x 272 B
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      // registers 4jj..4jj+3 hold d = 32dt + 8jj + 4*half + 0..3
      bf16x4 w;
#pragma unroll
      for (int t = 0; t < 4; ++t) w[t] = __bf16(oacc[dt][4 * jj + t] * inv);
      ostage[l32 * (kORow * 2) + (dt * 32 + 8 * jj + 4 * half) / 4] = __builtin_bit_cast(uint2, w);
    }
  // the staging area of wave w is only touched by wave w
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  const uint4* const orows = smem + wave * 32 * kORow;
  uint4* const odst = o + (qk_row0 + wave * 32) * 16;
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int rr = p * 4 + lane / 16;
    odst[rr * 16 + (lane & 15)] = orows[rr * kORow + (lane & 15)];
  }
  if (lse != nullptr && half == 0) {
    lse[qk_row0 + qrow] =
        (row_valid && l_run > 0.f) ? m_run * scale + __logf(l_run) : -INFINITY;
  }
}

template <int NW>
hipError_t launch_nw(const VsaGeom& g, const void* q, const void* k, const void* vt,
                     const int32_t* row_ptr, const int32_t* col, int uniform_k, int64_t nnz,
                     void* o, float* lse, hipStream_t s) {
  const int64_t rows = int64_t(g.batch) * g.heads * g.nb;
  const float scale = 1.0f / sqrtf(float(g.head_dim));
  const float scale_log2 = scale * 1.4426950408889634f;
  hipLaunchKernelGGL(attn_fwd_kernel<NW>, dim3(unsigned(rows)), dim3(NW * 64), 0, s,
                     static_cast<const uint4*>(q), static_cast<const uint4*>(k),
                     static_cast<const uint4*>(vt), row_ptr, col, uniform_k, nnz,
                     static_cast<uint4*>(o), lse, g, scale_log2, scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_fwd(const VsaGeom& g, const void* q, const void* k, const void* vt,
                           const int32_t* row_ptr, const int32_t* col, int uniform_k,
                           int64_t nnz, void* o, float* lse, hipStream_t s) {
  switch (g.vol / 32) {
    case 2: return launch_nw<2>(g, q, k, vt, row_ptr, col, uniform_k, nnz, o, lse, s);
    case 4: return launch_nw<4>(g, q, k, vt, row_ptr, col, uniform_k, nnz, o, lse, s);
    case 6: return launch_nw<6>(g, q, k, vt, row_ptr, col, uniform_k, nnz, o, lse, s);
    case 8: return launch_nw<8>(g, q, k, vt, row_ptr, col, uniform_k, nnz, o, lse, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vsa
