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
//   loaded).  K (64 x 128) and V^T (128 x 64) sub-tiles go HBM/L2 -> VGPR ->
//   LDS, double-buffered, one barrier per sub-tile; the next sub-tile's global
//   loads are in flight while the current one is computed.
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
// Online softmax (exact up to rounding): running max m and sum l per query in
// fp32, p = exp2(s*log2(e)/sqrt(D) - m*log2(e)/sqrt(D)) on the transcendental
// unit, P rounded to bf16 for the PV product, O rescaled by exp2 of the max
// change.  Padded keys of a partial sub-tile are masked to -inf.  A row
// without blocks leaves l = 0 and writes O = 0, LSE = -inf.

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
// 16-byte-unit swizzles that keep the MFMA operand reads conflict-free.
__device__ inline int k_pos(int row, int unit) { return row * 16 + (unit ^ (row & 15)); }
__device__ inline int v_pos(int d, int unit) { return d * 8 + (unit ^ ((d ^ (d >> 3)) & 7)); }

struct TileCursor {
  int64_t e;   // CSR entry
  int sub;     // 64-key sub-tile inside the block
  int j;       // key block id
  int cj;      // its valid-token count
};

// Move to the first sub-tile of the next valid CSR entry after `c.e`.
__device__ inline bool next_entry(TileCursor& c, int64_t end, const int32_t* __restrict__ col,
                                  const VsaGeom& g) {
  for (++c.e; c.e < end; ++c.e) {
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

__device__ inline bool next_tile(TileCursor& c, int64_t end, const int32_t* __restrict__ col,
                                 const VsaGeom& g) {
  if ((c.sub + 1) * kKvChunk < c.cj) {
    ++c.sub;
    return true;
  }
  return next_entry(c, end, col, g);
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(
    const uint4* __restrict__ q, const uint4* __restrict__ k, const uint4* __restrict__ vt,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col, int uniform_k,
    int64_t nnz, uint2* __restrict__ o, float* __restrict__ lse, VsaGeom g, float scale_log2,
    float scale) {
  constexpr int kThreads = NW * 64;
  constexpr int kPer = (kUnits + kThreads - 1) / kThreads;  // 16-byte units per thread
  constexpr bool kEven = kUnits % kThreads == 0;
  __shared__ __align__(16) uint4 lds[2][2][kUnits];  // [stage][K | V^T][unit]

  const int64_t nrows = int64_t(g.batch) * g.heads * g.nb;
  const int64_t r = xcd_remap(blockIdx.x, nrows);
  const int i = int(r % g.nb);
  const int64_t bh = r / g.nb;
  const int cq = block_count(g, i);
  const int tid = threadIdx.x;
  const int wave = tid / 64;
  const int lane = tid % 64;
  const int half = lane / 32;
  const int qrow = wave * 32 + (lane & 31);  // this lane's query row inside the block
  const bool active = wave * 32 < cq;        // wave-uniform

  int64_t beg, end;
  if (row_ptr != nullptr) {
    beg = min(max(int64_t(row_ptr[r]), int64_t(0)), nnz);
    end = min(max(int64_t(row_ptr[r + 1]), beg), nnz);
  } else {
    beg = r * uniform_k;
    end = beg + uniform_k;
  }

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

  const int64_t kv_chunks_per_head = g.npad / kKvChunk;
  const int chunks_per_block = g.vol / kKvChunk;
  uint4 pk[kPer], pv[kPer];

  auto load_tile = [&](const TileCursor& c) {
    const uint4* ks = k + (bh * g.npad + int64_t(c.j) * g.vol + int64_t(c.sub) * kKvChunk) * 16;
    const uint4* vs =
        vt + (bh * kv_chunks_per_head + int64_t(c.j) * chunks_per_block + c.sub) * kUnits;
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      if (kEven || tid + p * kThreads < kUnits) {
        pk[p] = ks[tid + p * kThreads];
        pv[p] = vs[tid + p * kThreads];
      }
    }
  };
  auto store_tile = [&](int stage) {
#pragma unroll
    for (int p = 0; p < kPer; ++p) {
      const int idx = tid + p * kThreads;
      if (kEven || idx < kUnits) {
        lds[stage][0][k_pos(kappa(idx / 16), idx % 16)] = pk[p];
        lds[stage][1][v_pos(idx / 8, idx % 8)] = pv[p];
      }
    }
  };

  TileCursor cur;
  cur.e = beg - 1;
  bool have = next_entry(cur, end, col, g);
  if (have) {
    load_tile(cur);
    store_tile(0);
  }
  __syncthreads();
  int stage = 0;

  while (have) {
    TileCursor nxt = cur;
    const bool have_next = next_tile(nxt, end, col, g);
    if (have_next) load_tile(nxt);

    if (active) {
      const uint4* kl = lds[stage][0];
      const uint4* vl = lds[stage][1];
      // ---- S^T = K Q^T for the 64 keys of this sub-tile (2 tiles of 32 keys)
      f32x16 st[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j) st[mt][j] = 0.f;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const int row = mt * 32 + (lane & 31);
          const bf16x8 a = as_bf16x8(kl[k_pos(row, 2 * s + half)]);
          st[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], st[mt], 0, 0, 0);
        }
      }
      // ---- mask keys past the block's valid count (only in its last sub-tile)
      const int valid = cur.cj - cur.sub * kKvChunk;
      if (valid < kKvChunk) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = mt * 32 + 16 * (j / 8) + 8 * half + (j % 8);
            if (key >= valid) st[mt][j] = -INFINITY;
          }
      }
      // ---- online softmax: row max over this lane's 32 keys and the partner lane's
      float mx = st[0][0];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = fmaxf(mx, st[mt][j]);
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                         false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * scale_log2);
      m_run = m_new;
      const float mb = m_new * scale_log2;
      float rs = 0.f;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float p = __builtin_amdgcn_exp2f(fmaf(st[mt][j], scale_log2, -mb));
          st[mt][j] = p;
          rs += p;
        }
      l_run = l_run * alpha + rs;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) oacc[dt][j] *= alpha;
      // ---- O^T += V^T P^T, 4 steps of 16 keys
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        bf16x8 pb;
#pragma unroll
        for (int t = 0; t < 8; ++t) pb[t] = __bf16(st[c / 2][8 * (c % 2) + t]);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const int d = dt * 32 + (lane & 31);
          const bf16x8 a = as_bf16x8(vl[v_pos(d, 2 * c + half)]);
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[dt], 0, 0, 0);
        }
      }
    }

    if (have_next) store_tile(stage ^ 1);
    __syncthreads();
    stage ^= 1;
    cur = nxt;
    have = have_next;
  }

  // ---- epilogue: combine the two lane halves' partial sums, normalise, store
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run),
                                                     __float_as_uint(l_run), false, false);
    l_run = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  const bool row_valid = active && qrow < cq;
  const float inv = (row_valid && l_run > 0.f) ? 1.f / l_run : 0.f;
  uint2* orow = o + (qk_row0 + qrow) * (kHeadDim / 4);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      // registers 4jj..4jj+3 hold d = 32dt + 8jj + 4*half + 0..3
      typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
      bf16x4 w;
#pragma unroll
      for (int t = 0; t < 4; ++t) w[t] = __bf16(oacc[dt][4 * jj + t] * inv);
      orow[(dt * 32 + 8 * jj + 4 * half) / 4] = __builtin_bit_cast(uint2, w);
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
                     static_cast<uint2*>(o), lse, g, scale_log2, scale);
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
