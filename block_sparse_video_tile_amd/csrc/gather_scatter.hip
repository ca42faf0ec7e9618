// Raster <-> block-major data movement for the VSA hot path on gfx950.
//
// "FastVideo VSA" user guide, intro: the post-patch latent grid is cut into
// spatiotemporal blocks; "Choose top-k" notes the padding overhead this
// introduces for shapes that do not divide evenly.  Edge blocks are padded
// to the block volume with zero rows that the attention kernel masks.
//
// All three kernels are HBM-bound streams: one workgroup per (batch, head,
// block), 16-byte loads and stores, one token row of one head (D = 128
// 16-bit elements, bf16 or fp16: the guide's "Verify routing and fallback"
// admits both) is 16 lanes x 16 bytes.

#include "attn_common.h"
#include "vsa_internal.h"

namespace vsa {
namespace {

constexpr int kThreads = 256;
constexpr int kUnitsPerRow = kHeadDim * 2 / 16;  // 16-byte units per token row

struct BlockBox {
  int t0, h0, w0, ct, ch, cw, cnt;
};

__device__ inline BlockBox block_box(const VsaGeom& g, int beta) {
  const int plane = g.nbh * g.nbw;
  const int it = beta / plane;
  const int rem = beta - it * plane;
  const int ih = rem / g.nbw;
  const int iw = rem - ih * g.nbw;
  BlockBox b;
  b.t0 = it * g.bt;
  b.h0 = ih * g.bh;
  b.w0 = iw * g.bw;
  b.ct = min(g.bt, g.T - b.t0);
  b.ch = min(g.bh, g.H - b.h0);
  b.cw = min(g.bw, g.W - b.w0);
  b.cnt = b.ct * b.ch * b.cw;
  return b;
}

// Raster token index of the r-th valid token of a block (raster order inside the box).
__device__ inline int64_t token_of(const VsaGeom& g, const BlockBox& b, int r) {
  const int dw = r % b.cw;
  const int q = r / b.cw;
  const int dh = q % b.ch;
  const int dt = q / b.ch;
  return (int64_t(b.t0 + dt) * g.H + (b.h0 + dh)) * g.W + (b.w0 + dw);
}

// The two 16-bit elements of a 32-bit word as fp32 (low half first): bf16 is
// the upper half of an fp32, fp16 converts exactly.
template <bool F16>
__device__ inline float elem_lo(uint32_t w) {
  if constexpr (F16) return float(__builtin_bit_cast(_Float16, uint16_t(w & 0xffffu)));
  else return __uint_as_float(w << 16);
}
template <bool F16>
__device__ inline float elem_hi(uint32_t w) {
  if constexpr (F16) return float(__builtin_bit_cast(_Float16, uint16_t(w >> 16)));
  else return __uint_as_float(w & 0xffff0000u);
}

// Q/K: raster [B,S,NH,D] -> blocked [B,NH,Npad,D], optional fp32 block means
// (or the means alone, for any of Q, K, V, when xb is null).
// The copy moves raw 16-bit elements; only the means depend on the type.
template <bool F16>
__global__ __launch_bounds__(kThreads) void gather_qk_kernel(const uint4* __restrict__ x,
                                                             uint4* __restrict__ xb,
                                                             float* __restrict__ pooled,
                                                             VsaGeom g) {
  __shared__ float red[kThreads / kUnitsPerRow][kHeadDim + 1];
  const int wg = blockIdx.x;
  // consecutive workgroups take the heads of one block: together they read
  // (or write) whole raster token rows, all heads contiguous
  const int nbh = g.batch * g.heads;
  const int beta = wg / nbh;
  const int bh = wg % nbh;  // b * heads + h
  const int h = bh % g.heads;
  const int b = bh / g.heads;
  const BlockBox box = block_box(g, beta);
  const int unit = threadIdx.x % kUnitsPerRow;
  const int lt = threadIdx.x / kUnitsPerRow;  // token lane, 16 tokens per pass
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int64_t dst0 = (int64_t(bh) * g.npad + int64_t(beta) * g.vol) * kUnitsPerRow;
  // xb == nullptr: pooling only (reads the valid tokens, writes the means)
  const int rows = xb != nullptr ? g.vol : box.cnt;
  for (int r = lt; r < rows; r += kThreads / kUnitsPerRow) {
    uint4 val = make_uint4(0u, 0u, 0u, 0u);
    if (r < box.cnt) {
      const int64_t s = token_of(g, box, r);
      val = x[((int64_t(b) * g.S + s) * g.heads + h) * kUnitsPerRow + unit];
      acc[0] += elem_lo<F16>(val.x); acc[1] += elem_hi<F16>(val.x);
      acc[2] += elem_lo<F16>(val.y); acc[3] += elem_hi<F16>(val.y);
      acc[4] += elem_lo<F16>(val.z); acc[5] += elem_hi<F16>(val.z);
      acc[6] += elem_lo<F16>(val.w); acc[7] += elem_hi<F16>(val.w);
    }
    if (xb != nullptr) xb[dst0 + int64_t(r) * kUnitsPerRow + unit] = val;
  }
  if (pooled != nullptr) {
#pragma unroll
    for (int i = 0; i < 8; ++i) red[lt][unit * 8 + i] = acc[i];
    __syncthreads();
    if (threadIdx.x < kHeadDim) {
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < kThreads / kUnitsPerRow; ++k) s += red[k][threadIdx.x];
      pooled[(int64_t(bh) * g.nb + beta) * kHeadDim + threadIdx.x] = s / float(box.cnt);
    }
  }
}

// V: raster [B,S,NH,D] -> blocked-V^T [B,NH,Npad/64,D,64] (each 64-token
// chunk stored d-major), transposed through LDS; optionally the fp32 mean of
// each block's valid tokens (the gate-compress branch pools values per tile
// as well).  The means are summed in the order of gather_qk_kernel (each
// thread its tokens in ascending order, then the 16 token lanes in order), so
// both kernels give the same bits.
//
// The transpose reads LDS with the gfx950 transposing read ds_read_b64_tr_b16:
// in each group of 16 lanes, lane i receives element i%4 of the 8-byte pieces
// addressed by lanes 4e + i/4 (e = 0..3).  Lane L of a group addresses token
// row t0 + L/4, columns d0 + 4(L%4) .. +3, so lane i receives tokens
// t0 .. t0+3 of column d0 + i; two reads (t0 and t0 + 4) give the 8 tokens of
// one 16-byte V^T unit.  With 288-byte LDS rows the 16 pieces of a read fall
// on 16 distinct 8-byte bank slots.
typedef short v4i16 __attribute__((ext_vector_type(4)));

__device__ inline v4i16 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)(const_cast<void*>(p)));
}

template <bool F16>
__global__ __launch_bounds__(kThreads) void gather_v_kernel(const uint4* __restrict__ x,
                                                            uint4* __restrict__ xbt,
                                                            float* __restrict__ pooled,
                                                            VsaGeom g) {
  constexpr int kRow = kHeadDim + 16;  // 16-bit elements per LDS row (288 bytes)
  __shared__ __align__(16) uint16_t tile[kKvChunk][kRow];
  __shared__ float red[kThreads / kUnitsPerRow][kHeadDim + 1];
  const int wg = blockIdx.x;
  const int nbh = g.batch * g.heads;
  const int beta = wg / nbh;  // consecutive workgroups: the heads of one block
  const int bh = wg % nbh;
  const int h = bh % g.heads;
  const int b = bh / g.heads;
  const BlockBox box = block_box(g, beta);
  const int unit = threadIdx.x % kUnitsPerRow;
  const int lt = threadIdx.x / kUnitsPerRow;  // token lane: tokens lt, lt + 16, ...
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int grp = lane / 16, li = lane % 16;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int chunks = g.vol / kKvChunk;
  for (int c = 0; c < chunks; ++c) {
    // load the chunk's 64 token rows (pad rows zero)
#pragma unroll
    for (int p = 0; p < kKvChunk / (kThreads / kUnitsPerRow); ++p) {
      const int tok = lt + p * (kThreads / kUnitsPerRow);
      const int r = c * kKvChunk + tok;
      uint4 val = make_uint4(0u, 0u, 0u, 0u);
      if (r < box.cnt) {
        const int64_t s = token_of(g, box, r);
        val = x[((int64_t(b) * g.S + s) * g.heads + h) * kUnitsPerRow + unit];
        acc[0] += elem_lo<F16>(val.x); acc[1] += elem_hi<F16>(val.x);
        acc[2] += elem_lo<F16>(val.y); acc[3] += elem_hi<F16>(val.y);
        acc[4] += elem_lo<F16>(val.z); acc[5] += elem_hi<F16>(val.z);
        acc[6] += elem_lo<F16>(val.w); acc[7] += elem_hi<F16>(val.w);
      }
      *reinterpret_cast<uint4*>(&tile[tok][unit * 8]) = val;
    }
    __syncthreads();
    // write 128 d-rows x 8 units of 8 tokens: each 16-lane group writes 16
    // consecutive columns of one token octet per pass, a wave 16 columns x 4
    // octets (16 rows x 64 contiguous bytes)
    uint4* dst = xbt + ((int64_t(bh) * (g.npad / kKvChunk) + int64_t(beta) * chunks + c) *
                        kHeadDim) * (kKvChunk * 2 / 16);
    const char* lds = reinterpret_cast<const char*>(&tile[0][0]);
#pragma unroll
    for (int it = 0; it < kHeadDim * 8 / 16 / (kThreads / 16); ++it) {
      const int task = it * (kThreads / 16) + wave * 4 + grp;
      const int cg = task / 8, ku = task % 8;
      const int col = 16 * cg + 4 * (li % 4);
      const v4i16 lo = lds_read_tr16(lds + ((8 * ku + li / 4) * kRow + col) * 2);
      const v4i16 hi = lds_read_tr16(lds + ((8 * ku + 4 + li / 4) * kRow + col) * 2);
      const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
      dst[int64_t(16 * cg + li) * 8 + ku] = make_uint4(l2.x, l2.y, h2.x, h2.y);
    }
    __syncthreads();
  }
  if (pooled != nullptr) {
#pragma unroll
    for (int i = 0; i < 8; ++i) red[lt][unit * 8 + i] = acc[i];
    __syncthreads();
    if (threadIdx.x < kHeadDim) {
      float s = 0.f;
#pragma unroll
      for (int k = 0; k < kThreads / kUnitsPerRow; ++k) s += red[k][threadIdx.x];
      pooled[(int64_t(bh) * g.nb + beta) * kHeadDim + threadIdx.x] = s / float(box.cnt);
    }
  }
}

// Eight fp32 values rounded to nearest-even in the element type, packed.
template <bool F16>
__device__ inline uint4 pack8(const float (&f)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (F16) {
      typedef _Float16 h2 __attribute__((ext_vector_type(2)));
      const h2 r = {_Float16(f[2 * e]), _Float16(f[2 * e + 1])};
      w[e] = __builtin_bit_cast(uint32_t, r);
    } else {
      typedef __bf16 b2 __attribute__((ext_vector_type(2)));
      const b2 r = {__bf16(f[2 * e]), __bf16(f[2 * e + 1])};
      w[e] = __builtin_bit_cast(uint32_t, r);
    }
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// O: blocked [B,NH,Npad,D] -> raster [B,S,NH,D]; pad rows are not read.
// With `oc` (coarse output [B,NH,nb,D] fp32) and `gate` (raster, elem) the
// token row written is O + gate * oc[block], in fp32, rounded once to elem:
// the sparse output compensated by the gated coarse branch ("FastVideo VSA"
// guide, "Checkpoint behavior").
template <bool F16>
__global__ __launch_bounds__(kThreads) void scatter_kernel(const uint4* __restrict__ ob,
                                                           const float* __restrict__ oc,
                                                           const uint4* __restrict__ gate,
                                                           uint4* __restrict__ o, VsaGeom g) {
  const int wg = blockIdx.x;
  const int nbh = g.batch * g.heads;
  const int beta = wg / nbh;  // consecutive workgroups: the heads of one block
  const int bh = wg % nbh;
  const int h = bh % g.heads;
  const int b = bh / g.heads;
  const BlockBox box = block_box(g, beta);
  const int unit = threadIdx.x % kUnitsPerRow;
  const int lt = threadIdx.x / kUnitsPerRow;
  const uint4* src = ob + (int64_t(bh) * g.npad + int64_t(beta) * g.vol) * kUnitsPerRow;
  float c[8];
  if (gate != nullptr) {
    const float4* cp =
        reinterpret_cast<const float4*>(oc + (int64_t(bh) * g.nb + beta) * kHeadDim + unit * 8);
    const float4 c0 = cp[0], c1 = cp[1];
    c[0] = c0.x; c[1] = c0.y; c[2] = c0.z; c[3] = c0.w;
    c[4] = c1.x; c[5] = c1.y; c[6] = c1.z; c[7] = c1.w;
  }
  for (int r = lt; r < box.cnt; r += kThreads / kUnitsPerRow) {
    const int64_t s = token_of(g, box, r);
    const int64_t at = ((int64_t(b) * g.S + s) * g.heads + h) * kUnitsPerRow + unit;
    uint4 val = src[int64_t(r) * kUnitsPerRow + unit];
    if (gate != nullptr) {
      const uint4 gv = gate[at];
      const uint32_t ow[4] = {val.x, val.y, val.z, val.w};
      const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
      float f[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        f[2 * e] = fmaf(tile::elem_to_f32<F16>(gw[e] & 0xffffu), c[2 * e], tile::elem_to_f32<F16>(ow[e] & 0xffffu));
        f[2 * e + 1] = fmaf(tile::elem_to_f32<F16>(gw[e] >> 16), c[2 * e + 1], tile::elem_to_f32<F16>(ow[e] >> 16));
      }
      val = pack8<F16>(f);
    }
    o[at] = val;
  }
}

}  // namespace

hipError_t launch_gather_qk(const VsaGeom& g, const void* x, void* xb, float* pooled,
                            hipStream_t s) {
  const int64_t grid = int64_t(g.batch) * g.heads * g.nb;
  if (g.dtype == VSA_DTYPE_FP16)
    hipLaunchKernelGGL(gather_qk_kernel<true>, dim3(unsigned(grid)), dim3(kThreads), 0, s,
                       static_cast<const uint4*>(x), static_cast<uint4*>(xb), pooled, g);
  else
    hipLaunchKernelGGL(gather_qk_kernel<false>, dim3(unsigned(grid)), dim3(kThreads), 0, s,
                       static_cast<const uint4*>(x), static_cast<uint4*>(xb), pooled, g);
  return hipGetLastError();
}

hipError_t launch_gather_v(const VsaGeom& g, const void* x, void* xbt, float* pooled,
                           hipStream_t s) {
  const int64_t grid = int64_t(g.batch) * g.heads * g.nb;
  if (g.dtype == VSA_DTYPE_FP16)
    hipLaunchKernelGGL(gather_v_kernel<true>, dim3(unsigned(grid)), dim3(kThreads), 0, s,
                       static_cast<const uint4*>(x), static_cast<uint4*>(xbt), pooled, g);
  else
    hipLaunchKernelGGL(gather_v_kernel<false>, dim3(unsigned(grid)), dim3(kThreads), 0, s,
                       static_cast<const uint4*>(x), static_cast<uint4*>(xbt), pooled, g);
  return hipGetLastError();
}

hipError_t launch_scatter(const VsaGeom& g, const void* ob, const float* oc, const void* gate,
                          void* o, hipStream_t s) {
  const int64_t grid = int64_t(g.batch) * g.heads * g.nb;
  if (g.dtype == VSA_DTYPE_FP16)
    hipLaunchKernelGGL(scatter_kernel<true>, dim3(unsigned(grid)), dim3(kThreads), 0, s,
                       static_cast<const uint4*>(ob), oc, static_cast<const uint4*>(gate),
                       static_cast<uint4*>(o), g);
  else
    hipLaunchKernelGGL(scatter_kernel<false>, dim3(unsigned(grid)), dim3(kThreads), 0, s,
                       static_cast<const uint4*>(ob), oc, static_cast<const uint4*>(gate),
                       static_cast<uint4*>(o), g);
  return hipGetLastError();
}

}  // namespace vsa
