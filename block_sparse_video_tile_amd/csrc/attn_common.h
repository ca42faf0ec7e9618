// MFMA tile helpers shared by the attention kernels (forward and backward)
// on gfx950: operand types, the 32x32x16 product for bf16 or fp16, rounding
// to the element type, the kappa row permutation, padded LDS tile geometry
// and direct global->LDS copies.  Internal; not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vsa_internal.h"

namespace vsa {
namespace tile {

// Eight 16-bit elements (one MFMA operand per lane), held as bf16 bit
// patterns and reinterpreted when the tensors are fp16.
typedef __bf16 ev8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kUnits = 1024;  // 16-byte units in one 64 x 128 sub-tile of 16-bit elements (16 KB)

__device__ inline ev8 as_ev8(uint4 v) { return __builtin_bit_cast(ev8, v); }

// D = A B + C on 32x32x16 tiles of bf16 (F16 = false) or fp16 operands.
template <bool F16>
__device__ inline f32x16 mfma_32x32x16(ev8 a, ev8 b, f32x16 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Two fp32 values rounded to nearest-even in the element type, low half first.
template <bool F16>
__device__ inline uint32_t pack2(float a, float b) {
  if constexpr (F16) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 r = {_Float16(a), _Float16(b)};
    return __builtin_bit_cast(uint32_t, r);
  } else {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const b2 r = {__bf16(a), __bf16(b)};
    return __builtin_bit_cast(uint32_t, r);
  }
}

// One 16-bit element (the low half of `u`) as fp32: bf16 is the upper half
// of an fp32, fp16 converts exactly.
template <bool F16>
__device__ inline float elem_to_f32(uint32_t u) {
  if constexpr (F16) return float(__builtin_bit_cast(_Float16, uint16_t(u)));
  else return __uint_as_float(u << 16);
}

// Dispatch is round-robin over the 8 XCDs; give each XCD a contiguous run of rows.
__device__ inline int64_t xcd_remap(int64_t wg, int64_t n) {
  const int64_t per = n / 8, rem = n % 8;
  const int64_t x = wg % 8, loc = wg / 8;
  return (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + loc;
}

// Block at position p of a head's cost order: blocks grouped by edge class
// (bit 2, 1, 0: the block is the last along T, H, W, the place where the
// grid edge cuts a block if it cuts one; a grid that divides an axis has
// last blocks of full size there), the classes by descending valid-token
// count (then class number), the blocks of a class ascending.  A bijection
// on [0, nb).
__device__ inline int block_in_cost_order(const VsaGeom& g, int p) {
  // the class holding p: the last k whose start is <= p (an empty class
  // shares its start with the next one, so it is passed over)
  int k = 0;
#pragma unroll
  for (int x = 1; x < 8; ++x) k += p >= g.cstart[x] ? 1 : 0;
  int c = g.corder[0], q = p;
#pragma unroll
  for (int x = 1; x < 8; ++x)
    if (k == x) {
      c = g.corder[x];
      q = p - g.cstart[x];
    }
  // q-th block of class c, W fastest; a cut axis holds the last block index
  int iw = g.nbw - 1, ih = g.nbh - 1, it = g.nbt - 1;
  if (!(c & 1)) {
    iw = q % (g.nbw - 1);
    q /= g.nbw - 1;
  }
  if (!(c & 2)) {
    ih = q % (g.nbh - 1);
    q /= g.nbh - 1;
  }
  if (!(c & 4)) it = q;
  return (it * g.nbh + ih) * g.nbw + iw;
}

// Dynamic row assignment of the balanced launch.  The rows are cut into 8
// queues of consecutive positions (the ranges xcd_remap gives the XCDs, i.e.
// whole heads); the position r of a row within its head's nb is read through
// block_in_cost_order, so each head hands out its full blocks first and its
// cheaper edge blocks last: the workgroups running at once on an XCD have
// about equal cost (they stream the head's key blocks in step, which keeps
// shared blocks in L2), and the rows left at the end of the kernel are the
// cheap ones.  queues[8] hands out tickets and queues[x] counts the items
// taken from queue x; all start at zero.  The launch has more workgroups
// than items; a workgroup whose ticket is below the item count takes the
// next item of its own XCD's queue or, once that is empty, of the other
// queues in turn, and the others leave at once.  Each XCD works through its
// share of the workgroups as its CUs free up, so an XCD that runs faster
// takes more rows.  A ticket holder always finds an item: a queue it finds
// empty stays empty, and if all 8 were empty every item would already be
// held by one of the fewer-than-items other ticket holders.  Thread 0
// claims; the row reaches the workgroup through LDS.  With `order` (block
// maps of their own row lengths), position p of the queues is row order[p]
// instead of the cost order above: the rows of each queue range in the claim
// order of a block map (order_rows_kernel).
//   Tail split (split > 0): the last s = min(count, split) rows of a queue
// of `count` rows are handed out as two items each, their first and second
// halves, one after the other; *part_sh receives 2 * slot + half for such an
// item (slots numbered queue by queue, split_slots in all) and -1 for a
// whole row.
struct QueueItem {
  uint32_t p;  // position of the row within its queue
  int part;    // -1, or 2 * slot + half
};
__device__ inline QueueItem queue_item(uint32_t t, uint32_t count, uint32_t s, uint32_t slot0) {
  if (t < count - s) return {t, -1};
  const uint32_t u = t - (count - s);
  return {count - s + u / 2, int(2 * (slot0 + u / 2) + (u & 1))};
}

__device__ inline int64_t claim_row(unsigned int* queues, int64_t nrows, const VsaGeom& g,
                                    int64_t* row_sh, const int32_t* order = nullptr,
                                    uint32_t split = 0, int* part_sh = nullptr) {
  if (threadIdx.x == 0) {
    int64_t row = -1;
    int part = -1;
    // rows number at most 2^30 (the plan's limit): 32-bit arithmetic
    const uint32_t n = uint32_t(nrows);
    const uint32_t per = n / 8, rem = n % 8;
    const uint32_t s_hi = min(split, per + 1), s_lo = min(split, per);
    const uint32_t items = n + rem * s_hi + (8 - rem) * s_lo;
    if (atomicAdd(&queues[8], 1u) < items) {
      const int home = int(__builtin_amdgcn_s_getreg((3 << 11) | 20) & 7u);  // HW_REG_XCC_ID
      for (int j = 0; j < 8; ++j) {
        const uint32_t x = (home + j) & 7;
        const uint32_t count = per + (x < rem ? 1 : 0);
        if (count == 0) continue;
        const uint32_t s = x < rem ? s_hi : s_lo;
        const uint32_t t = atomicAdd(&queues[x], 1u);
        if (t < count + s) {
          const QueueItem it =
              queue_item(t, count, s, x < rem ? x * s_hi : rem * s_hi + (x - rem) * s_lo);
          part = it.part;
          const uint32_t pos = (x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per) + it.p;
          const uint32_t nb = uint32_t(g.nb);
          if (order != nullptr) {
            // a permutation of the rows; anything else leaves the row undone
            // rather than addressing memory outside the tensors
            const int32_t o = order[pos];
            row = (o >= 0 && uint32_t(o) < n) ? int64_t(o) : -1;
          } else {
            row = int64_t(pos / nb) * nb + block_in_cost_order(g, int(pos % nb));
          }
          break;
        }
      }
    }
    *row_sh = row;
    if (part_sh != nullptr) *part_sh = part;
  }
  __syncthreads();
  return *row_sh;
}

// claim_row with the heads interleaved over the queues (uniform rows of a
// layer whose key/value blocks outgrow the memory-side cache when the 8 XCDs
// each work on a different head): queue x holds, for every head in turn, the
// blocks at positions x, x+8, x+16, ... of the head's cost order, so all
// XCDs work on the same one or two heads at a time and the blocks they
// stream stay cached.  Same tickets, stealing, exit rule and tail split as
// claim_row; queue x here holds heads * ceil((nb - x) / 8) rows, so its
// split slots are numbered from the sum over the queues before it.
__device__ inline int64_t claim_row_strided(unsigned int* queues, int64_t nrows,
                                            const VsaGeom& g, int64_t* row_sh,
                                            uint32_t split = 0, int* part_sh = nullptr) {
  if (threadIdx.x == 0) {
    int64_t row = -1;
    int part = -1;
    const uint32_t n = uint32_t(nrows);
    const uint32_t nb = uint32_t(g.nb), heads = n / nb;
    uint32_t items = 0;
    for (uint32_t x = 0; x < 8; ++x) {
      const uint32_t count = (nb / 8 + (x < nb % 8 ? 1u : 0u)) * heads;
      items += count + min(split, count);
    }
    if (atomicAdd(&queues[8], 1u) < items) {
      const int home = int(__builtin_amdgcn_s_getreg((3 << 11) | 20) & 7u);  // HW_REG_XCC_ID
      for (int j = 0; j < 8; ++j) {
        const uint32_t x = (home + j) & 7;
        const uint32_t cx = nb / 8 + (x < nb % 8 ? 1u : 0u);   // positions of x per head
        const uint32_t count = cx * heads;
        if (count == 0) continue;
        const uint32_t s = min(split, count);
        const uint32_t t = atomicAdd(&queues[x], 1u);
        if (t < count + s) {
          uint32_t slot0 = 0;
          for (uint32_t y = 0; y < x; ++y)
            slot0 += min(split, (nb / 8 + (y < nb % 8 ? 1u : 0u)) * heads);
          const QueueItem it = queue_item(t, count, s, slot0);
          part = it.part;
          const uint32_t head = it.p / cx, p = (it.p % cx) * 8 + x;
          row = int64_t(head) * nb + block_in_cost_order(g, int(p));
          break;
        }
      }
    }
    *row_sh = row;
    if (part_sh != nullptr) *part_sh = part;
  }
  __syncthreads();
  return *row_sh;
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

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// One wave copies 64 x 16 bytes from global memory straight into LDS: lane l
// reads `src + off` and its 16 bytes land at `dst + 16*l`.  `src` is uniform
// and the byte offset 16*off is formed in 32 bits (callers keep it below
// 2^32), so the copy takes the scalar-base + 32-bit vector-offset form.
__device__ inline void wave_copy_to_lds(const uint4* src, uint32_t off, uint4* dst) {
  // The empty asm keeps the byte offset a 32-bit value at the copy: offsets
  // that are loop-invariant would otherwise be widened to 64 bits once,
  // outside the loop, and every copy would pay a 64-bit address add.
  uint32_t bytes = off * 16u;
  asm volatile("" : "+v"(bytes));
  __builtin_amdgcn_global_load_lds(
      static_cast<const void*>(reinterpret_cast<const char*>(src) + bytes), (lds_ptr_t)(dst), 16,
      0, 0);
}

// The same copy issued from inline asm, to the LDS byte address `lds`
// (wave-uniform) from `src` + `bytes` (per lane).  The compiler then does not
// see an LDS write in flight, so it inserts no waits for it before LDS reads
// (it cannot tell which buffer a copy whose destination is computed at run
// time targets, and would wait for every copy before every read): the caller
// waits for these copies itself (s_waitcnt vmcnt) before the barrier that
// publishes them.
__device__ inline void wave_copy_to_lds_async(const void* src, uint32_t bytes, uint32_t lds) {
  // s_nop: one wait state between the write of M0 and the copy that reads it
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(bytes), "s"(src), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// LDS byte address of a pointer into a __shared__ array.
__device__ inline uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)(const_cast<void*>(p))));
}

}  // namespace tile
}  // namespace vsa
