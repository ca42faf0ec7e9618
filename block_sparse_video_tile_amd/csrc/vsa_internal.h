// Internal declarations shared by the host ABI (vsa_api.cpp) and the HIP
// kernel sources.  Not part of the public interface (include/vsa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vsa.h"

// Geometry of one plan, passed to kernels by value.
struct VsaGeom {
  int32_t T, H, W;        // latent grid
  int32_t bt, bh, bw;     // block size
  int32_t nbt, nbh, nbw;  // block grid
  int32_t nb;             // number of blocks
  int32_t vol;            // block volume V
  int32_t heads;
  int32_t batch;
  int32_t head_dim;
  int64_t S;              // tokens
  int64_t npad;           // nb * vol
  int32_t dtype;          // vsa_dtype of Q, K, V and O
  // A head's blocks in cost order (read by the balanced launches): blocks
  // grouped by edge class (bit 2, 1, 0 set when the block is the last along
  // T, H, W, where the grid edge cuts it if it cuts one), classes by
  // descending valid-token count, ties by class number, blocks of a class in
  // ascending index.  corder[k] is
  // the k-th class, cstart[k] the position of its first block.
  int32_t corder[8];
  int32_t cstart[8];
  // Balanced forward launches with uniform rows: 1 when the K and V of the 8
  // heads the XCDs would work on at once (8 * Npad * D * 2 bytes * 2) exceed
  // the 256 MB memory-side cache; the queues then interleave the heads'
  // blocks so that every XCD works on the same head (claim_row_strided).
  int32_t head_interleave;
};

struct vsa_plan_s {
  VsaGeom g;
  int32_t topk;   // 0 = map mode
  int32_t dtype;
};

namespace vsa {

constexpr int kHeadDim = 128;
constexpr int kKvChunk = 64;  // keys per attention sub-tile and per V^T chunk

// Valid-token count of block `beta` (host and device).
__host__ __device__ inline int block_count(const VsaGeom& g, int beta) {
  const int plane = g.nbh * g.nbw;
  const int it = beta / plane;
  const int rem = beta - it * plane;
  const int ih = rem / g.nbw;
  const int iw = rem - ih * g.nbw;
  const int ct = min(g.bt, g.T - it * g.bt);
  const int ch = min(g.bh, g.H - ih * g.bh);
  const int cw = min(g.bw, g.W - iw * g.bw);
  return ct * ch * cw;
}

// xb == nullptr: block means only (any role)
hipError_t launch_gather_qk(const VsaGeom& g, const void* x, void* xb, float* pooled,
                            hipStream_t s);
hipError_t launch_gather_v(const VsaGeom& g, const void* x, void* xbt, float* pooled,
                           hipStream_t s);
// gate == nullptr: plain scatter; otherwise O + gate * oc[block] (oc fp32 [B,NH,nb,D])
hipError_t launch_scatter(const VsaGeom& g, const void* ob, const float* oc, const void* gate,
                          void* o, hipStream_t s);
// Tail split of the backward's balanced launches (TailSplit below, with the
// same rule as the forward's): a split dQ row or dK/dV column leaves two
// partial sums over halves of its entries, NW waves x 128 x 64 lanes fp32
// per half (dkv: dV^T and dK^T tiles; dq: the first half of that).
constexpr size_t kBwdSplitHalfFloatsPerWave = 128 * 64;
// Device buffers of one backward call (blocked layouts; see vsa.h).
struct BwdArgs {
  const void *q, *k, *v, *o, *dout;   // token-major blocked inputs
  const float* lse;                   // forward LSE [B,NH,Npad]
  const int32_t* row_ptr;             // CSR (nullptr = uniform rows)
  const int32_t* col;
  int uniform_k;
  int64_t nnz;
  void *dq, *dk, *dv;                 // token-major blocked outputs
  // workspace
  float* dsum;                        // rowsum(dO * O) [B,NH,Npad]
  int32_t* tlist;                     // [B*NH*nb][nb] transposed block map
  int32_t* tcount;                    // [B*NH*nb]
  unsigned int* queues;               // row-queue counters (kAttnQueueBytes)
  unsigned int* split_flags;          // tail split: a counter per slot,
  int32_t* split_rows;                //   the row / column of each slot,
  float* split_part;                  //   two partial sums per slot
};
hipError_t launch_attn_bwd(const VsaGeom& g, const BwdArgs& a, hipStream_t s);

hipError_t launch_compress_attn(const VsaGeom& g, const float* qp, const float* kp,
                                const float* vp, float* oc, hipStream_t s);
hipError_t launch_score_topk(const VsaGeom& g, const float* qp, const float* kp, int topk,
                             int32_t* col, float* scores, hipStream_t s);
// queues == nullptr: one workgroup per row in a fixed order; otherwise 9
// device counters (kAttnQueueBytes of workspace) from which the workgroups
// of a larger launch claim their rows.  order: with queues and a block map
// (row_ptr), an int32 buffer of one entry per row that receives the rows of
// each queue in claim order (long rows first, then head by head by entry
// count; nullptr: claims in plain order).
constexpr size_t kAttnQueueBytes = 256;

// Tail split of the balanced forward launches.  The last kSplitPerQueue rows
// of each of the 8 row queues (the last rows the kernel hands out) are run as
// two halves, the first and the second half of the row's entries, each by a
// workgroup of its own; each half leaves its unnormalised (O, m, l) in the
// workspace and the half that finishes second merges both and writes the row.
// The kernel's last round then consists of half rows, so the CUs run out of
// work closer together.  A queue of c rows splits min(c, kSplitPerQueue).
// Launches whose longest queue holds more than kSplitMaxQueueRows rows (8
// rows for each of an XCD's 32 CUs) split none: over that many rounds the
// last round's idle time is a small share of the kernel and the split rows'
// second prologue and partial-result traffic cost about as much as they save
// (measured: a 27280-token layer of 24 heads, 360 rows per queue, +-0.5%;
// its 3-head shard, 45 rows per queue, 15% faster).
constexpr int kSplitPerQueue = 16;
constexpr int64_t kSplitMaxQueueRows = 256;
struct TailSplit {
  unsigned int* flags;  // one counter per split slot, cleared before the launch
  float* part;          // per slot and half: NW waves x 66 x 64 lanes fp32 (O^T, m, l)
  int32_t* rows;        // the row of each slot, written by its merge
  int32_t per_queue;    // 0: no split
};
// Split slots of a launch over `nrows` rows (queue x holds the rows that
// xcd_remap gives XCD x: nrows/8, the first nrows%8 queues one more).
__host__ __device__ inline int64_t split_slots(int64_t nrows, int per_queue) {
  const int64_t per = nrows / 8, rem = nrows % 8;
  const int64_t hi = per + 1 < per_queue ? per + 1 : per_queue;
  const int64_t lo = per < per_queue ? per : per_queue;
  return rem * hi + (8 - rem) * lo;
}
// Split slots of either claim rule of a plan: queues cut as xcd_remap cuts
// the rows, or (heads interleaved over the queues, uniform rows) queue x
// holding heads * ceil((nb - x) / 8) rows.
inline int64_t split_slots_max(const VsaGeom& g, int per_queue) {
  const int64_t heads = int64_t(g.batch) * g.heads;
  const int64_t plain = split_slots(heads * g.nb, per_queue);
  int64_t strided = 0;
  for (int x = 0; x < 8; ++x) {
    const int64_t count = (g.nb / 8 + (x < g.nb % 8 ? 1 : 0)) * heads;
    strided += count < per_queue ? count : per_queue;
  }
  return plain > strided ? plain : strided;
}
// Waves of the attention workgroup for a block volume (64-token blocks: 4).
inline int attn_waves(const VsaGeom& g) { return g.vol == 64 ? 4 : g.vol / 32; }
constexpr size_t kSplitHalfFloatsPerWave = 66 * 64;
// Bytes of the tail-split region of a plan: flags, rows, halves.
struct SplitLayout {
  size_t flags, rows, part, total;
};
inline SplitLayout split_layout(const VsaGeom& g) {
  const int64_t slots = split_slots_max(g, kSplitPerQueue);
  auto a256 = [](size_t n) { return (n + 255) & ~size_t(255); };
  SplitLayout l;
  l.flags = 0;
  l.rows = a256(size_t(slots) * 4);
  l.part = l.rows + a256(size_t(slots) * 4);
  l.total = l.part + size_t(slots) * 2 * attn_waves(g) * kSplitHalfFloatsPerWave * 4;
  return l;
}
inline TailSplit split_at(const VsaGeom& g, void* base) {
  const SplitLayout l = split_layout(g);
  char* b = static_cast<char*>(base);
  return TailSplit{reinterpret_cast<unsigned int*>(b + l.flags), reinterpret_cast<float*>(b + l.part),
                   reinterpret_cast<int32_t*>(b + l.rows), kSplitPerQueue};
}

// Bytes of the backward's tail-split region (counters, ids, partial sums of
// workgroups of vol/32 waves), 256-byte aligned parts.
struct BwdSplitLayout {
  size_t flags, rows, part, total;
};
inline BwdSplitLayout bwd_split_layout(const VsaGeom& g) {
  const int64_t slots = split_slots(int64_t(g.batch) * g.heads * g.nb, kSplitPerQueue);
  auto a256 = [](size_t n) { return (n + 255) & ~size_t(255); };
  BwdSplitLayout l;
  l.flags = 0;
  l.rows = a256(size_t(slots) * 4);
  l.part = l.rows + a256(size_t(slots) * 4);
  l.total = l.part + size_t(slots) * 2 * (g.vol / 32) * kBwdSplitHalfFloatsPerWave * 4;
  return l;
}

hipError_t launch_attn_fwd(const VsaGeom& g, const void* q, const void* k, const void* vt,
                           const int32_t* row_ptr, const int32_t* col, int uniform_k,
                           int64_t nnz, void* o, float* lse, unsigned int* queues,
                           int32_t* order, const TailSplit& ts, hipStream_t s);
// Fixed device scratch of the no-allocation attention entry point: the row
// queues, the claim order of the rows of a block map of at most
// kNoAllocMaxMapRows rows, then the tail-split region of at most 8 x
// kSplitPerQueue slots of 8-wave halves; and its device address on the
// current device.
constexpr int64_t kNoAllocMaxMapRows = int64_t(1) << 16;
constexpr size_t kNoAllocSplitBytes =
    2 * ((size_t(8 * kSplitPerQueue) * 4 + 255) & ~size_t(255)) +
    size_t(8 * kSplitPerQueue) * 2 * 8 * kSplitHalfFloatsPerWave * 4;
constexpr size_t kNoAllocScratchBytes =
    kAttnQueueBytes + size_t(kNoAllocMaxMapRows) * 4 + kNoAllocSplitBytes;
hipError_t noalloc_scratch(void** ptr);
// Raster [B,S,NH,D] q, k, v and o; gate (raster) and oc (fp32 [B,NH,nb,D])
// optional: o = attention + gate * oc[block].
hipError_t launch_attn_fwd_raster(const VsaGeom& g, const void* q, const void* k, const void* v,
                                  const int32_t* row_ptr, const int32_t* col, int uniform_k,
                                  int64_t nnz, void* o, float* lse, const void* gate,
                                  const float* oc, unsigned int* queues, int32_t* order,
                                  const TailSplit& ts, hipStream_t s);

// Measurement kernels (microbench.hip): `timing` holds 4 uint64 per wave.
hipError_t launch_mfma_peak(int num_workgroups, int iters, uint64_t* timing, hipStream_t s);
hipError_t launch_hbm_copy(const void* src, void* dst, int64_t bytes, hipStream_t s);

}  // namespace vsa
