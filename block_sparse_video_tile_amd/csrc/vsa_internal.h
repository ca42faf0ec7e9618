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
  // grouped by edge class (bit 2, 1, 0 set when the grid edge cuts the
  // block's T, H, W extent), classes by descending valid-token count, ties
  // by class number, blocks of a class in ascending index.  corder[k] is
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
hipError_t launch_attn_fwd(const VsaGeom& g, const void* q, const void* k, const void* vt,
                           const int32_t* row_ptr, const int32_t* col, int uniform_k,
                           int64_t nnz, void* o, float* lse, unsigned int* queues,
                           int32_t* order, hipStream_t s);
// Fixed device scratch of the no-allocation attention entry point: the row
// queues, then the claim order of the rows of a block map of at most
// kNoAllocMaxMapRows rows; and its device address on the current device.
constexpr int64_t kNoAllocMaxMapRows = int64_t(1) << 16;
constexpr size_t kNoAllocScratchBytes = kAttnQueueBytes + size_t(kNoAllocMaxMapRows) * 4;
hipError_t noalloc_scratch(void** ptr);
// Raster [B,S,NH,D] q, k, v and o; gate (raster) and oc (fp32 [B,NH,nb,D])
// optional: o = attention + gate * oc[block].
hipError_t launch_attn_fwd_raster(const VsaGeom& g, const void* q, const void* k, const void* v,
                                  const int32_t* row_ptr, const int32_t* col, int uniform_k,
                                  int64_t nnz, void* o, float* lse, const void* gate,
                                  const float* oc, unsigned int* queues, int32_t* order,
                                  hipStream_t s);

// Measurement kernels (microbench.hip): `timing` holds 4 uint64 per wave.
hipError_t launch_mfma_peak(int num_workgroups, int iters, uint64_t* timing, hipStream_t s);
hipError_t launch_hbm_copy(const void* src, void* dst, int64_t bytes, hipStream_t s);

}  // namespace vsa
