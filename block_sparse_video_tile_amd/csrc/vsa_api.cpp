// Host side of the C ABI declared in include/vsa.h: plan validation, the
// routing line, argument checks, and the sequencing of kernel launches.
// Every argument check runs before the first HIP call.

#include <algorithm>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>
#include <new>
#include <string>

#include "vsa_internal.h"

namespace {

thread_local std::string g_last_error;

vsa_status fail(vsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

vsa_status ok() {
  g_last_error.clear();
  return VSA_OK;
}

vsa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(VSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// True when any non-null pointer of the list is not a multiple of `a` bytes
// (element tensors are read and written as 16-byte units, fp32 and int32
// arrays as 4-byte words).
bool misaligned(uintptr_t a, std::initializer_list<const void*> ptrs) {
  for (const void* x : ptrs)
    if ((reinterpret_cast<uintptr_t>(x) & (a - 1)) != 0) return true;
  return false;
}

struct Workspace {
  size_t q, k, v, o, qp, kp, vp, oc, col, queue, split, total;
};

Workspace workspace_layout(const vsa_plan_s& p) {
  const VsaGeom& g = p.g;
  const size_t blk = size_t(g.batch) * g.heads * g.npad * g.head_dim * 2;
  const size_t pooled = size_t(g.batch) * g.heads * g.nb * g.head_dim * 4;
  const size_t col = size_t(g.batch) * g.heads * g.nb * (p.topk > 0 ? p.topk : 0) * 4;
  Workspace w;
  size_t off = 0;
  w.q = off; off += align256(blk);
  w.k = off; off += align256(blk);
  w.v = off; off += align256(blk);
  w.o = off; off += align256(blk);
  w.qp = off; off += align256(pooled);
  w.kp = off; off += align256(pooled);
  w.vp = off; off += align256(pooled);
  w.oc = off; off += align256(pooled);
  w.col = off; off += align256(col);
  w.queue = off; off += vsa::kAttnQueueBytes;
  w.split = off; off += align256(vsa::split_layout(g).total);
  w.total = off;
  return w;
}

// Workspace of the raster (gather-free) forward: pooled Q, K (and V and the
// coarse output for the gated branch) and the selected block ids.
struct FusedWorkspace {
  size_t qp, kp, vp, oc, col, queue, split, total;
};
FusedWorkspace fused_workspace_layout(const vsa_plan_s& p) {
  const VsaGeom& g = p.g;
  const size_t pooled = size_t(g.batch) * g.heads * g.nb * g.head_dim * 4;
  const size_t col = size_t(g.batch) * g.heads * g.nb * (p.topk > 0 ? p.topk : 0) * 4;
  FusedWorkspace w;
  size_t off = 0;
  w.qp = off; off += align256(pooled);
  w.kp = off; off += align256(pooled);
  w.vp = off; off += align256(pooled);
  w.oc = off; off += align256(pooled);
  w.col = off; off += align256(col);
  w.queue = off; off += vsa::kAttnQueueBytes;
  w.split = off; off += align256(vsa::split_layout(g).total);
  w.total = off;
  return w;
}

// Limits of the raster attention kernel: sub-tile descriptors hold the
// block's origin token in 21 bits, and a token's byte offset from its block
// origin in the raster tensor is a 32-bit value.
const char* raster_unsupported(const VsaGeom& g) {
  if (g.S >= (int64_t(1) << 21)) return "seq_len >= 2^21";
  const int64_t span = (int64_t(g.bt - 1) * g.H + (g.bh - 1)) * g.W + g.bw;
  if (span * g.heads * 256 >= (int64_t(1) << 32)) return "block span * num_heads too large";
  return nullptr;
}

struct BwdWorkspace {
  size_t dsum, tlist, tcount, queue, split, total;
};
BwdWorkspace bwd_workspace_layout(const vsa_plan_s& p) {
  const VsaGeom& g = p.g;
  const size_t heads = size_t(g.batch) * g.heads;
  BwdWorkspace w;
  size_t off = 0;
  w.dsum = off; off += align256(heads * g.npad * 4);
  w.tlist = off; off += align256(heads * g.nb * size_t(g.nb) * 4);
  w.tcount = off; off += align256(heads * g.nb * 4);
  w.queue = off; off += vsa::kAttnQueueBytes;
  w.split = off; off += align256(vsa::bwd_split_layout(g).total);
  w.total = off;
  return w;
}

}  // namespace

extern "C" {

const char* vsa_status_string(vsa_status st) {
  switch (st) {
    case VSA_OK: return "VSA_OK";
    case VSA_ERR_INVALID_ARGUMENT: return "VSA_ERR_INVALID_ARGUMENT";
    case VSA_ERR_UNSUPPORTED: return "VSA_ERR_UNSUPPORTED";
    case VSA_ERR_HIP: return "VSA_ERR_HIP";
  }
  return "VSA_ERR_UNKNOWN";
}

const char* vsa_last_error(void) { return g_last_error.c_str(); }

// Class order of a head's blocks for the balanced launches: the blocks of
// edge class c (bit 2, 1, 0: the block is the last along T, H, W, where the
// grid edge cuts it if it cuts one) number the product over the axes of 1
// (last) or blocks-along-the-axis - 1 (not last), and hold the product of
// the last extents (full where the grid divides the axis) and full block
// sizes as valid tokens.  Classes go by descending valid-token count, ties by class number.
static void fill_cost_order(VsaGeom& g) {
  const int nbd[3] = {g.nbt, g.nbh, g.nbw};
  const int full[3] = {g.bt, g.bh, g.bw};
  const int last[3] = {g.T - (g.nbt - 1) * g.bt, g.H - (g.nbh - 1) * g.bh,
                       g.W - (g.nbw - 1) * g.bw};
  int cnt[8], vol[8], ord[8];
  for (int c = 0; c < 8; ++c) {
    cnt[c] = 1;
    vol[c] = 1;
    for (int d = 0; d < 3; ++d) {
      const bool cut = (c >> (2 - d)) & 1;
      cnt[c] *= cut ? 1 : nbd[d] - 1;
      vol[c] *= cut ? last[d] : full[d];
    }
    ord[c] = c;
  }
  std::stable_sort(ord, ord + 8, [&](int a, int b) { return vol[a] > vol[b]; });
  int start = 0;
  for (int k = 0; k < 8; ++k) {
    g.corder[k] = ord[k];
    g.cstart[k] = start;
    start += cnt[ord[k]];
  }
}

vsa_status vsa_plan(const vsa_plan_desc* d, vsa_plan_t* out) {
  if (!d || !out) return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_plan: null desc or out pointer");
  *out = nullptr;
  for (int i = 0; i < 3; ++i) {
    if (d->dit_seq_shape[i] < 1)
      return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_plan: dit_seq_shape[%d] = %d must be >= 1", i,
                  d->dit_seq_shape[i]);
    if (d->block_size[i] < 1)
      return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_plan: block_size[%d] = %d must be >= 1", i,
                  d->block_size[i]);
  }
  if (d->batch < 1 || d->num_heads < 1 || d->head_dim < 1)
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_plan: batch, num_heads, head_dim must be >= 1");
  const int64_t T = d->dit_seq_shape[0], H = d->dit_seq_shape[1], W = d->dit_seq_shape[2];
  // products of three int32 extents can exceed int64: checked multiplication
  auto mul3 = [](int64_t a, int64_t b, int64_t c, int64_t* r) {
    return !__builtin_mul_overflow(a, b, r) && !__builtin_mul_overflow(*r, c, r);
  };
  int64_t thw = 0;
  if (!mul3(T, H, W, &thw))
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_plan: T*H*W overflows 64 bits");
  if (d->seq_len != thw)
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_plan: seq_len %lld != T*H*W = %lld",
                (long long)d->seq_len, (long long)thw);
  const int64_t nbt = (T + d->block_size[0] - 1) / d->block_size[0];
  const int64_t nbh = (H + d->block_size[1] - 1) / d->block_size[1];
  const int64_t nbw = (W + d->block_size[2] - 1) / d->block_size[2];
  int64_t nb = 0, vol = 0;
  if (!mul3(nbt, nbh, nbw, &nb) ||
      !mul3(d->block_size[0], d->block_size[1], d->block_size[2], &vol))
    return fail(VSA_ERR_UNSUPPORTED, "vsa_plan: problem too large for this implementation");
  if (d->topk < 0 || d->topk > nb)
    return fail(VSA_ERR_INVALID_ARGUMENT,
                "vsa_plan: topk %d outside [1, num_blocks=%lld] (0 selects map mode)", d->topk,
                (long long)nb);
  if (d->dtype != VSA_DTYPE_BF16 && d->dtype != VSA_DTYPE_FP16)
    return fail(VSA_ERR_UNSUPPORTED, "vsa_plan: dtype %d not implemented (bf16 or fp16)", d->dtype);
  if (d->head_dim != vsa::kHeadDim)
    return fail(VSA_ERR_UNSUPPORTED, "vsa_plan: head_dim %d not implemented (128 only)",
                d->head_dim);
  if (vol % 64 != 0 || vol > 256)
    return fail(VSA_ERR_UNSUPPORTED,
                "vsa_plan: block volume %lld not implemented (64, 128, 192 or 256)",
                (long long)vol);
  const int64_t npad = nb * vol;
  const int64_t elems = int64_t(d->batch) * d->num_heads * npad * d->head_dim;
  if (nb > (int64_t(1) << 20) || elems > (int64_t(1) << 40) ||
      int64_t(d->batch) * d->num_heads * nb > (int64_t(1) << 30))
    return fail(VSA_ERR_UNSUPPORTED, "vsa_plan: problem too large for this implementation");
  vsa_plan_s* p = new (std::nothrow) vsa_plan_s;
  if (!p) return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_plan: out of host memory");
  VsaGeom& g = p->g;
  g.T = int32_t(T); g.H = int32_t(H); g.W = int32_t(W);
  g.bt = d->block_size[0]; g.bh = d->block_size[1]; g.bw = d->block_size[2];
  g.nbt = int32_t(nbt); g.nbh = int32_t(nbh); g.nbw = int32_t(nbw);
  g.nb = int32_t(nb);
  g.vol = int32_t(vol);
  g.heads = d->num_heads;
  g.batch = d->batch;
  g.head_dim = d->head_dim;
  g.S = d->seq_len;
  g.npad = npad;
  g.dtype = d->dtype;
  fill_cost_order(g);
  // K and V of one head: Npad tokens x D x 2 bytes, twice; the 8 XCDs of the
  // balanced launch each work on one head unless that outgrows the 256 MB
  // memory-side (Infinity) cache.
  const int64_t kv_head_bytes = npad * d->head_dim * 2 * 2;
  g.head_interleave = 8 * kv_head_bytes > (int64_t(256) << 20) ? 1 : 0;
  p->topk = d->topk;
  p->dtype = d->dtype;
  *out = p;
  return ok();
}

vsa_status vsa_plan_destroy(vsa_plan_t plan) {
  delete plan;
  return ok();
}

vsa_status vsa_plan_get_info(vsa_plan_t p, vsa_plan_info* out) {
  if (!p || !out) return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_plan_get_info: null argument");
  const VsaGeom& g = p->g;
  out->block_grid[0] = g.nbt;
  out->block_grid[1] = g.nbh;
  out->block_grid[2] = g.nbw;
  out->num_blocks = g.nb;
  out->block_volume = g.vol;
  out->padded_len = g.npad;
  out->blocked_elems = int64_t(g.batch) * g.heads * g.npad * g.head_dim;
  out->pooled_elems = int64_t(g.batch) * g.heads * g.nb * g.head_dim;
  out->num_rows = int64_t(g.batch) * g.heads * g.nb;
  return ok();
}

vsa_status vsa_plan_describe(vsa_plan_t p, char* buf, size_t n) {
  if (!p || !buf) return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_plan_describe: null argument");
  const VsaGeom& g = p->g;
  char line[512];
  int len = snprintf(line, sizeof(line),
                     "seq_len=%lld, dit_seq_shape=(%d, %d, %d), block_size=(%d, %d, %d), "
                     "num_blocks=%d",
                     (long long)g.S, g.T, g.H, g.W, g.bt, g.bh, g.bw, g.nb);
  if (p->topk > 0) {
    len += snprintf(line + len, sizeof(line) - len, ", topk=%d, keep_ratio=%.1f%%, route=%s",
                    p->topk, 100.0 * p->topk / g.nb,
                    p->topk == g.nb ? "VSA_ALL_BLOCKS" : "VSA");
  }
  if (size_t(len) + 1 > n)
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_plan_describe: buffer of %zu bytes < %d needed",
                n, len + 1);
  memcpy(buf, line, size_t(len) + 1);
  return ok();
}

vsa_status vsa_plan_block_counts(vsa_plan_t p, int32_t* counts, int64_t n) {
  if (!p || !counts) return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_plan_block_counts: null argument");
  if (n < p->g.nb)
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_plan_block_counts: n = %lld < num_blocks = %d",
                (long long)n, p->g.nb);
  for (int b = 0; b < p->g.nb; ++b) counts[b] = vsa::block_count(p->g, b);
  return ok();
}

vsa_status vsa_gather(vsa_plan_t p, int32_t role, const void* x, void* xb, float* pooled,
                      void* stream) {
  if (!p || !x || (!xb && !pooled))
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_gather: null argument");
  if (role != VSA_ROLE_Q && role != VSA_ROLE_K && role != VSA_ROLE_V)
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_gather: unknown role %d", role);
  if (misaligned(16, {x, xb}) || misaligned(4, {pooled}))
    return fail(VSA_ERR_INVALID_ARGUMENT,
                "vsa_gather: x_raster and x_blk must be 16-byte aligned, pooled 4-byte aligned");
  if (!xb)  // block means only, for any role
    return hip_status(vsa::launch_gather_qk(p->g, x, nullptr, pooled, hipStream_t(stream)),
                      "vsa_gather(pooling)");
  if (role == VSA_ROLE_V)
    return hip_status(vsa::launch_gather_v(p->g, x, xb, pooled, hipStream_t(stream)),
                      "vsa_gather(V)");
  return hip_status(vsa::launch_gather_qk(p->g, x, xb, pooled, hipStream_t(stream)),
                    "vsa_gather(Q/K)");
}

vsa_status vsa_scatter(vsa_plan_t p, const void* ob, void* o, void* stream) {
  if (!p || !ob || !o) return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_scatter: null argument");
  if (misaligned(16, {ob, o}))
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_scatter: o_blk and o_raster not 16-byte aligned");
  return hip_status(vsa::launch_scatter(p->g, ob, nullptr, nullptr, o, hipStream_t(stream)),
                    "vsa_scatter");
}

vsa_status vsa_compress_attn(vsa_plan_t p, const float* qp, const float* kp, const float* vp,
                             float* oc, void* stream) {
  if (!p || !qp || !kp || !vp || !oc)
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_compress_attn: null argument");
  if ((reinterpret_cast<uintptr_t>(kp) & 15) != 0)
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_compress_attn: k_pooled not 16-byte aligned");
  if (misaligned(4, {qp, vp, oc}))
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_compress_attn: pooled arrays not 4-byte aligned");
  if (p->g.nb > 1024)
    return fail(VSA_ERR_UNSUPPORTED, "vsa_compress_attn: num_blocks %d > 1024 not implemented",
                p->g.nb);
  return hip_status(vsa::launch_compress_attn(p->g, qp, kp, vp, oc, hipStream_t(stream)),
                    "vsa_compress_attn");
}

vsa_status vsa_scatter_gated(vsa_plan_t p, const void* ob, const float* oc, const void* gate,
                             void* o, void* stream) {
  if (!p || !ob || !oc || !gate || !o)
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_scatter_gated: null argument");
  if ((reinterpret_cast<uintptr_t>(oc) & 15) != 0)
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_scatter_gated: o_coarse not 16-byte aligned");
  if (misaligned(16, {ob, gate, o}))
    return fail(VSA_ERR_INVALID_ARGUMENT,
                "vsa_scatter_gated: o_blk, gate and o_raster not 16-byte aligned");
  return hip_status(vsa::launch_scatter(p->g, ob, oc, gate, o, hipStream_t(stream)),
                    "vsa_scatter_gated");
}

vsa_status vsa_score_topk(vsa_plan_t p, const float* qp, const float* kp, int32_t topk,
                          int32_t* col, float* scores, void* stream) {
  if (!p || !qp || !kp || !col)
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_score_topk: null argument");
  if (topk < 1 || topk > p->g.nb)
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_score_topk: topk %d outside [1, %d]", topk,
                p->g.nb);
  if (misaligned(16, {kp}))
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_score_topk: k_pooled not 16-byte aligned");
  if (misaligned(4, {qp, col, scores}))
    return fail(VSA_ERR_INVALID_ARGUMENT,
                "vsa_score_topk: q_pooled, col_idx and scores not 4-byte aligned");
  if (p->g.nb > 1024)
    return fail(VSA_ERR_UNSUPPORTED, "vsa_score_topk: num_blocks %d > 1024 not implemented",
                p->g.nb);
  return hip_status(vsa::launch_score_topk(p->g, qp, kp, topk, col, scores, hipStream_t(stream)),
                    "vsa_score_topk");
}

}  // extern "C"

namespace {

// Argument checks shared by the attention entry points; returns ok() or the
// failure status (with its reason recorded).
vsa_status check_attn_args(const char* fn, vsa_plan_t p, const void* q, const void* k,
                           const void* v, const int32_t* row_ptr, const int32_t* col,
                           int32_t uniform_k, int64_t nnz, void* o) {
  if (!p || !q || !k || !v || !o) return fail(VSA_ERR_INVALID_ARGUMENT, "%s: null argument", fn);
  if (nnz < 0) return fail(VSA_ERR_INVALID_ARGUMENT, "%s: nnz < 0", fn);
  if (nnz > 0 && !col)
    return fail(VSA_ERR_INVALID_ARGUMENT, "%s: null col_idx with nnz > 0", fn);
  if (misaligned(16, {q, k, v, o}))
    return fail(VSA_ERR_INVALID_ARGUMENT, "%s: q, k, v and o must be 16-byte aligned", fn);
  if (misaligned(4, {row_ptr, col}))
    return fail(VSA_ERR_INVALID_ARGUMENT, "%s: row_ptr and col_idx must be 4-byte aligned", fn);
  const int64_t rows = int64_t(p->g.batch) * p->g.heads * p->g.nb;
  if (!row_ptr) {
    if (uniform_k < 0 || uniform_k > p->g.nb)
      return fail(VSA_ERR_INVALID_ARGUMENT, "%s: uniform_k %d outside [0, %d]", fn, uniform_k,
                  p->g.nb);
    if (nnz < rows * uniform_k)
      return fail(VSA_ERR_INVALID_ARGUMENT, "%s: nnz %lld < rows*uniform_k = %lld", fn,
                  (long long)nnz, (long long)(rows * uniform_k));
  }
  return ok();
}

vsa_status check_lse(const char* fn, const float* lse) {
  if (misaligned(4, {lse})) return fail(VSA_ERR_INVALID_ARGUMENT, "%s: lse not 4-byte aligned", fn);
  return ok();
}

vsa_status check_raster_args(const char* fn, vsa_plan_t p, const void* gate, const float* oc) {
  if ((gate == nullptr) != (oc == nullptr))
    return fail(VSA_ERR_INVALID_ARGUMENT, "%s: gate and o_coarse must both be given or both NULL",
                fn);
  if ((reinterpret_cast<uintptr_t>(oc) & 15) != 0)
    return fail(VSA_ERR_INVALID_ARGUMENT, "%s: o_coarse not 16-byte aligned", fn);
  if (misaligned(16, {gate}))
    return fail(VSA_ERR_INVALID_ARGUMENT, "%s: gate not 16-byte aligned", fn);
  if (const char* why = raster_unsupported(p->g))
    return fail(VSA_ERR_UNSUPPORTED, "%s: %s", fn, why);
  return ok();
}

// Workspace of the balanced attention launches: the row-queue counters, then
// one int32 per row for the claim order of a block map's rows, then the
// tail-split region (counters, rows, and the halves' partial results).
size_t attn_order_bytes(const VsaGeom& g) { return align256(size_t(g.batch) * g.heads * g.nb * 4); }
size_t attn_ws_bytes(const VsaGeom& g) {
  return vsa::kAttnQueueBytes + attn_order_bytes(g) + align256(vsa::split_layout(g).total);
}
// The three parts of a balanced launch's workspace (or of the fixed scratch).
struct AttnWs {
  unsigned int* queues;
  int32_t* order;
  vsa::TailSplit split;
};
AttnWs attn_ws_at(const VsaGeom& g, void* ws, size_t order_bytes) {
  char* b = static_cast<char*>(ws);
  return AttnWs{reinterpret_cast<unsigned int*>(b),
                reinterpret_cast<int32_t*>(b + vsa::kAttnQueueBytes),
                vsa::split_at(g, b + vsa::kAttnQueueBytes + order_bytes)};
}

vsa_status check_queue_workspace(const char* fn, vsa_plan_t p, void* ws, size_t ws_bytes) {
  if (!ws) return fail(VSA_ERR_INVALID_ARGUMENT, "%s: null workspace", fn);
  if (ws_bytes < attn_ws_bytes(p->g))
    return fail(VSA_ERR_INVALID_ARGUMENT, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes,
                attn_ws_bytes(p->g));
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0)
    return fail(VSA_ERR_INVALID_ARGUMENT, "%s: workspace not 256-byte aligned", fn);
  return ok();
}

}  // namespace

extern "C" {

vsa_status vsa_block_sparse_attn_fwd(vsa_plan_t p, const void* q, const void* k, const void* v,
                                     const int32_t* row_ptr, const int32_t* col,
                                     int32_t uniform_k, int64_t nnz, void* o, float* lse,
                                     void* stream) {
  static const char* fn = "vsa_block_sparse_attn_fwd";
  if (vsa_status st = check_attn_args(fn, p, q, k, v, row_ptr, col, uniform_k, nnz, o)) return st;
  if (vsa_status st = check_lse(fn, lse)) return st;
  return hip_status(vsa::launch_attn_fwd(p->g, q, k, v, row_ptr, col, uniform_k, nnz, o, lse,
                                         nullptr, nullptr, vsa::TailSplit{}, hipStream_t(stream)),
                    fn);
}

vsa_status vsa_attn_fwd_workspace_size(vsa_plan_t p, size_t* bytes) {
  if (!p || !bytes) return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_attn_fwd_workspace_size: null");
  *bytes = attn_ws_bytes(p->g);
  return ok();
}

vsa_status vsa_block_sparse_attn_fwd_ws(vsa_plan_t p, const void* q, const void* k, const void* v,
                                        const int32_t* row_ptr, const int32_t* col,
                                        int32_t uniform_k, int64_t nnz, void* o, float* lse,
                                        void* ws, size_t ws_bytes, void* stream) {
  static const char* fn = "vsa_block_sparse_attn_fwd_ws";
  if (vsa_status st = check_attn_args(fn, p, q, k, v, row_ptr, col, uniform_k, nnz, o)) return st;
  if (vsa_status st = check_lse(fn, lse)) return st;
  if (vsa_status st = check_queue_workspace(fn, p, ws, ws_bytes)) return st;
  const AttnWs a = attn_ws_at(p->g, ws, attn_order_bytes(p->g));
  return hip_status(vsa::launch_attn_fwd(p->g, q, k, v, row_ptr, col, uniform_k, nnz, o, lse,
                                         a.queues, a.order, a.split, hipStream_t(stream)),
                    fn);
}

vsa_status vsa_block_sparse_attn_fwd_noalloc(vsa_plan_t p, const void* q, const void* k,
                                             const void* v, const int32_t* row_ptr,
                                             const int32_t* col, int32_t uniform_k, int64_t nnz,
                                             void* o, float* lse, void* stream) {
  static const char* fn = "vsa_block_sparse_attn_fwd_noalloc";
  if (vsa_status st = check_attn_args(fn, p, q, k, v, row_ptr, col, uniform_k, nnz, o)) return st;
  if (vsa_status st = check_lse(fn, lse)) return st;
  // The scratch holds the 9 row-queue counters of the balanced launch (32-bit:
  // every plan's row count, at most 2^30, fits them) and, for a block map,
  // the claim order of at most kNoAllocMaxMapRows rows.
  const int64_t rows = int64_t(p->g.batch) * p->g.heads * p->g.nb;
  if (row_ptr != nullptr && rows > vsa::kNoAllocMaxMapRows)
    return fail(VSA_ERR_UNSUPPORTED,
                "%s: a block map of %lld rows exceeds the %lld rows of the fixed scratch "
                "(use vsa_block_sparse_attn_fwd_ws with a workspace)",
                fn, (long long)rows, (long long)vsa::kNoAllocMaxMapRows);
  void* ws = nullptr;
  if (hipError_t e = vsa::noalloc_scratch(&ws); e != hipSuccess)
    return hip_status(e, "vsa_block_sparse_attn_fwd_noalloc: scratch address");
  // the split region follows the order array of kNoAllocMaxMapRows rows; it
  // is sized for 8 x kSplitPerQueue slots of 8-wave halves, every plan's most
  if (vsa::split_layout(p->g).total > vsa::kNoAllocSplitBytes)
    return fail(VSA_ERR_UNSUPPORTED, "%s: tail-split region of %zu bytes exceeds the scratch's %zu",
                fn, vsa::split_layout(p->g).total, vsa::kNoAllocSplitBytes);
  const AttnWs a = attn_ws_at(p->g, ws, size_t(vsa::kNoAllocMaxMapRows) * 4);
  return hip_status(vsa::launch_attn_fwd(p->g, q, k, v, row_ptr, col, uniform_k, nnz, o, lse,
                                         a.queues, a.order, a.split, hipStream_t(stream)),
                    fn);
}

vsa_status vsa_block_sparse_attn_fwd_raster(vsa_plan_t p, const void* q, const void* k,
                                            const void* v, const int32_t* row_ptr,
                                            const int32_t* col, int32_t uniform_k, int64_t nnz,
                                            const void* gate, const float* oc, void* o,
                                            float* lse, void* stream) {
  static const char* fn = "vsa_block_sparse_attn_fwd_raster";
  if (vsa_status st = check_attn_args(fn, p, q, k, v, row_ptr, col, uniform_k, nnz, o)) return st;
  if (vsa_status st = check_lse(fn, lse)) return st;
  if (vsa_status st = check_raster_args(fn, p, gate, oc)) return st;
  return hip_status(vsa::launch_attn_fwd_raster(p->g, q, k, v, row_ptr, col, uniform_k, nnz, o,
                                                lse, gate, oc, nullptr, nullptr,
                                                vsa::TailSplit{}, hipStream_t(stream)),
                    fn);
}

vsa_status vsa_block_sparse_attn_fwd_raster_ws(vsa_plan_t p, const void* q, const void* k,
                                               const void* v, const int32_t* row_ptr,
                                               const int32_t* col, int32_t uniform_k, int64_t nnz,
                                               const void* gate, const float* oc, void* o,
                                               float* lse, void* ws, size_t ws_bytes,
                                               void* stream) {
  static const char* fn = "vsa_block_sparse_attn_fwd_raster_ws";
  if (vsa_status st = check_attn_args(fn, p, q, k, v, row_ptr, col, uniform_k, nnz, o)) return st;
  if (vsa_status st = check_lse(fn, lse)) return st;
  if (vsa_status st = check_raster_args(fn, p, gate, oc)) return st;
  if (vsa_status st = check_queue_workspace(fn, p, ws, ws_bytes)) return st;
  const AttnWs a = attn_ws_at(p->g, ws, attn_order_bytes(p->g));
  return hip_status(vsa::launch_attn_fwd_raster(p->g, q, k, v, row_ptr, col, uniform_k, nnz, o,
                                                lse, gate, oc, a.queues, a.order, a.split,
                                                hipStream_t(stream)),
                    fn);
}

vsa_status vsa_block_sparse_attn_bwd_workspace_size(vsa_plan_t p, size_t* bytes) {
  if (!p || !bytes)
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_block_sparse_attn_bwd_workspace_size: null");
  *bytes = bwd_workspace_layout(*p).total;
  return ok();
}

vsa_status vsa_block_sparse_attn_bwd(vsa_plan_t p, const void* q, const void* k, const void* v,
                                     const void* o, const void* dout, const float* lse,
                                     const int32_t* row_ptr, const int32_t* col,
                                     int32_t uniform_k, int64_t nnz, void* dq, void* dk, void* dv,
                                     void* ws, size_t ws_bytes, void* stream) {
  if (!p || !q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !ws)
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_block_sparse_attn_bwd: null argument");
  if (nnz < 0) return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_block_sparse_attn_bwd: nnz < 0");
  if (nnz > 0 && !col)
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_block_sparse_attn_bwd: null col_idx with nnz > 0");
  const int64_t rows = int64_t(p->g.batch) * p->g.heads * p->g.nb;
  if (!row_ptr) {
    if (uniform_k < 0 || uniform_k > p->g.nb)
      return fail(VSA_ERR_INVALID_ARGUMENT,
                  "vsa_block_sparse_attn_bwd: uniform_k %d outside [0, %d]", uniform_k, p->g.nb);
    if (nnz < rows * uniform_k)
      return fail(VSA_ERR_INVALID_ARGUMENT,
                  "vsa_block_sparse_attn_bwd: nnz %lld < rows*uniform_k = %lld", (long long)nnz,
                  (long long)(rows * uniform_k));
  }
  if (misaligned(16, {q, k, v, o, dout, dq, dk, dv}))
    return fail(VSA_ERR_INVALID_ARGUMENT,
                "vsa_block_sparse_attn_bwd: element tensors must be 16-byte aligned");
  if (misaligned(4, {lse, row_ptr, col}))
    return fail(VSA_ERR_INVALID_ARGUMENT,
                "vsa_block_sparse_attn_bwd: lse, row_ptr and col_idx must be 4-byte aligned");
  if (p->g.nb > 4096)
    return fail(VSA_ERR_UNSUPPORTED,
                "vsa_block_sparse_attn_bwd: num_blocks %d > 4096 not implemented", p->g.nb);
  const BwdWorkspace w = bwd_workspace_layout(*p);
  if (ws_bytes < w.total)
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_block_sparse_attn_bwd: workspace %zu bytes < %zu",
                ws_bytes, w.total);
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0)
    return fail(VSA_ERR_INVALID_ARGUMENT,
                "vsa_block_sparse_attn_bwd: workspace not 256-byte aligned");
  char* base = static_cast<char*>(ws);
  vsa::BwdArgs a;
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse;
  a.row_ptr = row_ptr; a.col = col; a.uniform_k = row_ptr ? 0 : uniform_k; a.nnz = nnz;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.dsum = reinterpret_cast<float*>(base + w.dsum);
  a.tlist = reinterpret_cast<int32_t*>(base + w.tlist);
  a.tcount = reinterpret_cast<int32_t*>(base + w.tcount);
  a.queues = reinterpret_cast<unsigned int*>(base + w.queue);
  const vsa::BwdSplitLayout sl = vsa::bwd_split_layout(p->g);
  a.split_flags = reinterpret_cast<unsigned int*>(base + w.split + sl.flags);
  a.split_rows = reinterpret_cast<int32_t*>(base + w.split + sl.rows);
  a.split_part = reinterpret_cast<float*>(base + w.split + sl.part);
  return hip_status(vsa::launch_attn_bwd(p->g, a, hipStream_t(stream)),
                    "vsa_block_sparse_attn_bwd");
}

vsa_status vsa_forward_workspace_size(vsa_plan_t p, size_t* bytes) {
  if (!p || !bytes) return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_forward_workspace_size: null");
  *bytes = workspace_layout(*p).total;
  return ok();
}

vsa_status vsa_forward(vsa_plan_t p, const void* q, const void* k, const void* v,
                       const void* gate, void* out, void* ws, size_t ws_bytes, int32_t* col_out,
                       float* lse, void* stream) {
  if (!p || !q || !k || !v || !out || !ws)
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_forward: null argument");
  if (p->topk < 1)
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_forward: plan is in map mode (topk == 0)");
  if (p->g.nb > 1024)
    return fail(VSA_ERR_UNSUPPORTED, "vsa_forward: num_blocks %d > 1024 not implemented",
                p->g.nb);
  const Workspace w = workspace_layout(*p);
  if (ws_bytes < w.total)
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_forward: workspace %zu bytes < %zu needed",
                ws_bytes, w.total);
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0)
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_forward: workspace not 256-byte aligned");
  if (misaligned(16, {q, k, v, gate, out}))
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_forward: q, k, v, gate and out must be 16-byte aligned");
  if (misaligned(4, {col_out, lse}))
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_forward: col_idx_out and lse must be 4-byte aligned");
  char* base = static_cast<char*>(ws);
  void* qb = base + w.q;
  void* kb = base + w.k;
  void* vb = base + w.v;
  void* ob = base + w.o;
  float* qp = reinterpret_cast<float*>(base + w.qp);
  float* kp = reinterpret_cast<float*>(base + w.kp);
  float* vp = reinterpret_cast<float*>(base + w.vp);
  float* oc = reinterpret_cast<float*>(base + w.oc);
  int32_t* col = col_out ? col_out : reinterpret_cast<int32_t*>(base + w.col);
  hipStream_t s = hipStream_t(stream);
  const VsaGeom& g = p->g;
  const int64_t nnz = int64_t(g.batch) * g.heads * g.nb * p->topk;
  hipError_t e;
  if ((e = vsa::launch_gather_qk(g, q, qb, qp, s)) != hipSuccess) return hip_status(e, "vsa_forward: gather Q");
  if ((e = vsa::launch_gather_qk(g, k, kb, kp, s)) != hipSuccess) return hip_status(e, "vsa_forward: gather K");
  if ((e = vsa::launch_gather_v(g, v, vb, gate ? vp : nullptr, s)) != hipSuccess)
    return hip_status(e, "vsa_forward: gather V");
  if ((e = vsa::launch_score_topk(g, qp, kp, p->topk, col, nullptr, s)) != hipSuccess)
    return hip_status(e, "vsa_forward: score/top-k");
  unsigned int* queues = reinterpret_cast<unsigned int*>(base + w.queue);
  if ((e = vsa::launch_attn_fwd(g, qb, kb, vb, nullptr, col, p->topk, nnz, ob, lse, queues,
                                nullptr, vsa::split_at(g, base + w.split), s)) != hipSuccess)
    return hip_status(e, "vsa_forward: attention");
  if (gate && (e = vsa::launch_compress_attn(g, qp, kp, vp, oc, s)) != hipSuccess)
    return hip_status(e, "vsa_forward: coarse attention");
  if ((e = vsa::launch_scatter(g, ob, gate ? oc : nullptr, gate, out, s)) != hipSuccess)
    return hip_status(e, "vsa_forward: scatter");
  return ok();
}

vsa_status vsa_forward_fused_workspace_size(vsa_plan_t p, size_t* bytes) {
  if (!p || !bytes)
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_forward_fused_workspace_size: null");
  *bytes = fused_workspace_layout(*p).total;
  return ok();
}

vsa_status vsa_forward_fused(vsa_plan_t p, const void* q, const void* k, const void* v,
                             const void* gate, void* out, void* ws, size_t ws_bytes,
                             int32_t* col_out, float* lse, void* stream) {
  if (!p || !q || !k || !v || !out || !ws)
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_forward_fused: null argument");
  if (p->topk < 1)
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_forward_fused: plan is in map mode (topk == 0)");
  if (p->g.nb > 1024)
    return fail(VSA_ERR_UNSUPPORTED, "vsa_forward_fused: num_blocks %d > 1024 not implemented",
                p->g.nb);
  if (const char* why = raster_unsupported(p->g))
    return fail(VSA_ERR_UNSUPPORTED, "vsa_forward_fused: %s", why);
  const FusedWorkspace w = fused_workspace_layout(*p);
  if (ws_bytes < w.total)
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_forward_fused: workspace %zu bytes < %zu needed",
                ws_bytes, w.total);
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0)
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_forward_fused: workspace not 256-byte aligned");
  if (misaligned(16, {q, k, v, gate, out}))
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_forward_fused: q, k, v, gate and out must be 16-byte aligned");
  if (misaligned(4, {col_out, lse}))
    return fail(VSA_ERR_INVALID_ARGUMENT, "vsa_forward_fused: col_idx_out and lse must be 4-byte aligned");
  char* base = static_cast<char*>(ws);
  float* qp = reinterpret_cast<float*>(base + w.qp);
  float* kp = reinterpret_cast<float*>(base + w.kp);
  float* vp = reinterpret_cast<float*>(base + w.vp);
  float* oc = reinterpret_cast<float*>(base + w.oc);
  int32_t* col = col_out ? col_out : reinterpret_cast<int32_t*>(base + w.col);
  hipStream_t s = hipStream_t(stream);
  const VsaGeom& g = p->g;
  const int64_t nnz = int64_t(g.batch) * g.heads * g.nb * p->topk;
  hipError_t e;
  if ((e = vsa::launch_gather_qk(g, q, nullptr, qp, s)) != hipSuccess)
    return hip_status(e, "vsa_forward_fused: pool Q");
  if ((e = vsa::launch_gather_qk(g, k, nullptr, kp, s)) != hipSuccess)
    return hip_status(e, "vsa_forward_fused: pool K");
  if ((e = vsa::launch_score_topk(g, qp, kp, p->topk, col, nullptr, s)) != hipSuccess)
    return hip_status(e, "vsa_forward_fused: score/top-k");
  if (gate) {
    if ((e = vsa::launch_gather_qk(g, v, nullptr, vp, s)) != hipSuccess)
      return hip_status(e, "vsa_forward_fused: pool V");
    if ((e = vsa::launch_compress_attn(g, qp, kp, vp, oc, s)) != hipSuccess)
      return hip_status(e, "vsa_forward_fused: coarse attention");
  }
  unsigned int* queues = reinterpret_cast<unsigned int*>(base + w.queue);
  if ((e = vsa::launch_attn_fwd_raster(g, q, k, v, nullptr, col, p->topk, nnz, out, lse, gate,
                                       gate ? oc : nullptr, queues, nullptr,
                                       vsa::split_at(g, base + w.split), s)) != hipSuccess)
    return hip_status(e, "vsa_forward_fused: attention");
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------- measurement kernels

extern "C" {

vsa_status vsa_bench_mfma_peak(int32_t num_workgroups, int32_t iters, uint64_t* timing,
                               int64_t* wall_clock_hz, void* stream) {
  static const char* fn = "vsa_bench_mfma_peak";
  if (!timing || !wall_clock_hz)
    return fail(VSA_ERR_INVALID_ARGUMENT, "%s: null timing or wall_clock_hz", fn);
  if (num_workgroups < 1 || num_workgroups > (1 << 20))
    return fail(VSA_ERR_INVALID_ARGUMENT, "%s: num_workgroups %d outside [1, 2^20]", fn,
                num_workgroups);
  if (iters < 1) return fail(VSA_ERR_INVALID_ARGUMENT, "%s: iters %d < 1", fn, iters);
  if ((reinterpret_cast<uintptr_t>(timing) & 7) != 0)
    return fail(VSA_ERR_INVALID_ARGUMENT, "%s: timing not 8-byte aligned", fn);
  int dev = 0, khz = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev);
  if (e != hipSuccess) return hip_status(e, "vsa_bench_mfma_peak: wall clock rate");
  *wall_clock_hz = int64_t(khz) * 1000;
  return hip_status(vsa::launch_mfma_peak(num_workgroups, iters, timing, hipStream_t(stream)), fn);
}

vsa_status vsa_bench_hbm_copy(const void* src, void* dst, int64_t bytes, void* stream) {
  static const char* fn = "vsa_bench_hbm_copy";
  if (!src || !dst) return fail(VSA_ERR_INVALID_ARGUMENT, "%s: null buffer", fn);
  if (bytes < 16 || bytes % 16 != 0)
    return fail(VSA_ERR_INVALID_ARGUMENT, "%s: bytes %lld not a positive multiple of 16", fn,
                (long long)bytes);
  if (((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15) != 0)
    return fail(VSA_ERR_INVALID_ARGUMENT, "%s: buffers not 16-byte aligned", fn);
  return hip_status(vsa::launch_hbm_copy(src, dst, bytes, hipStream_t(stream)), fn);
}

}  // extern "C"
