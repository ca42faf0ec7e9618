/*
 * vsa.h -- C ABI of the MI355X (gfx950) Video Sparse Attention hot path.
 *
 * What the path computes (the "FastVideo VSA" user guide, intro): the
 * post-patch latent grid (T, H, W) of a video DiT layer is cut into
 * spatiotemporal blocks; every key/value block is scored for every query
 * block, and exact softmax attention runs only against the top-k key/value
 * blocks of each query block.  The same guide's "Choose top-k" section gives
 * the shape vocabulary (seq_len, dit_seq_shape, block_size, num_blocks, topk,
 * keep_ratio) and states that top-k counts key/value blocks kept per query
 * block; "Verify routing and fallback" lists the kernel's operating
 * conditions (bf16/fp16 tensors, 256-token blocks, head_size**-0.5 scaling,
 * equal head counts, no mask, no sequence parallelism).  FastVideo's
 * h3-perf-stack commit log (sm_100a tile-64 route entry) adds 64-token 1-D
 * tiles and compacted block maps whose per-row counts differ from row to row
 * and may be zero.
 *
 * Conventions shared by every call:
 *   - Every function returns vsa_status; on failure vsa_last_error() returns
 *     a thread-local reason string.  Nothing aborts and no C++ exception
 *     crosses this boundary.
 *   - Device pointers are caller-owned HIP device allocations on the current
 *     device; the library never allocates, frees or retains them.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device work is enqueued asynchronously on it; no call synchronises the
 *     host.  Device faults surface at the caller's next synchronisation.
 *   - Element types: the Q, K, V and O tensors ("elem" below) are all of the
 *     plan's dtype, 2-byte bfloat16 or IEEE binary16 ("Verify routing and
 *     fallback" admits FP16 or BF16); fp32 is IEEE binary32, indices are
 *     int32.  Pooled means, scores and LSE are fp32 for either dtype.
 *   - Alignment: elem tensors (Q, K, V, O, gate, gradients) are read and
 *     written as 16-byte units and must be 16-byte aligned; k_pooled and
 *     o_coarse are read as float4 and must be 16-byte aligned too; every
 *     other fp32 or int32 array must be 4-byte aligned.  A misaligned
 *     pointer is INVALID_ARGUMENT.
 *   - Host-side argument checks happen before any HIP call, so every
 *     VSA_ERR_INVALID_ARGUMENT / VSA_ERR_UNSUPPORTED path works without a GPU.
 *
 * Layouts (B = batch, NH = heads, D = head_dim = 128, S = seq_len,
 * nb = num_blocks, V = block volume = bt*bh*bw, Npad = nb*V):
 *   raster   [B, S, NH, D]   token s = (t*H + h)*W + w, w fastest.
 *   blocked  [B, NH, Npad, D]  block b occupies rows b*V .. b*V+V-1; its
 *            c_b valid tokens come first in raster order, the remaining
 *            V - c_b rows are zero padding.  Used for Q, K and O.
 *   blocked-V^T [B, NH, Npad/64, D, 64]  the same token rows cut into
 *            64-token chunks, each chunk stored d-major (token index
 *            fastest), padding zero.  Used for V.
 *   pooled   [B, NH, nb, D] fp32.
 *   scores   [B, NH, nb, nb] fp32, row = query block, column = key block.
 *   CSR rows r = (b*NH + h)*nb + i; col_idx entries are key-block ids in
 *            [0, nb) of the same (b, h).
 *   lse      [B, NH, Npad] fp32, natural log; -inf on empty rows and pads.
 */
#ifndef VSA_H_
#define VSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum vsa_status {
  VSA_OK = 0,
  VSA_ERR_INVALID_ARGUMENT = 1, /* null pointer, inconsistent or out-of-range size */
  VSA_ERR_UNSUPPORTED = 2,      /* valid request outside what the kernels implement */
  VSA_ERR_HIP = 3               /* a HIP runtime call or kernel launch failed */
} vsa_status;

typedef enum vsa_dtype { VSA_DTYPE_BF16 = 0, VSA_DTYPE_FP16 = 1 } vsa_dtype;

typedef enum vsa_role { VSA_ROLE_Q = 0, VSA_ROLE_K = 1, VSA_ROLE_V = 2 } vsa_role;

/* Shape of one attention layer call ("FastVideo VSA" guide, "Choose top-k":
 * the fields of its routing log line). */
typedef struct vsa_plan_desc {
  int64_t seq_len;          /* S; must equal T*H*W */
  int32_t dit_seq_shape[3]; /* (T, H, W) post-patch latent grid, each >= 1 */
  int32_t block_size[3];    /* (bt, bh, bw); V = bt*bh*bw in {64, 128, 192, 256} */
  int32_t batch;            /* B >= 1 */
  int32_t num_heads;        /* NH >= 1; equal for Q, K and V */
  int32_t head_dim;         /* D; 128 is implemented */
  int32_t topk;             /* key blocks kept per query block, 1..nb; 0 = the
                               caller supplies a block map (CSR) instead */
  int32_t dtype;            /* vsa_dtype of Q, K, V and O: BF16 or FP16 */
} vsa_plan_desc;

/* Derived sizes of a plan (host values). */
typedef struct vsa_plan_info {
  int32_t block_grid[3];    /* (ceil(T/bt), ceil(H/bh), ceil(W/bw)) */
  int32_t num_blocks;       /* nb = product of block_grid */
  int32_t block_volume;     /* V */
  int64_t padded_len;       /* Npad = nb*V */
  int64_t blocked_elems;    /* B*NH*Npad*D elements of one blocked tensor */
  int64_t pooled_elems;     /* B*NH*nb*D */
  int64_t num_rows;         /* B*NH*nb CSR rows */
} vsa_plan_info;

typedef struct vsa_plan_s* vsa_plan_t;

/* Validate `desc` and build an immutable host-side plan.  Makes no HIP call.
 * Block ids are raster-ordered over the block grid (t-major); a block's valid
 * count is the product over t, h, w of min(b_d, G_d - i_d*b_d).
 * Errors: INVALID_ARGUMENT for null pointers, non-positive sizes,
 *   seq_len != T*H*W, topk < 0 or topk > nb ("Choose top-k": larger than
 *   num_blocks is invalid; "Enable the backend": it must be positive, with 0
 *   reserved here for map mode); UNSUPPORTED for head_dim != 128, a dtype
 *   other than BF16 or FP16, or V not in {64, 128, 192, 256}.
 * Ownership: *out is owned by the caller and released with vsa_plan_destroy;
 * a plan may be shared across threads and streams. */
vsa_status vsa_plan(const vsa_plan_desc* desc, vsa_plan_t* out);

/* Release a plan (NULL is accepted and ignored). */
vsa_status vsa_plan_destroy(vsa_plan_t plan);

/* Copy the derived sizes of `plan` into *out. */
vsa_status vsa_plan_get_info(vsa_plan_t plan, vsa_plan_info* out);

/* Write the NUL-terminated routing line of the plan into buf[0..buf_len):
 * "seq_len=S, dit_seq_shape=(T, H, W), block_size=(bt, bh, bw),
 *  num_blocks=nb, topk=k, keep_ratio=P%, route=VSA" with P = 100*k/nb to one
 * decimal, the fields of the routing log line in "Choose top-k".  The route
 * is VSA_ALL_BLOCKS when k == nb (the all-block path always runs the sparse
 * kernel) and the topk/keep_ratio/route fields are omitted in map mode.
 * Errors: INVALID_ARGUMENT if buf is NULL or buf_len is too small (nothing is
 * written beyond buf_len). */
vsa_status vsa_plan_describe(vsa_plan_t plan, char* buf, size_t buf_len);

/* Host array of the nb per-block valid-token counts, in block-id order.
 * `n` must be >= nb. */
vsa_status vsa_plan_block_counts(vsa_plan_t plan, int32_t* counts, int64_t n);

/* Raster -> blocked gather with tail padding (pad rows written as zero).
 * role Q or K: writes x_blk in the blocked layout and, if `pooled` is not
 * NULL, the fp32 mean of each block's valid tokens (the per-block pooled
 * vector the block score is built from: the guide's intro has every key block
 * scored per query block, and the h3 FastH3 log entry pools per tile).
 * role V: writes x_blk in the blocked-V^T layout and, if `pooled` is not
 * NULL, the fp32 mean of each block's valid values (the gate-compress
 * branch's pooled values; h3 FastH3 log entry: that branch pools per tile).
 * x_blk == NULL (any role, `pooled` required): the block means alone, read
 * straight from the raster tensor with nothing else written -- the pooling
 * pass of the gather-free path (vsa_forward_fused).
 * x_raster: device, B*S*NH*D elem.  x_blk: device, B*NH*Npad*D elem, or NULL.
 * pooled: device, B*NH*nb*D fp32, or NULL.
 * Errors: INVALID_ARGUMENT for a null plan or x_raster, both x_blk and pooled
 *   NULL, or an unknown role. */
vsa_status vsa_gather(vsa_plan_t plan, int32_t role, const void* x_raster, void* x_blk,
                      float* pooled, void* stream);

/* Blocked -> raster scatter of an output tensor: the inverse of vsa_gather's
 * token permutation, so that the attention output is handed back in the
 * post-patch latent order the layer received ("FastVideo VSA" guide, intro:
 * the blocks are a partition of that grid; "Choose top-k": padding of edge
 * blocks is an overhead of the tiling, not part of the result).  Pad rows are
 * dropped.  o_blk: device, blocked layout, elem.  o_raster: device, raster
 * layout, elem.  Errors: INVALID_ARGUMENT for a null plan or buffer. */
vsa_status vsa_scatter(vsa_plan_t plan, const void* o_blk, void* o_raster, void* stream);

/* Gate-compress (coarse) branch ("FastVideo VSA" guide, "Checkpoint
 * behavior": a learned to_gate_compress projection compensates the sparse
 * branch; h3 FastH3 log entry: the branch pools per tile).  The pages give
 * no formula; this computes attention among the per-tile pooled tokens:
 *   o_coarse[b,h,i] = sum_j softmax_j(q_pooled[b,h,i] . k_pooled[b,h,j] / sqrt(D))
 *                     * v_pooled[b,h,j]
 * over all nb blocks, in fp32.
 * q_pooled, k_pooled, v_pooled: device fp32 pooled layout (vsa_gather with
 * `pooled`), k_pooled 16-byte aligned.  o_coarse: device fp32, pooled layout.
 * Errors: INVALID_ARGUMENT for null or misaligned pointers; UNSUPPORTED for
 *   nb > 1024. */
vsa_status vsa_compress_attn(vsa_plan_t plan, const float* q_pooled, const float* k_pooled,
                             const float* v_pooled, float* o_coarse, void* stream);

/* Blocked -> raster scatter of the sparse output combined with the gated
 * coarse output: for every valid token s of block i,
 *   o_raster[b,s,h,:] = o_blk[b,h,row(s),:] + gate[b,s,h,:] * o_coarse[b,h,i,:]
 * elementwise in fp32, rounded once to elem.  gate: device elem raster
 * [B,S,NH,D] (the output of the caller's to_gate_compress projection).
 * o_coarse: device fp32 pooled layout, 16-byte aligned.  o_blk, o_raster as
 * for vsa_scatter.
 * Errors: INVALID_ARGUMENT for null or misaligned pointers. */
vsa_status vsa_scatter_gated(vsa_plan_t plan, const void* o_blk, const float* o_coarse,
                             const void* gate, void* o_raster, void* stream);

/* Block score and per-row top-k ("FastVideo VSA" guide, intro: every key
 * block is scored for every query block and the top-k are kept).
 * score[i][j] = dot(q_pooled[i], k_pooled[j]) in fp32 per (b, h); each row
 * keeps its `topk` largest scores, ties going to the lower block index, and
 * writes their block ids ascending to col_idx[row*topk .. row*topk+topk).
 * The rows are uniform CSR rows (row_ptr[r] = r*topk).
 * q_pooled, k_pooled: device fp32 pooled layout.  col_idx: device int32,
 * B*NH*nb*topk entries.  scores: device fp32 [B,NH,nb,nb] or NULL.
 * Errors: INVALID_ARGUMENT for null inputs or topk outside [1, nb]. */
vsa_status vsa_score_topk(vsa_plan_t plan, const float* q_pooled, const float* k_pooled,
                          int32_t topk, int32_t* col_idx, float* scores, void* stream);

/* Block-sparse attention forward on blocked tensors ("FastVideo VSA" guide,
 * intro: attention only against the selected blocks; "Verify routing and
 * fallback": non-causal, equal Q/KV lengths, scale head_dim**-0.5, equal head
 * counts; h3-perf-stack log, sm_100a entry: non-uniform and zero-count rows).
 * For every valid query token of block i in row r the output is
 *   softmax_j(q . k_j / sqrt(D)) v_j over the valid tokens of the blocks
 *   listed in row r,
 * padded keys masked; an empty row yields O = 0 and LSE = -inf; pad query
 * rows are written as 0 (LSE -inf).
 * q_blk, k_blk: device elem blocked layout.  v_blk: device elem blocked-V^T.
 * Products and softmax run in fp32; P is rounded to elem for the PV product
 * and O is rounded to elem.
 * row_ptr: device int32 [B*NH*nb + 1] CSR offsets into col_idx, or NULL for
 *   uniform rows of `uniform_k` entries each (row r uses entries
 *   r*uniform_k .. r*uniform_k + uniform_k - 1).
 * col_idx: device int32 block ids, `nnz` entries (nnz = B*NH*nb*uniform_k in
 *   uniform mode).  Row offsets are clamped to [0, nnz] and ids outside
 *   [0, nb) are skipped, so a malformed map cannot read out of bounds.  Ids in
 *   a row must be unique (a repeated id weighs that block twice); ascending
 *   order is recommended for cache reuse, the result does not depend on it.
 * o_blk: device elem blocked layout.  lse: device fp32 [B,NH,Npad] or NULL.
 * Errors: INVALID_ARGUMENT for null pointers, nnz < 0, uniform_k outside
 *   [0, nb] in uniform mode. */
vsa_status vsa_block_sparse_attn_fwd(vsa_plan_t plan, const void* q_blk, const void* k_blk,
                                     const void* v_blk, const int32_t* row_ptr,
                                     const int32_t* col_idx, int32_t uniform_k, int64_t nnz,
                                     void* o_blk, float* lse, void* stream);

/* The same attention on raster tensors, with no gather or scatter pass
 * ("FastVideo VSA" guide, "Choose top-k": tiling shapes that do not divide
 * the grid cost routing and padding overhead; this variant leaves the tokens
 * where they are).  Each query block's tokens and the selected key blocks'
 * tokens are located by block index arithmetic inside the kernel, O is
 * written straight to its raster rows, and the result is identical to
 * vsa_block_sparse_attn_fwd followed by vsa_scatter (same products in the
 * same order).
 * q, k, v, o_raster: device elem raster [B,S,NH,D] (16-byte aligned rows).
 * lse: device fp32 [B,NH,Npad] in the blocked row order, or NULL.
 * row_ptr, col_idx, uniform_k, nnz: as for vsa_block_sparse_attn_fwd.
 * gate, o_coarse: both NULL, or the gate (device elem raster) and the coarse
 *   output (device fp32 pooled layout, 16-byte aligned): each token row is
 *   then written as vsa_scatter_gated writes it, O + gate * o_coarse[block],
 *   bit for bit.
 * Errors: as vsa_block_sparse_attn_fwd, plus INVALID_ARGUMENT for only one of
 *   gate / o_coarse or a misaligned o_coarse, and UNSUPPORTED for
 *   seq_len >= 2^21 or (block span in tokens) * NH * 256 >= 2^32. */
vsa_status vsa_block_sparse_attn_fwd_raster(vsa_plan_t plan, const void* q, const void* k,
                                            const void* v, const int32_t* row_ptr,
                                            const int32_t* col_idx, int32_t uniform_k,
                                            int64_t nnz, const void* gate,
                                            const float* o_coarse, void* o_raster, float* lse,
                                            void* stream);

/* Balanced launches of the two attention forwards above: the same operation
 * and the same arguments, plus a device workspace.  Instead of a fixed row
 * per workgroup, each workgroup of a launch with a quarter more workgroups
 * than rows takes the next row from one of 8 row queues (one per XCD, each a
 * contiguous range of rows, i.e. whole heads): its own XCD's queue, or once
 * that is empty the others', and the workgroups left over when every row is
 * taken exit at once.  XCDs that run faster thus finish more rows and the
 * kernel does not wait for the slowest one.  Within a head the queue hands
 * out the query blocks in cost order: blocks the grid edge does not cut
 * first, then the edge blocks by descending valid-token count, so the
 * workgroups running together cost about the same (they share key blocks in
 * L2) and the cheap rows come last; a block map's rows are handed out long
 * rows first, then head by head by entry count.
 * Tail split: when no queue holds more than 256 rows (a launch of a few
 * rounds of rows per CU, such as one GPU's share of a head-sharded layer),
 * the last min(16, rows of the queue) rows of each queue are handed out as
 * two halves, the first and the second half of the row's entries, each
 * computed by its own workgroup; each half leaves its unnormalised output,
 * running max and sum in the workspace and the half that finishes second
 * merges the two (the softmax merge of two key sets) and writes the row.
 * Rows handed out whole are bit-identical to the unbalanced launch; split
 * rows sum in another order and agree with it to within the last bit of the
 * element type, independently of which half finishes last.
 * The queue and split counters live in the workspace and are cleared by a
 * kernel on `stream` before the attention kernel, so the workspace needs no
 * initialisation; it must not be used by another call while this one runs
 * (concurrent calls need their own workspaces).
 * vsa_attn_fwd_workspace_size writes the bytes needed: 256 bytes of queue
 *   counters, 4 bytes per row (the claim order of a block map), and the
 *   split region (8 bytes per split slot plus two halves of waves x 16.5 KB,
 *   at most 128 slots: 34.6 MB for 256-token blocks), each 256-byte aligned.
 * ws: device memory, 256-byte aligned, ws_bytes at least that size; owned by
 *   the caller.
 * Errors: as the unbalanced entry points, plus INVALID_ARGUMENT for a null,
 *   misaligned or too small workspace. */
vsa_status vsa_attn_fwd_workspace_size(vsa_plan_t plan, size_t* bytes);
vsa_status vsa_block_sparse_attn_fwd_ws(vsa_plan_t plan, const void* q_blk, const void* k_blk,
                                        const void* v_blk, const int32_t* row_ptr,
                                        const int32_t* col_idx, int32_t uniform_k, int64_t nnz,
                                        void* o_blk, float* lse, void* ws, size_t ws_bytes,
                                        void* stream);
vsa_status vsa_block_sparse_attn_fwd_raster_ws(vsa_plan_t plan, const void* q, const void* k,
                                               const void* v, const int32_t* row_ptr,
                                               const int32_t* col_idx, int32_t uniform_k,
                                               int64_t nnz, const void* gate,
                                               const float* o_coarse, void* o_raster, float* lse,
                                               void* ws, size_t ws_bytes, void* stream);

/* vsa_block_sparse_attn_fwd_ws without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The row-queue counters, the claim
 * order of a block map of at most 65536 rows and the tail-split region of at
 * most 128 slots live in a library-owned static device array of 34.9 MB per
 * GPU, which stays allocated until the process ends; the call itself
 * allocates nothing and clears the counters with a small kernel on `stream`
 * (no memset); its results equal vsa_block_sparse_attn_fwd_ws bit for bit.  Every
 * call on a GPU shares that GPU's array: calls that may overlap on one GPU
 * (other streams or threads without ordering between them) race and must be
 * serialised by the caller.  Arguments, outputs and errors as
 * vsa_block_sparse_attn_fwd_ws (minus the workspace), plus HIP if the
 * scratch address cannot be looked up on the current device. */
vsa_status vsa_block_sparse_attn_fwd_noalloc(vsa_plan_t plan, const void* q_blk,
                                             const void* k_blk, const void* v_blk,
                                             const int32_t* row_ptr, const int32_t* col_idx,
                                             int32_t uniform_k, int64_t nnz, void* o_blk,
                                             float* lse, void* stream);

/* Bytes of device workspace vsa_block_sparse_attn_bwd needs for this plan:
 * rowsum(dO*O) [B,NH,Npad] fp32, the transposed block map
 * (B*NH*nb*nb + B*NH*nb int32), the row-queue counters of its balanced
 * launches (rows and columns are claimed per XCD at run time, as in
 * vsa_block_sparse_attn_fwd_ws) and their tail-split region (at most 128
 * split rows or columns, each leaving two partial gradient sums of vol/32
 * waves x 32 KB; the gradients of a split row are the sum of its halves,
 * added in an order-independent way), each 256-byte aligned. */
vsa_status vsa_block_sparse_attn_bwd_workspace_size(vsa_plan_t plan, size_t* bytes);

/* Gradients of vsa_block_sparse_attn_fwd (h3-perf-stack log, sm_100a route
 * entry: the route's fallback kernels keep the entire gradient path).  With
 * the forward's LSE the probabilities are recomputed exactly:
 *   P = exp(q.k/sqrt(D) - LSE_q), D_q = sum_d dO_q*O_q, dS = P (dO V^T - D_q),
 *   dQ = dS K / sqrt(D),  dK_j += dS^T Q / sqrt(D),  dV_j += P^T dO
 * over the valid tokens of the blocks of each row; a block listed m times in
 * a row counts m times, as in the forward.  Products and softmax in fp32, P
 * and dS rounded to elem for the matrix products, gradients rounded to elem.
 * q_blk, k_blk, o_blk, do_blk: device elem blocked layout (do_blk is the
 *   output gradient gathered like Q).  v_blk: device elem blocked layout --
 *   token-major, i.e. V gathered with role Q or K, NOT the V^T layout.
 * lse: device fp32 [B,NH,Npad], as written by the forward on the same map.
 * row_ptr, col_idx, uniform_k, nnz: the forward's map, same rules.
 * dq_blk, dk_blk, dv_blk: device elem blocked layout; pad rows are written 0.
 * workspace: device buffer of vsa_block_sparse_attn_bwd_workspace_size bytes,
 *   256-byte aligned, not shared with a concurrently running call.
 * Errors: INVALID_ARGUMENT for null pointers, nnz < 0, uniform_k outside
 *   [0, nb], a short or misaligned workspace; UNSUPPORTED for nb > 4096. */
vsa_status vsa_block_sparse_attn_bwd(vsa_plan_t plan, const void* q_blk, const void* k_blk,
                                     const void* v_blk, const void* o_blk, const void* do_blk,
                                     const float* lse, const int32_t* row_ptr,
                                     const int32_t* col_idx, int32_t uniform_k, int64_t nnz,
                                     void* dq_blk, void* dk_blk, void* dv_blk, void* workspace,
                                     size_t workspace_bytes, void* stream);

/* Bytes of device workspace vsa_forward needs for this plan (blocked Q, K,
 * V, O, pooled Q, K and V, the coarse output, the selected block ids, and the
 * row queues and tail-split region of the balanced attention launch, each
 * 256-byte aligned). */
vsa_status vsa_forward_workspace_size(vsa_plan_t plan, size_t* bytes);

/* The whole hot path for a plan with topk >= 1, raster in and raster out:
 * gather Q, K (with pooling) and V; score and top-k; block-sparse attention;
 * scatter O.  The attention step is the balanced launch of
 * vsa_block_sparse_attn_fwd_ws.  q, k, v: device elem raster.  out: device
 * elem raster.
 * gate: device elem raster [B,S,NH,D] or NULL.  NULL runs the sparse branch
 * alone (the guide's "Checkpoint behavior": without to_gate_compress
 * weights there is no compensation); otherwise V is pooled too, the coarse
 * branch runs (vsa_compress_attn) and the output is written as by
 * vsa_scatter_gated.
 * workspace: device buffer of at least vsa_forward_workspace_size bytes,
 * 256-byte aligned, not shared with a concurrently running call.
 * col_idx_out: optional device int32 copy target for the selected ids
 * (B*NH*nb*topk) or NULL.  lse: optional device fp32 [B,NH,Npad] or NULL.
 * Errors: INVALID_ARGUMENT for null pointers or a map-mode plan (topk == 0). */
vsa_status vsa_forward(vsa_plan_t plan, const void* q, const void* k, const void* v,
                       const void* gate, void* out, void* workspace, size_t workspace_bytes,
                       int32_t* col_idx_out, float* lse, void* stream);

/* Bytes of device workspace vsa_forward_fused needs for this plan (pooled Q,
 * K and V, the coarse output, the selected block ids and the attention row
 * queues and tail-split region, each 256-byte aligned; no blocked copies of
 * the tensors). */
vsa_status vsa_forward_fused_workspace_size(vsa_plan_t plan, size_t* bytes);

/* The whole hot path without the gather and scatter passes: the block means
 * of Q and K are read from the raster tensors (vsa_gather with x_blk NULL),
 * score and top-k select the blocks, and vsa_block_sparse_attn_fwd_raster_ws
 * attends and writes the raster output.  With `gate` the means of V and the
 * coarse branch are computed first and the attention epilogue writes
 * O + gate * o_coarse[block] as vsa_scatter_gated does.  Arguments, outputs
 * and errors as for vsa_forward, with the workspace sized by
 * vsa_forward_fused_workspace_size; plus UNSUPPORTED where the raster
 * attention is. */
vsa_status vsa_forward_fused(vsa_plan_t plan, const void* q, const void* k, const void* v,
                             const void* gate, void* out, void* workspace,
                             size_t workspace_bytes, int32_t* col_idx_out, float* lse,
                             void* stream);

/* ---- Measurement kernels: the roofline denominators of the kernels above,
 * measured on the machine that runs them (dense bf16 matrix-core rate and
 * engine clock, plain copy bandwidth).  They compute nothing of the method.
 *
 * vsa_bench_mfma_peak: launches num_workgroups workgroups of 4 waves; every
 * wave issues iters * 16 v_mfma_f32_32x32x16_bf16 (32768 flops each) on four
 * independent accumulators and records, in lane 0, timing[4w + 0] = shader
 * clock cycles and timing[4w + 1] = constant-rate wall-clock ticks spent in
 * its loop (timing[4w + 2] holds a checksum of the products, [4w + 3] = 0);
 * w = workgroup * 4 + wave.  timing: device, 16*num_workgroups uint64,
 * 8-byte aligned.  *wall_clock_hz (host) receives the wall clock's rate, so
 * cycles / (ticks / rate) is the engine clock the loop ran at.  Flops / the
 * kernel's duration is the sustained dense bf16 rate.
 * Errors: INVALID_ARGUMENT for null pointers, num_workgroups outside
 *   [1, 2^20], iters < 1 or a misaligned timing buffer; HIP for a failed
 *   device query or launch. */
vsa_status vsa_bench_mfma_peak(int32_t num_workgroups, int32_t iters, uint64_t* timing,
                               int64_t* wall_clock_hz, void* stream);

/* vsa_bench_hbm_copy: dst[0 .. bytes) = src[0 .. bytes) with 16-byte loads
 * and stores (bytes read + bytes written = 2 * bytes of HBM traffic when the
 * buffers exceed the caches).  src, dst: device, 16-byte aligned, not
 * overlapping.  Errors: INVALID_ARGUMENT for null or misaligned buffers or
 * bytes not a positive multiple of 16; HIP for a failed launch. */
vsa_status vsa_bench_hbm_copy(const void* src, void* dst, int64_t bytes, void* stream);

/* Static description of a status code. */
const char* vsa_status_string(vsa_status status);

/* Reason for the most recent failure on the calling thread ("" if none). */
const char* vsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* VSA_H_ */
