"""CPU oracle for the Video Sparse Attention (VSA) hot path -- TEST INFRASTRUCTURE.

This module is test infrastructure, not product code.  Only the test suite,
the package's smoke check and the benchmark's CPU-baseline leg may import or
run it.  It shares no code with the HIP path (no kernels, headers, tables or
helpers) and imports nothing from it.

It is a plain, slow, obviously correct float64 implementation of what the hot
path computes, written from the pages:

* "FastVideo VSA" (vllm-omni user guide), intro: the post-patch latent grid is
  partitioned into spatiotemporal blocks; for every query block the key/value
  blocks are scored and attention is computed only against the selected
  top-k blocks.
* same guide, "Choose top-k": the routing log line (seq_len, dit_seq_shape,
  block_size, num_blocks, topk, keep_ratio); top-k counts key/value blocks
  kept per query block; topk > num_blocks is invalid.
* same guide, "Enable the backend": top-k must be positive.
* same guide, intro and "Verify routing and fallback": non-causal
  self-attention, equal Q/KV lengths, standard head_size**-0.5 scaling, equal
  Q/K/V head counts, no mask, 256-token blocks.
* FastVideo h3-perf-stack commit log, sm_100a tile-64 route entry: a boolean
  block map compacted into per-row index lists with NON-uniform per-row counts
  and zero-count rows; text-prefix query tiles dense, video tiles prefix +
  top-k.
* same log, FastH3 example entry: the gate-compress branch pools per tile
  (the block score uses per-block pooled queries and keys).
* same guide, "Checkpoint behavior": checkpoints with learned
  to_gate_compress weights use that projection to compensate the sparse
  branch; without them VSA runs the sparse branch alone.

Readings where the pages are silent (each also listed with the design notes):
  R1 tokens are in raster order s = (t*H + h)*W + w;
  R2 blocks are numbered raster-wise over the block grid, t-major;
  R3 a block's pooled vector is the mean over its VALID tokens (edge blocks
     divide by their own token count, not by the full block volume);
  R4 the block score is the raw dot product of pooled query and pooled key
     (no scale, no softmax -- both are monotone per row);
  R5 ties in the top-k go to the lower block index; the ranking uses the
     float64 scores as computed here (no rounding to a device precision:
     rows whose k-th and (k+1)-th scores lie within the stated 1e-3 margin
     are near-ties, where a lower-precision implementation may differ);
  R6 a selected row is reported sorted ascending by block index;
  R7 no block is forced into its own row (pure top-k);
  R8 an empty row gives O = 0 and LSE = -inf;
  R9 padded tokens of edge blocks take no part in any softmax (masked);
  R15 the gate-compress (coarse) branch is attention among the per-tile pooled
     tokens: block i's pooled query attends over every block's pooled key
     with the standard head_size**-0.5 scale (its logits are the R4 block
     scores, scaled) and returns the softmax-weighted mean of the pooled
     values -- the pages give no formula, this is the plainest reading;
  R16 the gated output is the sparse output plus the gate times the coarse
     output of the token's block, elementwise; the gate is a tensor shaped
     like Q (the projection's output, supplied by the caller); no gate means
     the sparse output alone.

Precision: every function computes in float64 except the two *_f32 ones,
which take the same steps in float32 torch-CPU ops.  They exist for the
layer-sized shapes (the timed CPU baseline, and checking every output row of
a full layer), where the float64 loop is too slow; they are pinned to the
float64 functions and to the brute-force formulation on small shapes.

Parity pins for every function live in tests/test_oracle_pins.py.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "Plan", "make_plan", "routing_line", "token_block_ids", "block_token_lists",
    "pool_blocks", "block_scores", "select_topk", "selection_to_csr",
    "map_to_csr", "block_sparse_attention", "vsa_reference", "valid_flops",
    "compress_attention", "gated_combine", "vsa_gated_reference",
    "block_sparse_attention_bwd", "block_sparse_attention_f32", "vsa_reference_f32",
]


class Plan:
    """Partition of a (T, H, W) latent grid into (bt, bh, bw) blocks.

    "FastVideo VSA" guide, intro and "Choose top-k": num_blocks is the number
    of spatiotemporal blocks the post-patch latent grid is cut into; edge
    blocks are partial (readings R1, R2).
    """

    def __init__(self, seq_len, dit_seq_shape, block_size, topk=None):
        t, h, w = (int(x) for x in dit_seq_shape)
        bt, bh, bw = (int(x) for x in block_size)
        if min(t, h, w, bt, bh, bw) < 1:
            raise ValueError("grid and block sizes must be positive")
        if int(seq_len) != t * h * w:
            raise ValueError(f"seq_len {seq_len} != T*H*W = {t * h * w}")
        self.seq_len = int(seq_len)
        self.dit_seq_shape = (t, h, w)
        self.block_size = (bt, bh, bw)
        self.block_grid = (math.ceil(t / bt), math.ceil(h / bh), math.ceil(w / bw))
        nt, nh, nw = self.block_grid
        self.num_blocks = nt * nh * nw
        self.block_volume = bt * bh * bw
        if topk is not None:
            topk = int(topk)
            # "Enable the backend": top-k must be positive.
            # "Choose top-k": topk > num_blocks is invalid for the shape.
            if topk < 1 or topk > self.num_blocks:
                raise ValueError(f"topk {topk} outside [1, {self.num_blocks}]")
        self.topk = topk

    def block_extent(self, beta):
        """(origin, size) of block ``beta`` along t, h, w (sizes clipped at the grid edge)."""
        nt, nh, nw = self.block_grid
        it, rem = divmod(int(beta), nh * nw)
        ih, iw = divmod(rem, nw)
        org = (it * self.block_size[0], ih * self.block_size[1], iw * self.block_size[2])
        size = tuple(min(b, g - o) for b, g, o in zip(self.block_size, self.dit_seq_shape, org))
        return org, size

    def block_counts(self):
        """Valid-token count of every block, in block-id order."""
        return np.array([int(np.prod(self.block_extent(b)[1])) for b in range(self.num_blocks)],
                        dtype=np.int64)

    def keep_ratio(self):
        return None if self.topk is None else self.topk / self.num_blocks


def make_plan(seq_len, dit_seq_shape, block_size, topk=None) -> Plan:
    return Plan(seq_len, dit_seq_shape, block_size, topk)


def routing_line(plan: Plan) -> str:
    """The fields of the routing log line ("FastVideo VSA" guide, "Choose top-k").

    keep_ratio is topk / num_blocks as a percentage with one decimal.  The route
    is VSA for a sparse selection and VSA_ALL_BLOCKS when every block is kept
    (the all-block path of "Choose top-k"; this path always runs the sparse
    computation, it never switches to dense SDPA).
    """
    t, h, w = plan.dit_seq_shape
    bt, bh, bw = plan.block_size
    parts = [f"seq_len={plan.seq_len}", f"dit_seq_shape=({t}, {h}, {w})",
             f"block_size=({bt}, {bh}, {bw})", f"num_blocks={plan.num_blocks}"]
    if plan.topk is not None:
        parts.append(f"topk={plan.topk}")
        parts.append(f"keep_ratio={100.0 * plan.topk / plan.num_blocks:.1f}%")
        parts.append("route=" + ("VSA_ALL_BLOCKS" if plan.topk == plan.num_blocks else "VSA"))
    return ", ".join(parts)


def token_block_ids(plan: Plan) -> np.ndarray:
    """Block id of every token s (readings R1, R2)."""
    t, h, w = plan.dit_seq_shape
    bt, bh, bw = plan.block_size
    nt, nh, nw = plan.block_grid
    tt, hh, ww = np.meshgrid(np.arange(t), np.arange(h), np.arange(w), indexing="ij")
    beta = ((tt // bt) * nh + (hh // bh)) * nw + (ww // bw)
    return beta.reshape(-1)


def block_token_lists(plan: Plan):
    """For every block, the token indices it holds, ascending (raster order)."""
    beta = token_block_ids(plan)
    order = np.argsort(beta, kind="stable")
    bounds = np.searchsorted(beta[order], np.arange(plan.num_blocks + 1))
    return [order[bounds[b]:bounds[b + 1]] for b in range(plan.num_blocks)]


def pool_blocks(x, plan: Plan) -> np.ndarray:
    """Per-(batch, head, block) mean of x over the block's valid tokens (R3).

    x: [B, S, heads, D] (any float dtype; upcast to float64).
    Returns [B, heads, num_blocks, D] float64.
    """
    x = np.asarray(x, dtype=np.float64)
    lists = block_token_lists(plan)
    out = np.empty((x.shape[0], x.shape[2], plan.num_blocks, x.shape[3]))
    for b_id, toks in enumerate(lists):
        out[:, :, b_id, :] = x[:, toks, :, :].mean(axis=1)
    return out


def block_scores(qbar, kbar) -> np.ndarray:
    """Coarse block score sigma[i, j] = qbar_i . kbar_j per (batch, head) (R4).

    "FastVideo VSA" guide, intro: for every query block VSA scores the
    key/value blocks.  qbar, kbar: [B, heads, nb, D] -> [B, heads, nb, nb].
    """
    return np.matmul(np.asarray(qbar, np.float64), np.swapaxes(np.asarray(kbar, np.float64), -1, -2))


def select_topk(scores, k):
    """Per-row top-k of the block scores ("FastVideo VSA" guide, intro and "Choose top-k").

    Keeps the k highest-scoring key blocks of each query-block row, ranking
    the float64 scores with ties to the lower block index (R5): the key is
    (-score, block index), ascending.  Each row is returned sorted ascending
    (R6).

    Returns (sel int64 [..., nb, k], margin float64 [..., nb]) where margin is
    the gap between the k-th and (k+1)-th largest scores of the row (+inf
    when k == nb): rows with a small margin are near-ties.
    """
    s64 = np.asarray(scores, np.float64)
    nb = s64.shape[-1]
    if not 1 <= k <= nb:
        raise ValueError(f"topk {k} outside [1, {nb}]")
    rows = s64.reshape(-1, nb)
    sel = np.empty((rows.shape[0], k), dtype=np.int64)
    margin = np.empty(rows.shape[0])
    idx = np.arange(nb)
    for r in range(rows.shape[0]):
        # primary key: score descending; secondary key: block index ascending
        order = np.lexsort((idx, -rows[r]))
        sel[r] = np.sort(order[:k])
        desc = rows[r][order]
        margin[r] = math.inf if k == nb else desc[k - 1] - desc[k]
    return sel.reshape(*s64.shape[:-1], k), margin.reshape(s64.shape[:-1])


def selection_to_csr(sel):
    """Uniform selection [B, heads, nb, k] -> CSR (row_ptr, col_idx), rows (b, h, i)."""
    sel = np.asarray(sel)
    k = sel.shape[-1]
    rows = int(np.prod(sel.shape[:-1]))
    row_ptr = np.arange(rows + 1, dtype=np.int64) * k
    return row_ptr, sel.reshape(-1).astype(np.int64)


def map_to_csr(block_map):
    """Compact a boolean block map [..., nq, nk] into CSR lists.

    FastVideo h3-perf-stack commit log, sm_100a tile-64 route entry: the
    boolean map is compacted into per-row index lists whose counts may differ
    from row to row and may be zero.  Rows are the flattened leading indices.
    """
    m = np.asarray(block_map, dtype=bool)
    flat = m.reshape(-1, m.shape[-1])
    counts = flat.sum(axis=1)
    row_ptr = np.zeros(flat.shape[0] + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    col_idx = np.nonzero(flat)[1].astype(np.int64)
    return row_ptr, col_idx


def block_sparse_attention(q, k, v, plan: Plan, row_ptr, col_idx, query_rows=None):
    """Exact softmax attention of each query over the tokens of its row's blocks.

    "FastVideo VSA" guide, intro: attention is computed only against the
    selected blocks; "Verify routing and fallback": non-causal, scale
    head_size**-0.5, equal head counts, no mask.  Padded positions do not exist
    here: each block contributes only its valid tokens (R9).  Empty rows give
    O = 0, LSE = -inf (R8).

    q, k, v: [B, S, heads, D].  row_ptr/col_idx: CSR over rows (b, h, i).
    query_rows: optional iterable of row ids (b*heads + h)*nb + i to compute;
    other rows are left as NaN (for sampled checks of large shapes).
    Returns (O [B, S, heads, D] float64, LSE [B, S, heads] float64, natural log).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    bsz, s, nh, d = q.shape
    nb = plan.num_blocks
    lists = block_token_lists(plan)
    scale = 1.0 / math.sqrt(d)
    full = query_rows is None
    out = np.zeros_like(q) if full else np.full_like(q, np.nan)
    lse = np.full((bsz, s, nh), -np.inf) if full else np.full((bsz, s, nh), np.nan)
    rows = range(bsz * nh * nb) if full else query_rows
    for r in rows:
        b, rem = divmod(int(r), nh * nb)
        h, i = divmod(rem, nb)
        qtok = lists[i]
        cols = col_idx[row_ptr[r]:row_ptr[r + 1]]
        if len(cols) == 0:
            out[b, qtok, h, :] = 0.0
            lse[b, qtok, h] = -np.inf
            continue
        ktok = np.concatenate([lists[j] for j in cols])
        logits = (q[b, qtok, h, :] @ k[b, ktok, h, :].T) * scale
        mx = logits.max(axis=1, keepdims=True)
        p = np.exp(logits - mx)
        denom = p.sum(axis=1, keepdims=True)
        out[b, qtok, h, :] = (p @ v[b, ktok, h, :]) / denom
        lse[b, qtok, h] = (mx + np.log(denom))[:, 0]
    return out, lse


def vsa_reference(q, k, v, dit_seq_shape, block_size, topk):
    """Whole hot path: plan -> pool -> score -> top-k -> attention.

    Returns a dict with the plan, pooled means, scores, selection, margins,
    CSR, and the attention output / LSE.
    """
    s = q.shape[1]
    plan = make_plan(s, dit_seq_shape, block_size, topk)
    qbar = pool_blocks(q, plan)
    kbar = pool_blocks(k, plan)
    sc = block_scores(qbar, kbar)
    sel, margin = select_topk(sc, topk)
    row_ptr, col_idx = selection_to_csr(sel)
    o, lse = block_sparse_attention(q, k, v, plan, row_ptr, col_idx)
    return dict(plan=plan, qbar=qbar, kbar=kbar, scores=sc, sel=sel, margin=margin,
                row_ptr=row_ptr, col_idx=col_idx, out=o, lse=lse)


def compress_attention(qbar, kbar, vbar, head_dim):
    """Gate-compress (coarse) branch: attention among the per-tile pooled tokens (R15).

    h3-perf-stack log, FastH3 example entry: the gate-compress branch pools
    per tile.  For every (batch, head), block i's pooled query attends over
    the pooled keys of all blocks with the standard head_size**-0.5 scale
    ("Verify routing and fallback") and takes the softmax-weighted mean of
    the pooled values.  qbar, kbar, vbar: [B, heads, nb, D] ->
    [B, heads, nb, D] float64.
    """
    logits = block_scores(qbar, kbar) / math.sqrt(head_dim)
    mx = logits.max(axis=-1, keepdims=True)
    p = np.exp(logits - mx)
    return np.matmul(p, np.asarray(vbar, np.float64)) / p.sum(axis=-1, keepdims=True)


def gated_combine(o_sparse, o_coarse, gate, plan: Plan):
    """Sparse output plus the gated coarse output of each token's block (R16).

    "FastVideo VSA" guide, "Checkpoint behavior": a learned to_gate_compress
    projection compensates the sparse branch; without it the sparse branch is
    used alone (gate None).  out[b, s, h] = o_sparse[b, s, h] +
    gate[b, s, h] * o_coarse[b, h, block(s)], all [.., D] elementwise.
    o_sparse, gate: [B, S, heads, D]; o_coarse: [B, heads, nb, D].
    """
    o_sparse = np.asarray(o_sparse, np.float64)
    if gate is None:
        return o_sparse
    beta = token_block_ids(plan)
    per_token = np.asarray(o_coarse, np.float64)[:, :, beta, :]      # [B, heads, S, D]
    return o_sparse + np.asarray(gate, np.float64) * np.swapaxes(per_token, 1, 2)


def vsa_gated_reference(q, k, v, gate, dit_seq_shape, block_size, topk):
    """Whole path with the gate-compress branch: vsa_reference, pooled values,
    the coarse attention and the gated combination (R15, R16)."""
    ref = vsa_reference(q, k, v, dit_seq_shape, block_size, topk)
    vbar = pool_blocks(v, ref["plan"])
    oc = compress_attention(ref["qbar"], ref["kbar"], vbar, np.asarray(q).shape[-1])
    ref.update(vbar=vbar, o_coarse=oc, gated_out=gated_combine(ref["out"], oc, gate, ref["plan"]))
    return ref


def block_sparse_attention_bwd(q, k, v, do, plan: Plan, row_ptr, col_idx):
    """Gradients of block_sparse_attention with respect to q, k and v.

    h3-perf-stack log, sm_100a route entry: the forward-only route falls back
    to the Triton tile-64 kernels, which keep the entire gradient path; this
    is that gradient.  The forward is, per query token,
    O = softmax(l) V over the valid tokens of the row's blocks with
    l = q K^T / sqrt(D); its exact gradients (the softmax Jacobian written
    out) are, with P the softmax probabilities and dO the output gradient:
      dV_j += P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(dO * O)),
      dQ = dS K / sqrt(D),  dK_j += dS^T Q / sqrt(D),
    summed over every row that selected block j (a block listed twice in a
    row counts twice, as in the forward).  Empty rows contribute nothing.
    q, k, v, do: [B, S, heads, D].  Returns (dq, dk, dv) float64, same shape.
    """
    q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
    bsz, s, nh, d = q.shape
    nb = plan.num_blocks
    lists = block_token_lists(plan)
    scale = 1.0 / math.sqrt(d)
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for r in range(bsz * nh * nb):
        b, rem = divmod(r, nh * nb)
        h, i = divmod(rem, nb)
        cols = col_idx[row_ptr[r]:row_ptr[r + 1]]
        if len(cols) == 0:
            continue
        qtok = lists[i]
        ktok = np.concatenate([lists[j] for j in cols])
        qi, kj, vj, doi = q[b, qtok, h], k[b, ktok, h], v[b, ktok, h], do[b, qtok, h]
        logits = (qi @ kj.T) * scale
        p = np.exp(logits - logits.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        o = p @ vj
        dp = doi @ vj.T
        ds = p * (dp - (doi * o).sum(axis=1, keepdims=True))
        dq[b, qtok, h] += (ds @ kj) * scale
        # keys may repeat within a row: accumulate per occurrence
        np.add.at(dk[:, :, h], (b, ktok), (ds.T @ qi) * scale)
        np.add.at(dv[:, :, h], (b, ktok), p.T @ doi)
    return dq, dk, dv


def valid_flops(plan: Plan, row_ptr, col_idx, head_dim) -> int:
    """Multiply-add work of the attention counted on valid tokens only.

    For every row (query block i) and every selected block j: 2*D flops for
    q.k and 2*D for p*v per (valid query, valid key) pair.
    """
    c = plan.block_counts()
    nb = plan.num_blocks
    row_ptr = np.asarray(row_ptr, np.int64)
    col_idx = np.asarray(col_idx, np.int64)
    rows = len(row_ptr) - 1
    keys_per_row = np.add.reduceat(np.append(c[col_idx], 0), row_ptr[:-1]) if len(col_idx) else np.zeros(rows, np.int64)
    keys_per_row = np.where(np.diff(row_ptr) > 0, keys_per_row, 0)
    q_counts = np.tile(c, rows // nb)
    return int(4 * head_dim * np.sum(q_counts * keys_per_row))


def block_sparse_attention_f32(q, k, v, plan: Plan, row_ptr, col_idx, heads=None):
    """block_sparse_attention in float32 torch-CPU ops (same steps, row by row).

    For every row (batch b, head h, query block i): the logits of the block's
    valid queries against the concatenated valid keys of the row's blocks,
    scaled by head_size**-0.5, a max-subtracted softmax, and the product with
    the same keys' values ("FastVideo VSA" guide, intro and "Verify routing
    and fallback").  Empty rows give O = 0 and LSE = -inf (R8).

    q, k, v: [B, S, heads, D] torch tensors or arrays (cast to float32).
    heads: optional iterable of head indices to compute (every batch); the
    other heads' outputs are NaN.  Returns (O [B, S, heads, D],
    LSE [B, S, heads]) as float32 torch tensors; LSE is the natural log.
    """
    import torch
    q, k, v = (torch.as_tensor(x).to(torch.float32) for x in (q, k, v))
    bsz, s, nh, d = q.shape
    nb = plan.num_blocks
    lists = [torch.as_tensor(t, dtype=torch.long) for t in block_token_lists(plan)]
    row_ptr = np.asarray(row_ptr, np.int64)
    col_idx = np.asarray(col_idx, np.int64)
    scale = 1.0 / math.sqrt(d)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((bsz, s, nh), float("nan"))
    for b in range(bsz):
        for h in (range(nh) if heads is None else heads):
            qh, kh, vh = q[b, :, h].contiguous(), k[b, :, h].contiguous(), v[b, :, h].contiguous()
            for i in range(nb):
                r = (b * nh + h) * nb + i
                qtok = lists[i]
                cols = col_idx[row_ptr[r]:row_ptr[r + 1]]
                if len(cols) == 0:
                    out[b, qtok, h] = 0.0
                    lse[b, qtok, h] = float("-inf")
                    continue
                ktok = torch.cat([lists[j] for j in cols])
                logits = (qh[qtok] @ kh[ktok].T) * scale
                mx = logits.amax(dim=1, keepdim=True)
                p = torch.exp(logits - mx)
                denom = p.sum(dim=1, keepdim=True)
                out[b, qtok, h] = (p @ vh[ktok]) / denom
                lse[b, qtok, h] = (mx + torch.log(denom))[:, 0]
    return out, lse


def vsa_reference_f32(q, k, v, dit_seq_shape, block_size, topk, heads=None):
    """Whole hot path in float32 torch-CPU ops: plan, pool, score, top-k, attention.

    Same steps as vsa_reference: block means over valid tokens (R3), raw dot
    product scores (R4), per-row top-k on the float32 scores with ties to the
    lower block index (a stable sort of the negated scores, R5), rows sorted
    ascending (R6), then block_sparse_attention_f32.  heads: optional subset
    of heads to attend (pooling, scoring and selection cover every head).
    Returns a dict with the plan, the selection, the CSR and O / LSE.
    """
    import torch
    q, k, v = (torch.as_tensor(x).to(torch.float32) for x in (q, k, v))
    plan = make_plan(q.shape[1], dit_seq_shape, block_size, topk)
    beta = torch.as_tensor(token_block_ids(plan), dtype=torch.long)
    counts = torch.as_tensor(plan.block_counts(), dtype=torch.float32)

    def pool(x):
        sums = torch.zeros(x.shape[0], plan.num_blocks, x.shape[2], x.shape[3])
        sums.index_add_(1, beta, x)
        return (sums / counts[None, :, None, None]).permute(0, 2, 1, 3)   # [B, heads, nb, D]

    scores = pool(q) @ pool(k).transpose(-1, -2)
    order = torch.sort(-scores, dim=-1, stable=True).indices[..., :topk]
    sel = torch.sort(order, dim=-1).values.numpy().astype(np.int64)
    row_ptr, col_idx = selection_to_csr(sel)
    o, lse = block_sparse_attention_f32(q, k, v, plan, row_ptr, col_idx, heads=heads)
    return dict(plan=plan, scores=scores, sel=sel, row_ptr=row_ptr, col_idx=col_idx, out=o,
                lse=lse)
