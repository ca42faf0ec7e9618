"""Pins for the CPU oracle against what the pages and the mathematics fix.

None of these re-types the oracle's own formula: each checks a value the pages
print, a hand-derived closed form, an invariant, a brute-force formulation of
a different shape (a dense S x S softmax with a keep-mask), or a library
routine for a special case (torch's fp64 scaled-dot-product attention).
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from vsa_inputs import WORKLOADS, make_planted_block_means, make_qkv, make_tile64_map, bf16_to_f64


def _golden_fields(path):
    out = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split("=", 1)
            out[key] = val
    return out


def _line_fields(line):
    # split "k=v, k=(a, b, c), ..." on the commas that start a new key
    fields, cur = [], ""
    depth = 0
    for ch in line:
        if ch == "(":
            depth += 1
        elif ch == ")":
            depth -= 1
        if ch == "," and depth == 0:
            fields.append(cur.strip())
            cur = ""
        else:
            cur += ch
    fields.append(cur.strip())
    return dict(f.split("=", 1) for f in fields)


# ---------------------------------------------------------------- a1: plan

def test_routing_line_matches_page_worked_example(golden_dir):
    page = _golden_fields(os.path.join(golden_dir, "routing_line.txt"))
    plan = oracle.make_plan(27280, (31, 22, 40), (4, 8, 8), 64)
    ours = _line_fields(oracle.routing_line(plan))
    shared = [k for k in page if k != "checkpoint_mode"]
    assert set(shared) <= set(ours)
    for k in shared:
        assert ours[k] == page[k], k


@pytest.mark.parametrize("shape,block,nb", [
    ((8, 16, 16), (4, 8, 8), 8),          # 2*2*2
    ((31, 22, 40), (4, 8, 8), 120),       # 8*3*5
    ((81, 30, 52), (4, 8, 8), 588),       # 21*4*7
    ((1, 1, 33280), (1, 1, 64), 520),     # 33280/64
    ((7, 13, 10), (4, 8, 8), 8),          # 2*2*2
    ((1, 1, 640), (1, 1, 64), 10),
])
def test_num_blocks_closed_form(shape, block, nb):
    plan = oracle.make_plan(int(np.prod(shape)), shape, block)
    assert plan.num_blocks == nb
    assert int(plan.block_counts().sum()) == plan.seq_len


@pytest.mark.parametrize("shape,hist", [
    # hand-derived: t extents {4 x7, 3 x1}, h {8, 8, 6}, w {8 x5}
    ((31, 22, 40), {256: 70, 192: 45, 144: 5}),
    # t {4 x20, 1 x1}, h {8 x3, 6}, w {8 x6, 4}
    ((81, 30, 52), {256: 360, 192: 120, 128: 60, 96: 20, 64: 18, 48: 6, 32: 3, 24: 1}),
])
def test_block_count_histograms(shape, hist):
    plan = oracle.make_plan(int(np.prod(shape)), shape, (4, 8, 8))
    vals, cnts = np.unique(plan.block_counts(), return_counts=True)
    assert dict(zip(vals.tolist(), cnts.tolist())) == hist


def test_padded_tiny_counts_in_block_order():
    # (7,13,10) / (4,8,8): t extents (4,3), h (8,5), w (8,2); ids t-major
    plan = oracle.make_plan(910, (7, 13, 10), (4, 8, 8))
    assert plan.block_counts().tolist() == [256, 64, 160, 40, 192, 48, 120, 30]


@pytest.mark.parametrize("k,text", [(64, "53.3%"), (16, "13.3%"), (32, "26.7%"), (120, "100.0%")])
def test_keep_ratio_text(k, text):
    plan = oracle.make_plan(27280, (31, 22, 40), (4, 8, 8), k)
    assert _line_fields(oracle.routing_line(plan))["keep_ratio"] == text
    route = _line_fields(oracle.routing_line(plan))["route"]
    assert route == ("VSA_ALL_BLOCKS" if k == 120 else "VSA")


@pytest.mark.parametrize("seq,k", [(27280, 0), (27280, 121), (27281, 64), (27280, -3)])
def test_plan_rejects_invalid(seq, k):
    with pytest.raises(ValueError):
        oracle.make_plan(seq, (31, 22, 40), (4, 8, 8), k)


def test_token_partition_hand_points_and_invariants():
    plan = oracle.make_plan(910, (7, 13, 10), (4, 8, 8))
    beta = oracle.token_block_ids(plan)
    # hand-picked tokens: s = (t*13 + h)*10 + w
    assert beta[0] == 0                            # (0,0,0)
    assert beta[(0 * 13 + 0) * 10 + 8] == 1        # w=8 -> second w block
    assert beta[(0 * 13 + 8) * 10 + 0] == 2        # h=8 -> second h block
    assert beta[(4 * 13 + 0) * 10 + 0] == 4        # t=4 -> second t block
    assert beta[909] == 7                          # last token (6,12,9)
    # each block's tokens form one aligned box, and the boxes tile the grid
    lists = oracle.block_token_lists(plan)
    seen = np.zeros(910, bool)
    for b, toks in enumerate(lists):
        t, rem = np.divmod(toks, 130)
        h, w = np.divmod(rem, 10)
        box = (np.ptp(t) + 1) * (np.ptp(h) + 1) * (np.ptp(w) + 1)
        assert box == len(toks) == plan.block_counts()[b]
        assert t.min() % 4 == 0 and h.min() % 8 == 0 and w.min() % 8 == 0
        assert np.all(np.diff(toks) > 0)   # raster order inside the block
        assert not seen[toks].any()
        seen[toks] = True
    assert seen.all()


# ---------------------------------------------------------------- a3: pool

@pytest.mark.parametrize("shape", [(7, 13, 10), (8, 16, 16), (5, 9, 17)])
def test_pool_planted_means_exact(shape):
    x, mu = make_planted_block_means(11, 1, 2, shape, (4, 8, 8), 16)
    plan = oracle.make_plan(int(np.prod(shape)), shape, (4, 8, 8))
    got = oracle.pool_blocks(bf16_to_f64(x), plan)
    want = mu.reshape(1, 2, plan.num_blocks, 16).numpy().astype(np.float64)
    assert np.array_equal(got, want)   # edge blocks divide by their own count


def test_pool_shift_and_within_block_permutation():
    wl = WORKLOADS["padded_tiny"]
    q, _, _ = make_qkv(wl)
    x = bf16_to_f64(q)
    plan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size)
    base = oracle.pool_blocks(x, plan)
    np.testing.assert_allclose(oracle.pool_blocks(x + 3.25, plan), base + 3.25, atol=1e-12)
    perm = np.arange(wl.seq_len)
    for toks in oracle.block_token_lists(plan):
        perm[toks] = toks[::-1]
    np.testing.assert_allclose(oracle.pool_blocks(x[:, perm], plan), base, atol=1e-12)


# ---------------------------------------------------------------- a4: score

def test_score_planted_integer_products():
    shape = (7, 13, 10)
    xq, muq = make_planted_block_means(21, 1, 2, shape, (4, 8, 8), 32)
    xk, muk = make_planted_block_means(22, 1, 2, shape, (4, 8, 8), 32)
    plan = oracle.make_plan(910, shape, (4, 8, 8))
    sc = oracle.block_scores(oracle.pool_blocks(bf16_to_f64(xq), plan),
                             oracle.pool_blocks(bf16_to_f64(xk), plan))
    a = muq.reshape(1, 2, 8, 32)
    b = muk.reshape(1, 2, 8, 32)
    for h in range(2):
        for i in range(8):
            for j in range(8):
                want = int(sum(int(a[0, h, i, d]) * int(b[0, h, j, d]) for d in range(32)))
                assert sc[0, h, i, j] == want   # query rows, key columns (not transposed)


# ---------------------------------------------------------------- a5: top-k

def test_topk_hand_examples_with_ties():
    row = np.array([[3.0, 5.0, 5.0, 1.0, 5.0, 2.0]])
    sel, margin = oracle.select_topk(row, 2)
    assert sel.tolist() == [[1, 2]]           # three-way tie at 5: lowest two indices
    assert margin.tolist() == [0.0]
    sel, _ = oracle.select_topk(row, 4)
    assert sel.tolist() == [[0, 1, 2, 4]]
    sel, margin = oracle.select_topk(row, 1)
    assert sel.tolist() == [[1]]
    sel, margin = oracle.select_topk(np.array([[-1.0, -0.5, -2.0]]), 2)
    assert sel.tolist() == [[0, 1]] and margin.tolist() == [1.0]


def test_topk_all_blocks_and_invariants():
    rng = np.random.default_rng(5)
    sc = rng.standard_normal((2, 3, 17, 17))
    sel, margin = oracle.select_topk(sc, 17)
    assert np.all(sel == np.arange(17)) and np.all(np.isinf(margin))
    for k in (1, 5, 16):
        sel, margin = oracle.select_topk(sc, k)
        flat = sc.reshape(-1, 17)
        for r, srow in enumerate(sel.reshape(-1, k)):
            assert len(set(srow.tolist())) == k and np.all(np.diff(srow) > 0)
            unsel = np.setdiff1d(np.arange(17), srow)
            assert flat[r, srow].min() >= flat[r, unsel].max()
            assert margin.reshape(-1)[r] == pytest.approx(flat[r, srow].min() - flat[r, unsel].max())


def test_topk_planted_exact_ties_prefer_lower_index():
    # planted integer block means with deliberately repeated key means: equal
    # scores are exact, so the lower block index must win.
    shape = (8, 16, 16)
    xq, _ = make_planted_block_means(31, 1, 1, shape, (4, 8, 8), 8, lo=1, hi=2)
    xk, muk = make_planted_block_means(32, 1, 1, shape, (4, 8, 8), 8, lo=0, hi=1)
    plan = oracle.make_plan(2048, shape, (4, 8, 8))
    qbar = oracle.pool_blocks(bf16_to_f64(xq), plan)
    kbar = oracle.pool_blocks(bf16_to_f64(xk), plan)
    sc = oracle.block_scores(qbar, kbar)
    sel, _ = oracle.select_topk(sc, 3)
    for i in range(8):
        row = sc[0, 0, i]
        # hand rule: walk scores high to low, within equal scores low index first
        order = sorted(range(8), key=lambda j: (-row[j], j))[:3]
        assert sel[0, 0, i].tolist() == sorted(order)


def test_topk_ranks_full_precision_scores():
    # Two scores closer than one float32 ulp: rounded to float32 they would
    # tie and the lower index would win; the definition ranks the scores
    # themselves, so the larger one (the higher index here) is kept.
    a = 1.0
    b = 1.0 + 2.0 ** -30
    assert np.float32(a) == np.float32(b) and b > a
    sel, margin = oracle.select_topk(np.array([[a, b, 0.5]]), 1)
    assert sel.tolist() == [[1]] and margin.tolist() == [b - a]
    sel, _ = oracle.select_topk(np.array([[0.25, a, -3.0, b]]), 2)
    assert sel.tolist() == [[1, 3]]
    sel, _ = oracle.select_topk(np.array([[0.25, a, -3.0, b]]), 1)
    assert sel.tolist() == [[3]]


# ---------------------------------------------------------------- CSR compaction

def test_map_to_csr_hand_example():
    m = np.array([[1, 0, 1, 0],
                  [0, 0, 0, 0],
                  [1, 1, 1, 1]], dtype=bool)
    rp, ci = oracle.map_to_csr(m)
    assert rp.tolist() == [0, 2, 2, 6]
    assert ci.tolist() == [0, 2, 0, 1, 2, 3]


# ---------------------------------------------------------------- a6: attention

def _dense_masked(q, k, v, keep):
    """Brute force: full S x S softmax per (batch, head) with a token keep-mask."""
    b, s, h, d = q.shape
    out = np.zeros_like(q)
    lse = np.full((b, s, h), -np.inf)
    for bi in range(b):
        for hi in range(h):
            logits = q[bi, :, hi] @ k[bi, :, hi].T / math.sqrt(d)
            logits = np.where(keep[bi, hi], logits, -np.inf)
            for si in range(s):
                row = logits[si]
                if np.all(np.isinf(row)):
                    continue
                m = row.max()
                p = np.exp(row - m)
                out[bi, si, hi] = p @ v[bi, :, hi] / p.sum()
                lse[bi, si, hi] = m + math.log(p.sum())
    return out, lse


def _token_keep(plan, row_ptr, col_idx, b, h):
    beta = oracle.token_block_ids(plan)
    nb = plan.num_blocks
    keep = np.zeros((b, h, plan.seq_len, plan.seq_len), bool)
    for bi in range(b):
        for hi in range(h):
            bm = np.zeros((nb, nb), bool)
            for i in range(nb):
                r = (bi * h + hi) * nb + i
                bm[i, col_idx[row_ptr[r]:row_ptr[r + 1]]] = True
            keep[bi, hi] = bm[beta[:, None], beta[None, :]]
    return keep


@pytest.mark.parametrize("k", [1, 4, 8])
def test_attention_matches_dense_masked_bruteforce(k):
    wl = WORKLOADS["padded_tiny"]
    q, kk, v = (bf16_to_f64(t) for t in make_qkv(wl))
    ref = oracle.vsa_reference(q, kk, v, wl.dit_seq_shape, wl.block_size, k)
    keep = _token_keep(ref["plan"], ref["row_ptr"], ref["col_idx"], 1, 2)
    o, lse = _dense_masked(q, kk, v, keep)
    np.testing.assert_allclose(ref["out"], o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ref["lse"], lse, rtol=0, atol=1e-12)


def test_attention_csr_with_zero_rows_matches_bruteforce():
    wl = WORKLOADS["tile64_tiny"]
    q, kk, v = (bf16_to_f64(t) for t in make_qkv(wl))
    rp, ci, nt = make_tile64_map(wl)
    assert np.any(np.diff(rp) == 0)      # the map has empty rows
    plan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size)
    o, lse = oracle.block_sparse_attention(q, kk, v, plan, rp, ci)
    keep = _token_keep(plan, rp, ci, 1, 2)
    ob, lb = _dense_masked(q, kk, v, keep)
    np.testing.assert_allclose(o, ob, atol=1e-12)
    assert np.array_equal(np.isinf(lse), np.isinf(lb))
    np.testing.assert_allclose(lse[np.isfinite(lse)], lb[np.isfinite(lb)], atol=1e-12)
    # empty rows: O = 0, LSE = -inf
    nb = plan.num_blocks
    for r in np.nonzero(np.diff(rp) == 0)[0]:
        b, rem = divmod(int(r), 2 * nb)
        h, i = divmod(rem, nb)
        toks = oracle.block_token_lists(plan)[i]
        assert np.all(o[b, toks, h] == 0) and np.all(np.isneginf(lse[b, toks, h]))


@pytest.mark.parametrize("name", ["tiny", "padded_tiny"])
def test_all_blocks_equals_library_dense_attention(name):
    wl = WORKLOADS[name]
    q, kk, v = make_qkv(wl)
    nb = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size).num_blocks
    ref = oracle.vsa_reference(bf16_to_f64(q), bf16_to_f64(kk), bf16_to_f64(v),
                               wl.dit_seq_shape, wl.block_size, nb)
    tq, tk, tv = (t.to(torch.float64).permute(0, 2, 1, 3) for t in (q, kk, v))
    dense = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).permute(0, 2, 1, 3)
    np.testing.assert_allclose(ref["out"], dense.numpy(), atol=1e-12)
    logits = (tq @ tk.transpose(-1, -2)) / math.sqrt(wl.head_dim)
    np.testing.assert_allclose(ref["lse"], torch.logsumexp(logits, -1).permute(0, 2, 1).numpy(),
                               atol=1e-12)


def test_attention_special_values():
    wl = WORKLOADS["padded_tiny"]
    q, kk, _ = (bf16_to_f64(t) for t in make_qkv(wl))
    plan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size, 3)
    rng = np.random.default_rng(9)
    sel = np.sort(np.stack([rng.choice(8, 3, replace=False) for _ in range(16)]), axis=1)
    rp, ci = oracle.selection_to_csr(sel.reshape(1, 2, 8, 3))
    # V == 1 -> O == 1
    o, _ = oracle.block_sparse_attention(q, kk, np.ones_like(q), plan, rp, ci)
    np.testing.assert_allclose(o, 1.0, atol=1e-13)
    # convex hull: each output lies within [min, max] of its selected V rows
    v = rng.standard_normal(q.shape)
    o, _ = oracle.block_sparse_attention(q, kk, v, plan, rp, ci)
    lists = oracle.block_token_lists(plan)
    for r in range(16):
        h, i = divmod(r, 8)
        keys = np.concatenate([lists[j] for j in ci[rp[r]:rp[r + 1]]])
        lo = v[0, keys, h].min(axis=0)
        hi = v[0, keys, h].max(axis=0)
        oq = o[0, lists[i], h]
        assert np.all(oq >= lo - 1e-12) and np.all(oq <= hi + 1e-12)


def test_attention_one_hot_values_give_probability_rows():
    # D == S, V = identity: O[s, :] is the probability row of query s
    shape, block = (2, 4, 4), (2, 2, 2)
    s = 32
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, s, 1, s))
    kk = rng.standard_normal((1, s, 1, s))
    v = np.eye(s).reshape(1, s, 1, s)
    plan = oracle.make_plan(s, shape, block, 3)
    sc = rng.standard_normal((1, 1, plan.num_blocks, plan.num_blocks))
    sel, _ = oracle.select_topk(sc, 3)
    rp, ci = oracle.selection_to_csr(sel)
    o, _ = oracle.block_sparse_attention(q, kk, v, plan, rp, ci)
    beta = oracle.token_block_ids(plan)
    np.testing.assert_allclose(o[0, :, 0].sum(axis=1), 1.0, atol=1e-13)
    for tok in range(s):
        chosen = sel[0, 0, beta[tok]]
        assert np.all(o[0, tok, 0][~np.isin(beta, chosen)] == 0.0)
        assert np.all(o[0, tok, 0][np.isin(beta, chosen)] > 0.0)


def test_self_block_only_equals_dense_within_each_block():
    wl = WORKLOADS["padded_tiny"]
    q, kk, v = make_qkv(wl)
    plan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size)
    nb = plan.num_blocks
    sel = np.tile(np.arange(nb)[:, None], (1, 2, 1, 1)).reshape(1, 2, nb, 1)
    rp, ci = oracle.selection_to_csr(sel)
    o, _ = oracle.block_sparse_attention(bf16_to_f64(q), bf16_to_f64(kk), bf16_to_f64(v), plan, rp, ci)
    for toks in oracle.block_token_lists(plan):
        idx = torch.as_tensor(toks)
        tq, tk, tv = (t[:, idx].to(torch.float64).permute(0, 2, 1, 3) for t in (q, kk, v))
        dense = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).permute(0, 2, 1, 3)
        np.testing.assert_allclose(o[:, toks], dense.numpy(), atol=1e-12)


def test_key_permutation_inside_blocks_leaves_output():
    wl = WORKLOADS["padded_tiny"]
    q, kk, v = (bf16_to_f64(t) for t in make_qkv(wl))
    ref = oracle.vsa_reference(q, kk, v, wl.dit_seq_shape, wl.block_size, 4)
    perm = np.arange(wl.seq_len)
    rng = np.random.default_rng(1)
    for toks in oracle.block_token_lists(ref["plan"]):
        perm[toks] = rng.permutation(toks)
    o2, _ = oracle.block_sparse_attention(q, kk[:, perm], v[:, perm], ref["plan"],
                                          ref["row_ptr"], ref["col_idx"])
    np.testing.assert_allclose(o2, ref["out"], atol=1e-12)


def test_sampled_rows_agree_with_full_computation():
    wl = WORKLOADS["padded_tiny"]
    q, kk, v = (bf16_to_f64(t) for t in make_qkv(wl))
    ref = oracle.vsa_reference(q, kk, v, wl.dit_seq_shape, wl.block_size, 4)
    o, lse = oracle.block_sparse_attention(q, kk, v, ref["plan"], ref["row_ptr"], ref["col_idx"],
                                           query_rows=[3, 12])
    lists = oracle.block_token_lists(ref["plan"])
    for r in (3, 12):
        h, i = divmod(r, 8)
        np.testing.assert_array_equal(o[0, lists[i], h], ref["out"][0, lists[i], h])


def test_valid_flops_hand_count():
    plan = oracle.make_plan(910, (7, 13, 10), (4, 8, 8))
    counts = [256, 64, 160, 40, 192, 48, 120, 30]
    rp = np.array([0, 2, 2, 3, 3, 3, 3, 3, 4])      # one head, rows 0..7
    ci = np.array([0, 7, 5, 1])
    want = 4 * 128 * (counts[0] * (256 + 30) + counts[2] * 48 + counts[7] * 64)
    assert oracle.valid_flops(plan, rp, ci, 128) == want


# ------------------------------------------------- f1: gate-compress (coarse) branch

def test_compress_one_token_blocks_equal_library_dense_attention():
    # With 1-token tiles the per-tile pooling is the identity, so the coarse
    # branch is plain attention over the tokens: torch's fp64 SDPA.
    shape, heads, d = (2, 3, 4), 2, 16
    s = int(np.prod(shape))
    plan = oracle.make_plan(s, shape, (1, 1, 1))
    rng = np.random.default_rng(21)
    q, k, v = (rng.standard_normal((1, s, heads, d)) for _ in range(3))
    qb, kb, vb = (oracle.pool_blocks(x, plan) for x in (q, k, v))
    assert np.array_equal(qb, np.swapaxes(q, 1, 2))
    oc = oracle.compress_attention(qb, kb, vb, d)
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v))
    dense = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)
    np.testing.assert_allclose(oc, dense.numpy(), rtol=0, atol=1e-12)


def test_compress_closed_form_two_blocks():
    # D = 4: logits (2*1/2, 0) = (1, 0), weights e/(e+1) and 1/(e+1)
    qb = np.array([[[[2.0, 0, 0, 0]]]])
    kb = np.array([[[[1.0, 0, 0, 0], [0.0, 0, 0, 0]]]])
    vb = np.array([[[[1.0, 2, 0, 0], [0.0, 0, 4, 0]]]])
    e = math.e
    want = np.array([e / (e + 1), 2 * e / (e + 1), 4 / (e + 1), 0.0])
    np.testing.assert_allclose(oracle.compress_attention(qb, kb, vb, 4)[0, 0, 0], want,
                               rtol=0, atol=1e-15)


def test_compress_single_block_and_zero_queries():
    rng = np.random.default_rng(22)
    vb = rng.standard_normal((1, 2, 1, 8))
    # one block: the softmax over one key is 1
    out = oracle.compress_attention(rng.standard_normal((1, 2, 1, 8)),
                                    rng.standard_normal((1, 2, 1, 8)), vb, 8)
    np.testing.assert_allclose(out, vb, rtol=0, atol=1e-15)
    # zero queries: every logit is 0, the output is the plain mean of the values
    vb = rng.standard_normal((1, 2, 5, 8))
    out = oracle.compress_attention(np.zeros((1, 2, 5, 8)), rng.standard_normal((1, 2, 5, 8)),
                                    vb, 8)
    np.testing.assert_allclose(out, np.broadcast_to(vb.mean(axis=2, keepdims=True), out.shape),
                               rtol=0, atol=1e-14)


def test_gated_combine_special_cases():
    wl = WORKLOADS["padded_tiny"]
    plan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size)
    rng = np.random.default_rng(23)
    o_sparse = rng.standard_normal((1, wl.seq_len, 2, 4))
    o_coarse = rng.standard_normal((1, 2, plan.num_blocks, 4))
    assert np.array_equal(oracle.gated_combine(o_sparse, o_coarse, None, plan), o_sparse)
    assert np.array_equal(oracle.gated_combine(o_sparse, o_coarse, np.zeros_like(o_sparse), plan),
                          o_sparse)
    # sparse 0 and gate 1: every token carries its block's coarse output;
    # token (t, h, w) = (5, 12, 9) is s = (5*13 + 12)*10 + 9 = 779, block
    # (5//4, 12//8, 9//8) = (1, 1, 1) -> id (1*2 + 1)*2 + 1 = 7
    out = oracle.gated_combine(np.zeros_like(o_sparse), o_coarse, np.ones_like(o_sparse), plan)
    assert np.array_equal(out[0, 779], o_coarse[0, :, 7])
    assert np.array_equal(out[0, 0], o_coarse[0, :, 0])
    for b_id, toks in enumerate(oracle.block_token_lists(plan)):
        for s in toks[:3]:
            assert np.array_equal(out[0, s], o_coarse[0, :, b_id])


def test_gated_reference_whole_path_by_loops():
    wl = WORKLOADS["tiny"]
    q, kk, v = (bf16_to_f64(t) for t in make_qkv(wl))
    gate = np.random.default_rng(24).standard_normal(q.shape)
    ref = oracle.vsa_gated_reference(q, kk, v, gate, wl.dit_seq_shape, wl.block_size, wl.topk)
    plan, d = ref["plan"], wl.head_dim
    lists = oracle.block_token_lists(plan)
    for h in range(wl.heads):
        for i, toks in enumerate(lists):
            qb = q[0, toks, h].mean(axis=0)
            logits = np.array([qb @ kk[0, lists[j], h].mean(axis=0) for j in range(len(lists))])
            w = np.exp(logits / math.sqrt(d) - (logits / math.sqrt(d)).max())
            oc = sum(w[j] * v[0, lists[j], h].mean(axis=0) for j in range(len(lists))) / w.sum()
            for s in toks:
                want = ref["out"][0, s, h] + gate[0, s, h] * oc
                np.testing.assert_allclose(ref["gated_out"][0, s, h], want, rtol=0, atol=1e-12)


# ------------------------------------------------- f2: backward of the attention

def _torch_masked_grads(q, k, v, do, keep):
    """fp64 autograd of a dense S x S attention under a token keep-mask; fully
    masked query rows output 0 (and so get no gradient)."""
    tq, tk, tv = (torch.from_numpy(x).requires_grad_(True) for x in (q, k, v))
    d = q.shape[-1]
    logits = torch.einsum("bshd,bthd->bhst", tq, tk) / math.sqrt(d)
    km = torch.from_numpy(keep)
    anyk = km.any(dim=-1, keepdim=True)
    logits = torch.where(km, logits, torch.full_like(logits, -1e300))
    p = torch.softmax(torch.where(anyk, logits, torch.zeros_like(logits)), dim=-1) * anyk
    o = torch.einsum("bhst,bthd->bshd", p, tv)
    (o * torch.from_numpy(do)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("k", [1, 4])
def test_backward_matches_torch_autograd_masked(k):
    wl = WORKLOADS["padded_tiny"]
    q, kk, v = (bf16_to_f64(t) for t in make_qkv(wl))
    do = np.random.default_rng(31).standard_normal(q.shape)
    ref = oracle.vsa_reference(q, kk, v, wl.dit_seq_shape, wl.block_size, k)
    keep = _token_keep(ref["plan"], ref["row_ptr"], ref["col_idx"], 1, 2)
    got = oracle.block_sparse_attention_bwd(q, kk, v, do, ref["plan"], ref["row_ptr"],
                                            ref["col_idx"])
    for g, w in zip(got, _torch_masked_grads(q, kk, v, do, keep)):
        np.testing.assert_allclose(g, w, rtol=0, atol=1e-11)


def test_backward_csr_with_zero_rows_matches_torch_autograd():
    wl = WORKLOADS["tile64_tiny"]
    q, kk, v = (bf16_to_f64(t) for t in make_qkv(wl))
    rp, ci, _ = make_tile64_map(wl)
    plan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size)
    do = np.random.default_rng(32).standard_normal(q.shape)
    keep = _token_keep(plan, rp, ci, 1, 2)
    got = oracle.block_sparse_attention_bwd(q, kk, v, do, plan, rp, ci)
    for g, w in zip(got, _torch_masked_grads(q, kk, v, do, keep)):
        np.testing.assert_allclose(g, w, rtol=0, atol=1e-11)
    # query tokens of empty rows get no gradient
    nb = plan.num_blocks
    for r in np.nonzero(np.diff(rp) == 0)[0]:
        h, i = divmod(int(r), nb)
        assert np.all(got[0][0, oracle.block_token_lists(plan)[i], h] == 0)


def test_backward_all_blocks_equals_sdpa_autograd():
    wl = WORKLOADS["tiny"]
    q, kk, v = (bf16_to_f64(t) for t in make_qkv(wl))
    plan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size)
    nb = plan.num_blocks
    rp, ci = oracle.selection_to_csr(np.tile(np.arange(nb), (1, wl.heads, nb, 1)))
    do = np.random.default_rng(33).standard_normal(q.shape)
    got = oracle.block_sparse_attention_bwd(q, kk, v, do, plan, rp, ci)
    tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3).requires_grad_(True) for x in (q, kk, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)
    (o * torch.from_numpy(do).permute(0, 2, 1, 3)).sum().backward()
    for g, t in zip(got, (tq, tk, tv)):
        np.testing.assert_allclose(g, t.grad.permute(0, 2, 1, 3).numpy(), rtol=0, atol=1e-11)


def test_backward_constant_values_give_zero_qk_gradients():
    # if every value row is the same vector the output does not depend on the
    # logits, so dQ = dK = 0 and dV of each key is the probability-weighted dO
    wl = WORKLOADS["padded_tiny"]
    q, kk, _ = (bf16_to_f64(t) for t in make_qkv(wl))
    v = np.broadcast_to(np.linspace(-1, 1, wl.head_dim), q.shape).copy()
    do = np.random.default_rng(34).standard_normal(q.shape)
    ref = oracle.vsa_reference(q, kk, v, wl.dit_seq_shape, wl.block_size, 3)
    dq, dk, dv = oracle.block_sparse_attention_bwd(q, kk, v, do, ref["plan"], ref["row_ptr"],
                                                   ref["col_idx"])
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12
    # sum of dV over keys = sum of dO over queries with a non-empty row
    np.testing.assert_allclose(dv.sum(axis=1), do.sum(axis=1), rtol=0, atol=1e-10)


def test_backward_repeated_block_counts_twice():
    # a row listing block 1 twice is attention over block 1's keys duplicated
    shape, block = (2, 8, 8), (1, 8, 8)
    plan = oracle.make_plan(128, shape, block)
    rng = np.random.default_rng(35)
    q, k, v, do = (rng.standard_normal((1, 128, 1, 16)) for _ in range(4))
    rp, ci = np.array([0, 2, 3]), np.array([1, 1, 0])
    dq, dk, dv = oracle.block_sparse_attention_bwd(q, k, v, do, plan, rp, ci)
    toks0, toks1 = oracle.block_token_lists(plan)
    tq = torch.from_numpy(q[0, toks0, 0]).requires_grad_(True)
    tk = torch.from_numpy(k[0, toks1, 0]).requires_grad_(True)
    tv = torch.from_numpy(v[0, toks1, 0]).requires_grad_(True)
    kk2, vv2 = torch.cat([tk, tk]), torch.cat([tv, tv])
    o = torch.softmax(tq @ kk2.T / 4.0, dim=-1) @ vv2
    (o * torch.from_numpy(do[0, toks0, 0])).sum().backward()
    np.testing.assert_allclose(dq[0, toks0, 0], tq.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dk[0, toks1, 0], tk.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(dv[0, toks1, 0], tv.grad.numpy(), rtol=0, atol=1e-11)


def test_backward_finite_differences():
    wl = WORKLOADS["padded_tiny"]
    q, kk, v = (bf16_to_f64(t) for t in make_qkv(wl))
    plan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size, 2)
    ref = oracle.vsa_reference(q, kk, v, wl.dit_seq_shape, wl.block_size, 2)
    rp, ci = ref["row_ptr"], ref["col_idx"]
    do = np.random.default_rng(36).standard_normal(q.shape)
    grads = oracle.block_sparse_attention_bwd(q, kk, v, do, plan, rp, ci)

    def loss(qq, kk_, vv):
        return float((oracle.block_sparse_attention(qq, kk_, vv, plan, rp, ci)[0] * do).sum())
    eps = 1e-5
    for which, idx in ((0, (0, 5, 1, 3)), (1, (0, 700, 0, 17)), (2, (0, 130, 1, 64))):
        args = [q.copy(), kk.copy(), v.copy()]
        args[which][idx] += eps
        up = loss(*args)
        args[which][idx] -= 2 * eps
        dn = loss(*args)
        assert abs((up - dn) / (2 * eps) - grads[which][idx]) < 1e-6
