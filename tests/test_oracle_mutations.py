"""Plant plausible mistakes in the CPU oracle and check that a pin catches each.

Every mutation here is applied to the oracle only, on the CPU, for the
duration of one test (monkeypatch).  A mutation that no pin catches would mean
the pins leave that part of the oracle unchecked.
"""
import math

import numpy as np
import pytest

import oracle
import oracle.vsa_oracle as ov
import tests.test_oracle_pins as pins


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(ov, name, fn)
    monkeypatch.setattr(oracle, name, fn)


def _fails(check, *args):
    with pytest.raises(AssertionError):
        check(*args)


def test_pool_divided_by_block_volume_is_caught(monkeypatch):
    def bad_pool(x, plan):
        x = np.asarray(x, np.float64)
        out = np.empty((x.shape[0], x.shape[2], plan.num_blocks, x.shape[3]))
        for b_id, toks in enumerate(ov.block_token_lists(plan)):
            out[:, :, b_id, :] = x[:, toks].sum(axis=1) / plan.block_volume
        return out
    _patch(monkeypatch, "pool_blocks", bad_pool)
    _fails(pins.test_pool_planted_means_exact, (7, 13, 10))


def test_transposed_scores_are_caught(monkeypatch):
    _patch(monkeypatch, "block_scores",
           lambda qb, kb: np.matmul(np.asarray(kb, float), np.swapaxes(np.asarray(qb, float), -1, -2)))
    _fails(pins.test_score_planted_integer_products)


def test_tie_to_higher_index_is_caught(monkeypatch):
    orig = ov.select_topk

    def bad(scores, k):
        s = np.asarray(scores, np.float64)
        flipped, m = orig(s[..., ::-1], k)
        return np.sort(s.shape[-1] - 1 - flipped, axis=-1), m
    _patch(monkeypatch, "select_topk", bad)
    _fails(pins.test_topk_hand_examples_with_ties)


def test_keeping_smallest_scores_is_caught(monkeypatch):
    orig = ov.select_topk
    _patch(monkeypatch, "select_topk", lambda s, k: orig(-np.asarray(s, np.float64), k))
    _fails(pins.test_topk_hand_examples_with_ties)


def test_ranking_float32_rounded_scores_is_caught(monkeypatch):
    orig = ov.select_topk

    def bad(scores, k):
        s = np.asarray(scores, np.float64)
        sel, _ = orig(s.astype(np.float32).astype(np.float64), k)
        return sel, orig(s, k)[1]
    _patch(monkeypatch, "select_topk", bad)
    _fails(pins.test_topk_ranks_full_precision_scores)


def _attention_with(logit_fn):
    def att(q, k, v, plan, row_ptr, col_idx, query_rows=None):
        q, k, v = (np.asarray(t, np.float64) for t in (q, k, v))
        bsz, s, nh, d = q.shape
        nb = plan.num_blocks
        lists = ov.block_token_lists(plan)
        out = np.zeros_like(q)
        lse = np.full((bsz, s, nh), -np.inf)
        for r in range(bsz * nh * nb):
            b, rem = divmod(r, nh * nb)
            h, i = divmod(rem, nb)
            cols = col_idx[row_ptr[r]:row_ptr[r + 1]]
            if len(cols) == 0:
                continue
            qt = lists[i]
            kt = np.concatenate([lists[j] for j in cols])
            lg = logit_fn(q[b, qt, h], k[b, kt, h], d)
            p = np.exp(lg - lg.max(axis=1, keepdims=True))
            out[b, qt, h] = p @ v[b, kt, h] / p.sum(axis=1, keepdims=True)
            lse[b, qt, h] = np.log(np.exp(lg).sum(axis=1))
        return out, lse
    return att


def test_missing_softmax_scale_is_caught(monkeypatch):
    _patch(monkeypatch, "block_sparse_attention", _attention_with(lambda qq, kk, d: qq @ kk.T))
    _fails(pins.test_all_blocks_equals_library_dense_attention, "tiny")


def test_wrong_scale_sign_is_caught(monkeypatch):
    _patch(monkeypatch, "block_sparse_attention",
           _attention_with(lambda qq, kk, d: -(qq @ kk.T) / math.sqrt(d)))
    _fails(pins.test_attention_matches_dense_masked_bruteforce, 4)


def test_keys_from_query_block_is_caught(monkeypatch):
    # a wrong index: attend to the query block's own tokens instead of the row's blocks
    orig = ov.block_sparse_attention

    def bad(q, k, v, plan, row_ptr, col_idx, query_rows=None):
        nb = plan.num_blocks
        rows = len(row_ptr) - 1
        cnt = np.diff(row_ptr)
        ci = np.concatenate([np.full(cnt[r], r % nb) for r in range(rows)]).astype(np.int64)
        return orig(q, k, v, plan, row_ptr, ci, query_rows)
    _patch(monkeypatch, "block_sparse_attention", bad)
    _fails(pins.test_attention_matches_dense_masked_bruteforce, 4)


def test_w_major_block_numbering_is_caught(monkeypatch):
    def bad_ids(plan):
        t, h, w = plan.dit_seq_shape
        bt, bh, bw = plan.block_size
        nt, nh, nw = plan.block_grid
        tt, hh, ww = np.meshgrid(np.arange(t), np.arange(h), np.arange(w), indexing="ij")
        return (((ww // bw) * nh + (hh // bh)) * nt + (tt // bt)).reshape(-1)
    _patch(monkeypatch, "token_block_ids", bad_ids)
    _fails(pins.test_token_partition_hand_points_and_invariants)


def test_floor_block_grid_is_caught(monkeypatch):
    class FloorPlan(ov.Plan):
        def __init__(self, *a, **kw):
            super().__init__(*a, **kw)
            self.block_grid = tuple(g // b for g, b in zip(self.dit_seq_shape, self.block_size))
            nt, nh, nw = self.block_grid
            self.num_blocks = nt * nh * nw
    _patch(monkeypatch, "make_plan", lambda *a, **kw: FloorPlan(*a, **kw))
    _fails(pins.test_routing_line_matches_page_worked_example, pins.os.path.join(
        pins.os.path.dirname(pins.__file__), "golden"))


def test_coarse_without_scale_is_caught(monkeypatch):
    def bad(qb, kb, vb, d):
        lg = ov.block_scores(qb, kb)
        p = np.exp(lg - lg.max(axis=-1, keepdims=True))
        return np.matmul(p, vb) / p.sum(axis=-1, keepdims=True)
    _patch(monkeypatch, "compress_attention", bad)
    _fails(pins.test_compress_closed_form_two_blocks)


def test_coarse_transposed_logits_are_caught(monkeypatch):
    def bad(qb, kb, vb, d):
        lg = np.swapaxes(ov.block_scores(qb, kb), -1, -2) / math.sqrt(d)
        p = np.exp(lg - lg.max(axis=-1, keepdims=True))
        return np.matmul(p, vb) / p.sum(axis=-1, keepdims=True)
    _patch(monkeypatch, "compress_attention", bad)
    _fails(pins.test_compress_one_token_blocks_equal_library_dense_attention)


def test_coarse_softmax_over_queries_is_caught(monkeypatch):
    def bad(qb, kb, vb, d):
        lg = ov.block_scores(qb, kb) / math.sqrt(d)
        p = np.exp(lg - lg.max(axis=-2, keepdims=True))
        return np.matmul(p / p.sum(axis=-2, keepdims=True), vb)
    _patch(monkeypatch, "compress_attention", bad)
    _fails(pins.test_compress_one_token_blocks_equal_library_dense_attention)


def test_gate_broadcast_by_token_index_is_caught(monkeypatch):
    def bad(o_sparse, o_coarse, gate, plan):
        o_sparse = np.asarray(o_sparse, np.float64)
        if gate is None:
            return o_sparse
        beta = np.arange(o_sparse.shape[1]) % plan.num_blocks
        return o_sparse + gate * np.swapaxes(np.asarray(o_coarse)[:, :, beta, :], 1, 2)
    _patch(monkeypatch, "gated_combine", bad)
    _fails(pins.test_gated_combine_special_cases)


def _bwd_variant(drop_d_term=False, unscaled_dk=False, plain_assign=False):
    def bwd(q, k, v, do, plan, row_ptr, col_idx):
        q, k, v, do = (np.asarray(x, np.float64) for x in (q, k, v, do))
        bsz, s, nh, d = q.shape
        nb = plan.num_blocks
        lists = ov.block_token_lists(plan)
        sc = 1.0 / math.sqrt(d)
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for r in range(bsz * nh * nb):
            b, rem = divmod(r, nh * nb)
            h, i = divmod(rem, nb)
            cols = col_idx[row_ptr[r]:row_ptr[r + 1]]
            if len(cols) == 0:
                continue
            qt, kt = lists[i], np.concatenate([lists[j] for j in cols])
            lg = q[b, qt, h] @ k[b, kt, h].T * sc
            p = np.exp(lg - lg.max(axis=1, keepdims=True))
            p /= p.sum(axis=1, keepdims=True)
            dp = do[b, qt, h] @ v[b, kt, h].T
            corr = 0.0 if drop_d_term else (do[b, qt, h] * (p @ v[b, kt, h])).sum(axis=1, keepdims=True)
            ds = p * (dp - corr)
            dq[b, qt, h] += ds @ k[b, kt, h] * sc
            gk = ds.T @ q[b, qt, h] * (1.0 if unscaled_dk else sc)
            gv = p.T @ do[b, qt, h]
            if plain_assign:
                dk[b, kt, h] += gk
                dv[b, kt, h] += gv
            else:
                np.add.at(dk[:, :, h], (b, kt), gk)
                np.add.at(dv[:, :, h], (b, kt), gv)
        return dq, dk, dv
    return bwd


def test_backward_without_rowsum_term_is_caught(monkeypatch):
    _patch(monkeypatch, "block_sparse_attention_bwd", _bwd_variant(drop_d_term=True))
    _fails(pins.test_backward_matches_torch_autograd_masked, 4)


def test_backward_unscaled_dk_is_caught(monkeypatch):
    _patch(monkeypatch, "block_sparse_attention_bwd", _bwd_variant(unscaled_dk=True))
    _fails(pins.test_backward_all_blocks_equals_sdpa_autograd)


def test_backward_dropping_repeated_keys_is_caught(monkeypatch):
    _patch(monkeypatch, "block_sparse_attention_bwd", _bwd_variant(plain_assign=True))
    _fails(pins.test_backward_repeated_block_counts_twice)


def test_backward_mutation_harness_is_faithful(monkeypatch):
    # the unmutated copy passes the pins the mutations fail
    _patch(monkeypatch, "block_sparse_attention_bwd", _bwd_variant())
    pins.test_backward_matches_torch_autograd_masked(4)
    pins.test_backward_repeated_block_counts_twice()


# ------------------------------------------ the float32 forms (test_oracle_f32_pins.py)

import tests.test_oracle_f32_pins as f32pins  # noqa: E402


def test_f32_attention_without_scale_is_caught(monkeypatch):
    import torch
    orig = ov.block_sparse_attention_f32

    def bad(q, k, v, plan, row_ptr, col_idx, heads=None):
        d = torch.as_tensor(q).shape[-1]
        # logits unscaled: feed q * sqrt(d) to the correct function
        return orig(torch.as_tensor(q).to(torch.float32) * math.sqrt(d), k, v, plan, row_ptr,
                    col_idx, heads)
    _patch(monkeypatch, "block_sparse_attention_f32", bad)
    _fails(f32pins.test_f32_attention_matches_dense_masked_bruteforce, 4)


def test_f32_selection_tie_to_higher_index_is_caught(monkeypatch):
    orig = ov.vsa_reference_f32

    def bad(q, k, v, dit_seq_shape, block_size, topk, heads=None):
        ref = orig(q, k, v, dit_seq_shape, block_size, topk, heads)
        s = ref["scores"]
        nb = s.shape[-1]
        import torch
        order = torch.sort(-s.flip(-1), dim=-1, stable=True).indices[..., :topk]
        ref["sel"] = np.sort((nb - 1 - order).numpy(), axis=-1)
        return ref
    _patch(monkeypatch, "vsa_reference_f32", bad)
    _fails(f32pins.test_f32_selection_planted_exact_ties_prefer_lower_index)
