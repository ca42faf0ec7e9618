"""Pins for the float32 torch-CPU forms of the oracle (block_sparse_attention_f32,
vsa_reference_f32), which serve the layer-sized checks and the timed CPU
baseline.

Each is checked against what fixes it independently of its own code: the
brute-force dense S x S softmax with a token keep-mask, the float64 oracle
(itself pinned in test_oracle_pins.py), planted integer inputs whose block
means and scores are exact in float32, and the special cases of the
definition (empty rows, every block kept equals dense attention).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from tests.test_oracle_pins import _dense_masked, _token_keep
from vsa_inputs import WORKLOADS, bf16_to_f64, make_planted_block_means, make_qkv, make_tile64_map

F32_TOL = 2e-5   # float32 rounding of O (|O| < 5) and LSE over at most a few thousand keys


@pytest.mark.parametrize("k", [1, 4, 8])
def test_f32_attention_matches_dense_masked_bruteforce(k):
    wl = WORKLOADS["padded_tiny"]
    q, kk, v = make_qkv(wl)
    q64, k64, v64 = (bf16_to_f64(t) for t in (q, kk, v))
    ref = oracle.vsa_reference(q64, k64, v64, wl.dit_seq_shape, wl.block_size, k)
    o, lse = oracle.block_sparse_attention_f32(q, kk, v, ref["plan"], ref["row_ptr"],
                                               ref["col_idx"])
    keep = _token_keep(ref["plan"], ref["row_ptr"], ref["col_idx"], 1, 2)
    ob, lb = _dense_masked(q64, k64, v64, keep)
    assert o.dtype == torch.float32
    np.testing.assert_allclose(o.numpy(), ob, rtol=0, atol=F32_TOL)
    np.testing.assert_allclose(lse.numpy(), lb, rtol=0, atol=F32_TOL)


def test_f32_attention_csr_zero_rows_and_head_subset():
    wl = WORKLOADS["tile64_tiny"]
    q, kk, v = make_qkv(wl)
    rp, ci, _ = make_tile64_map(wl)
    plan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size)
    ref_o, ref_l = oracle.block_sparse_attention(bf16_to_f64(q), bf16_to_f64(kk),
                                                 bf16_to_f64(v), plan, rp, ci)
    o, lse = oracle.block_sparse_attention_f32(q, kk, v, plan, rp, ci)
    np.testing.assert_allclose(o.numpy(), ref_o, rtol=0, atol=F32_TOL)
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isneginf(lse.numpy()), ~fin)
    np.testing.assert_allclose(lse.numpy()[fin], ref_l[fin], rtol=0, atol=F32_TOL)
    nb = plan.num_blocks
    lists = oracle.block_token_lists(plan)
    for r in np.nonzero(np.diff(rp) == 0)[0]:
        h, i = divmod(int(r), nb)
        assert torch.all(o[0, lists[i], h] == 0)
    # a subset of heads: those heads identical, the others left as NaN
    o1, l1 = oracle.block_sparse_attention_f32(q, kk, v, plan, rp, ci, heads=[1])
    assert torch.equal(o1[:, :, 1], o[:, :, 1])
    assert torch.all(torch.isnan(o1[:, :, 0])) and torch.all(torch.isnan(l1[:, :, 0]))


@pytest.mark.parametrize("name", ["tiny", "padded_tiny"])
def test_f32_all_blocks_equals_library_dense_attention(name):
    wl = WORKLOADS[name]
    q, kk, v = make_qkv(wl)
    nb = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size).num_blocks
    ref = oracle.vsa_reference_f32(q, kk, v, wl.dit_seq_shape, wl.block_size, nb)
    assert np.array_equal(ref["sel"], np.broadcast_to(np.arange(nb), ref["sel"].shape))
    tq, tk, tv = (t.to(torch.float64).permute(0, 2, 1, 3) for t in (q, kk, v))
    dense = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv).permute(0, 2, 1, 3)
    np.testing.assert_allclose(ref["out"].numpy(), dense.numpy(), rtol=0, atol=F32_TOL)
    logits = (tq @ tk.transpose(-1, -2)) / math.sqrt(wl.head_dim)
    np.testing.assert_allclose(ref["lse"].numpy(),
                               torch.logsumexp(logits, -1).permute(0, 2, 1).numpy(), rtol=0,
                               atol=F32_TOL)


@pytest.mark.parametrize("name,k", [("tiny", 4), ("padded_tiny", 3), ("padded_tiny", 5)])
def test_f32_selection_equals_float64_outside_near_ties(name, k):
    wl = WORKLOADS[name]
    q, kk, v = make_qkv(wl)
    ref32 = oracle.vsa_reference_f32(q, kk, v, wl.dit_seq_shape, wl.block_size, k)
    ref64 = oracle.vsa_reference(bf16_to_f64(q), bf16_to_f64(kk), bf16_to_f64(v),
                                 wl.dit_seq_shape, wl.block_size, k)
    np.testing.assert_allclose(ref32["scores"].numpy(), ref64["scores"], rtol=0,
                               atol=1e-5 * max(1.0, np.abs(ref64["scores"]).max()))
    exact = ref64["margin"] >= 1e-3
    assert exact.mean() > 0.8
    assert np.array_equal(ref32["sel"][exact], ref64["sel"][exact])


def test_f32_selection_planted_exact_ties_prefer_lower_index():
    # integer block means: float32 pooling and scores are exact, so ties are
    # real ties and the lower block index must win
    shape = (8, 16, 16)
    xq, _ = make_planted_block_means(31, 1, 2, shape, (4, 8, 8), 128, lo=1, hi=2)
    xk, _ = make_planted_block_means(32, 1, 2, shape, (4, 8, 8), 128, lo=0, hi=1)
    for k in (1, 3, 5):
        ref = oracle.vsa_reference_f32(xq, xk, xk, shape, (4, 8, 8), k)
        sc = ref["scores"].numpy().astype(np.float64)
        for b, h, i in np.ndindex(1, 2, 8):
            row = sc[b, h, i]
            want = sorted(sorted(range(8), key=lambda j: (-row[j], j))[:k])
            assert ref["sel"][b, h, i].tolist() == want
