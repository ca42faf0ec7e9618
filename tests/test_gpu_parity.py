"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Tolerances for floating-point outputs are the ones the problem statement
fixes for bf16 inputs with fp32 accumulation: attention output max-abs 2e-2
and mean-abs 2e-3 against the fp64 oracle.  Integer and layout work (gather,
scatter, the selected block ids) must match bit for bit; selection rows whose
gap between the k-th and (k+1)-th oracle score is below 1e-3 are near-ties and
are instead checked for validity (every selected block scores within 1e-3 of
the k-th best).
"""
import math

import numpy as np
import pytest
import torch

import block_sparse_video_tile_amd as vsa
import oracle
from tests.gpu_common import (DEV, MARGIN, MAX_ABS, MEAN_ABS, _attend, _compare_rows,
                              _full_forward, _gather_all, _host, _plan, _say,
                              blocked_positions, check_full_forward, compare_all_rows, need_gpu)
from vsa_inputs import (WORKLOADS, bf16_to_f64, make_planted_block_means, make_qkv,
                        make_tile64_map)

pytestmark = pytest.mark.gpu



@pytest.fixture(autouse=True)
def _need_gpu(request):
    need_gpu(request)


# ------------------------------------------------------------------ gather / scatter

@pytest.mark.parametrize("name", ["tiny", "padded_tiny", "tile64_tiny"])
def test_gather_scatter_roundtrip_and_layout(name):
    wl = WORKLOADS[name]
    q, k, v = make_qkv(wl)
    plan = _plan(wl)
    oplan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size)
    qb, kb, vb, qp, kp = _gather_all(plan, q, k, v)
    torch.cuda.synchronize()
    vol = oplan.block_volume
    qbh, vbh = qb.cpu(), vb.cpu()
    for beta, toks in enumerate(oracle.block_token_lists(oplan)):
        c = len(toks)
        # valid rows are the block's tokens in raster order, pad rows zero (bitwise)
        assert torch.equal(qbh[:, :, beta * vol:beta * vol + c], q[:, toks].permute(0, 2, 1, 3))
        assert torch.all(qbh[:, :, beta * vol + c:(beta + 1) * vol].view(torch.int16) == 0)
        # V^T: chunk-major, d rows, 64 tokens per chunk
        chunks = vbh[:, :, beta * (vol // 64):(beta + 1) * (vol // 64)]   # [B,NH,ch,D,64]
        flat = chunks.permute(0, 1, 2, 4, 3).reshape(wl.batch, wl.heads, vol, wl.head_dim)
        assert torch.equal(flat[:, :, :c], v[:, toks].permute(0, 2, 1, 3))
        assert torch.all(flat[:, :, c:].view(torch.int16) == 0)
    out = torch.empty_like(q, device=DEV)
    vsa.vsa_scatter(plan, kb, out)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), k)


@pytest.mark.parametrize("name", ["tiny", "padded_tiny", "wan5b_k64"])
def test_pooled_means(name):
    wl = WORKLOADS[name]
    q, k, v = make_qkv(wl)
    plan = _plan(wl)
    oplan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size)
    _, _, _, qp, kp = _gather_all(plan, q, k, v)
    for dev, x in ((qp, q), (kp, k)):
        ref = oracle.pool_blocks(bf16_to_f64(x), oplan)
        np.testing.assert_allclose(_host(dev), ref, rtol=0, atol=1e-5)


@pytest.mark.parametrize("name", ["padded_tiny", "wan5b_k64"])
def test_pooled_v_from_the_v_gather_equals_the_means_only_pass(name):
    """The V gather sums each block in the order of the means-only pass, so the
    blocked and the gather-free paths feed the coarse branch the same bits."""
    wl = WORKLOADS[name]
    _, _, v = make_qkv(wl)
    plan = _plan(wl)
    oplan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size)
    dv = v.to(DEV)
    vb = torch.empty(plan.blocked_vt_shape(), dtype=torch.bfloat16, device=DEV)
    vp = torch.empty(plan.pooled_shape(), dtype=torch.float32, device=DEV)
    vp_alone = torch.full_like(vp, 7.0)
    vsa.vsa_gather(plan, vsa.VSA_ROLE_V, dv, vb, vp)
    vsa.vsa_gather(plan, vsa.VSA_ROLE_V, dv, None, vp_alone)
    torch.cuda.synchronize()
    assert torch.equal(vp.cpu(), vp_alone.cpu())
    np.testing.assert_allclose(_host(vp), oracle.pool_blocks(bf16_to_f64(v), oplan), rtol=0,
                               atol=1e-5)


def test_pooled_planted_exact():
    shape = (7, 13, 10)
    x, mu = make_planted_block_means(11, 1, 2, shape, (4, 8, 8), 128)
    plan = vsa.vsa_plan(910, shape, (4, 8, 8), batch=1, num_heads=2, topk=2)
    qb = torch.empty(plan.blocked_shape(), dtype=torch.bfloat16, device=DEV)
    qp = torch.empty(plan.pooled_shape(), dtype=torch.float32, device=DEV)
    vsa.vsa_gather(plan, vsa.VSA_ROLE_Q, x.to(DEV), qb, qp)
    assert np.array_equal(_host(qp), mu.reshape(1, 2, 8, 128).numpy().astype(np.float32))


# ------------------------------------------------------------------ score / top-k

def _check_selection(plan, oplan, qp, kp, k, q64, k64, allow_near_ties=True):
    rows = plan.num_rows()
    col = torch.empty(rows * k, dtype=torch.int32, device=DEV)
    sc = torch.empty((plan.batch, plan.heads, plan.num_blocks, plan.num_blocks),
                     dtype=torch.float32, device=DEV)
    vsa.vsa_score_topk(plan, qp, kp, k, col, sc)
    gsel = col.cpu().numpy().reshape(plan.batch, plan.heads, plan.num_blocks, k)
    ref_sc = oracle.block_scores(oracle.pool_blocks(q64, oplan), oracle.pool_blocks(k64, oplan))
    sel, margin = oracle.select_topk(ref_sc, k)
    np.testing.assert_allclose(_host(sc), ref_sc, rtol=0, atol=1e-4 * max(1, np.abs(ref_sc).max()))
    exact = margin >= MARGIN
    assert np.array_equal(gsel[exact], sel[exact])
    near = np.argwhere(~exact)
    for idx in near:
        row_sc = ref_sc[tuple(idx)]
        kth = np.sort(row_sc)[::-1][k - 1]
        g = gsel[tuple(idx)]
        assert len(set(g.tolist())) == k and np.all(np.diff(g) > 0)
        assert np.all(row_sc[g] >= kth - MARGIN)
    if not allow_near_ties:
        assert len(near) == 0
    return gsel, sel, margin, len(near)


@pytest.mark.parametrize("name,k", [("tiny", 4), ("tiny", 1), ("tiny", 8), ("padded_tiny", 3),
                                    ("wan5b_k64", 64), ("wan5b_k16", 16), ("wan5b_k120", 120)])
def test_score_topk_matches_oracle(name, k):
    wl = WORKLOADS[name]
    q, kk, v = make_qkv(wl)
    plan = _plan(wl, k)
    oplan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size)
    _, _, _, qp, kp = _gather_all(plan, q, kk, v)
    _, _, _, n_near = _check_selection(plan, oplan, qp, kp, k, bf16_to_f64(q), bf16_to_f64(kk))
    _say(f"    near-tie rows excluded from the exact check: {n_near} of {plan.num_rows()}")
    assert n_near <= 0.10 * plan.num_rows()


def test_topk_planted_exact_ties():
    shape = (8, 16, 16)
    xq, _ = make_planted_block_means(31, 1, 2, shape, (4, 8, 8), 128, lo=1, hi=2)
    xk, _ = make_planted_block_means(32, 1, 2, shape, (4, 8, 8), 128, lo=0, hi=1)
    plan = vsa.vsa_plan(2048, shape, (4, 8, 8), batch=1, num_heads=2, topk=3)
    oplan = oracle.make_plan(2048, shape, (4, 8, 8))
    _, _, _, qp, kp = _gather_all(plan, xq, xk, xk)
    for k in (1, 3, 5, 8):
        # integer scores: exact on both sides, ties broken to the lower index
        gsel, sel, margin, _ = _check_selection(plan, oplan, qp, kp, k, bf16_to_f64(xq),
                                                bf16_to_f64(xk))
        assert np.array_equal(gsel, sel)


# ------------------------------------------------------------------ attention

def _oracle_map_attention(name, k):
    wl = WORKLOADS[name]
    q, kk, v = make_qkv(wl)
    plan = _plan(wl, k)
    q64, k64, v64 = bf16_to_f64(q), bf16_to_f64(kk), bf16_to_f64(v)
    ref = oracle.vsa_reference(q64, k64, v64, wl.dit_seq_shape, wl.block_size, k)
    qb, kb, vb, _, _ = _gather_all(plan, q, kk, v)
    ob, lse = _attend(plan, qb, kb, vb, None, ref["col_idx"], uniform_k=k)
    return wl, plan, ref, ob, lse


@pytest.mark.parametrize("name,k", [("tiny", 4), ("tiny", 8), ("tiny", 1), ("padded_tiny", 1),
                                    ("padded_tiny", 4), ("padded_tiny", 8)])
def test_attention_fed_oracle_map(name, k):
    wl, plan, ref, ob, lse = _oracle_map_attention(name, k)
    mx, mean, lerr = _compare_rows(ref["plan"], _host(ob), _host(lse), ref["out"], ref["lse"],
                                   range(plan.num_rows()), wl.heads, ref["plan"].block_volume)
    _say(f"    max-abs {mx:.3e} mean-abs {mean:.3e} lse {lerr:.2e}")
    assert mx <= MAX_ABS and mean <= MEAN_ABS and lerr <= 1e-3


def test_attention_csr_nonuniform_with_zero_rows():
    wl = WORKLOADS["tile64_tiny"]
    q, kk, v = make_qkv(wl)
    rp, ci, _ = make_tile64_map(wl)
    assert np.any(np.diff(rp) == 0)
    plan = _plan(wl)
    oplan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size)
    ref_o, ref_l = oracle.block_sparse_attention(bf16_to_f64(q), bf16_to_f64(kk), bf16_to_f64(v),
                                                 oplan, rp, ci)
    qb, kb, vb, _, _ = _gather_all(plan, q, kk, v)
    ob, lse = _attend(plan, qb, kb, vb, rp, ci)
    mx, mean, lerr = _compare_rows(oplan, _host(ob), _host(lse), ref_o, ref_l,
                                   range(plan.num_rows()), wl.heads, 64)
    assert mx <= MAX_ABS and mean <= MEAN_ABS and lerr <= 1e-3
    obh = _host(ob)
    for r in np.nonzero(np.diff(rp) == 0)[0]:
        h, i = divmod(int(r), oplan.num_blocks)
        assert np.all(obh[0, h, i * 64:(i + 1) * 64] == 0)


def test_attention_uniform_k_zero_writes_zero():
    wl = WORKLOADS["tiny"]
    q, kk, v = make_qkv(wl)
    plan = _plan(wl)
    qb, kb, vb, _, _ = _gather_all(plan, q, kk, v)
    ob, lse = _attend(plan, qb, kb, vb, None, np.zeros(1, np.int32), uniform_k=0)
    assert torch.all(ob == 0) and torch.all(torch.isneginf(lse))


def test_attention_malformed_map_is_sanitised():
    # ids outside [0, nb) are skipped and row offsets clamp to [0, nnz]
    wl = WORKLOADS["padded_tiny"]
    q, kk, v = make_qkv(wl)
    plan = _plan(wl)
    oplan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size)
    rows = plan.num_rows()
    rng = np.random.default_rng(2)
    ci = rng.integers(-3, 11, size=5 * rows).astype(np.int32)
    rp = np.arange(rows + 1, dtype=np.int64) * 5
    rp[-3:] = [5 * rows + 7, 5 * rows + 9, 5 * rows + 40]   # offsets past nnz
    rp[4] = rp[3] - 2                                       # a decreasing offset
    clean_rp, clean_ci = [0], []
    for r in range(rows):
        beg = min(max(int(rp[r]), 0), len(ci))
        end = min(max(int(rp[r + 1]), beg), len(ci))
        row = [int(j) for j in ci[beg:end] if 0 <= j < oplan.num_blocks]
        clean_ci += row
        clean_rp.append(len(clean_ci))
    # repeated ids within a row weigh a block twice in both implementations only if the
    # oracle is given the same repeats, which it is (clean_ci keeps them)
    ref_o, ref_l = oracle.block_sparse_attention(bf16_to_f64(q), bf16_to_f64(kk), bf16_to_f64(v),
                                                 oplan, np.array(clean_rp), np.array(clean_ci))
    qb, kb, vb, _, _ = _gather_all(plan, q, kk, v)
    ob, lse = _attend(plan, qb, kb, vb, rp.astype(np.int32), ci)
    mx, mean, _ = _compare_rows(oplan, _host(ob), None, ref_o, ref_l, range(rows), wl.heads,
                                oplan.block_volume)
    assert mx <= MAX_ABS and mean <= MEAN_ABS


def test_forward_tiny_end_to_end_and_deterministic():
    for name in ("tiny", "padded_tiny"):
        wl = WORKLOADS[name]
        q, kk, v = make_qkv(wl)
        plan = _plan(wl)
        ref = oracle.vsa_reference(bf16_to_f64(q), bf16_to_f64(kk), bf16_to_f64(v),
                                   wl.dit_seq_shape, wl.block_size, wl.topk)
        ws = torch.empty(vsa.vsa_forward_workspace_size(plan), dtype=torch.uint8, device=DEV)
        outs = []
        for _ in range(2):
            out = torch.empty(plan.raster_shape(), dtype=torch.bfloat16, device=DEV)
            col = torch.empty(plan.num_rows() * wl.topk, dtype=torch.int32, device=DEV)
            vsa.vsa_forward(plan, q.to(DEV), kk.to(DEV), v.to(DEV), out, ws, col)
            outs.append((out.cpu(), col.cpu()))
        assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
        exact = (ref["margin"] >= MARGIN).reshape(-1)
        assert np.array_equal(outs[0][1].numpy().reshape(-1, wl.topk)[exact],
                              ref["sel"].reshape(-1, wl.topk)[exact])
        if exact.all():
            err = np.abs(outs[0][0].double().numpy() - ref["out"])
            assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS


# ------------------------------------------------------------------ full-size shapes

@pytest.mark.parametrize("name,k", [("wan5b_k64", None), ("wan5b_k16", None), ("wan5b_k32", None),
                                    ("wan13b_long", None)])
def test_full_size_forward_every_row(name, k):
    # every row of every head vs the float32 oracle, four whole heads vs float64
    check_full_forward(name, k)


def test_head_shard_with_split_rows_every_row():
    """One GPU's share of an 8-way head shard of the 27280-token layer (3
    heads, 360 rows): the balanced launch splits the last 16 rows of each
    queue into halves merged across workgroups; every row of all three heads
    against the float32 and the float64 oracle."""
    check_full_forward("wan5b_k64_h3", fp64_heads=(0, 1, 2))


def test_full_size_attention_fed_oracle_map_every_row():
    """Attention fed the float64 oracle's own selection (not the GPU's), every row."""
    wl = WORKLOADS["wan5b_k64"]
    k = wl.topk
    q, kk, v = make_qkv(wl)
    plan = _plan(wl, k)
    oplan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size, k)
    q64, k64 = bf16_to_f64(q), bf16_to_f64(kk)
    sc = oracle.block_scores(oracle.pool_blocks(q64, oplan), oracle.pool_blocks(k64, oplan))
    sel, margin = oracle.select_topk(sc, k)
    _say(f"    oracle map: near-tie rows {int((margin < MARGIN).sum())} of {margin.size}")
    rp, ci = oracle.selection_to_csr(sel)
    qb, kb, vb, _, _ = _gather_all(plan, q, kk, v)
    ob, lse = _attend(plan, qb, kb, vb, None, ci, uniform_k=k)
    out = torch.empty(plan.raster_shape(), dtype=torch.bfloat16, device=DEV)
    vsa.vsa_scatter(plan, ob, out)
    torch.cuda.synchronize()
    o32, l32 = oracle.block_sparse_attention_f32(q, kk, v, oplan, rp, ci)
    compare_all_rows("oracle map, all rows vs float32 oracle", out.cpu(), o32, lse.cpu().numpy(),
                     l32.numpy(), oplan)
    # pad query slots of the blocked output are written as zero
    _, _, pads = blocked_positions(oplan)
    assert torch.all(ob[:, :, pads] == 0)


def test_all_blocks_equals_dense_attention_full_size():
    # topk == num_blocks: the sparse kernel over every block is dense attention
    wl, k, q, kk, v, plan, out, col, lse = check_full_forward("wan5b_k120")
    assert np.array_equal(col.reshape(-1, 120), np.tile(np.arange(120), (plan.num_rows(), 1)))
    # two whole heads against torch's dense attention over all 27280 tokens
    for h in (0, 23):
        tq, tk, tv = (t[0, :, h].to(torch.float32) for t in (q, kk, v))
        errs = []
        for c0 in range(0, wl.seq_len, 2048):
            dense = torch.nn.functional.scaled_dot_product_attention(
                tq[None, c0:c0 + 2048], tk[None], tv[None])[0]
            errs.append((out[0, c0:c0 + 2048, h].to(torch.float32) - dense).abs())
        err = torch.cat(errs)
        _say(f"    head {h} vs dense SDPA: max-abs {err.max().item():.3e} "
             f"mean-abs {err.mean().item():.3e}")
        assert err.max().item() <= MAX_ABS and err.mean().item() <= MEAN_ABS


@pytest.mark.parametrize("name", ["tile64_csr", "tile64_csr_zero"])
def test_tile64_csr_full_size_every_row(name):
    wl = WORKLOADS[name]
    q, kk, v = make_qkv(wl)
    rp, ci, nt = make_tile64_map(wl)
    plan = _plan(wl)
    oplan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size)
    qb, kb, vb, _, _ = _gather_all(plan, q, kk, v)
    ob, lse = _attend(plan, qb, kb, vb, rp, ci)
    torch.cuda.synchronize()
    # 1-D 64-token tiles of a 64-divisible sequence: the blocked layout is the raster one
    got = ob.cpu().permute(0, 2, 1, 3)
    o32, l32 = oracle.block_sparse_attention_f32(q, kk, v, oplan, rp, ci)
    compare_all_rows("all rows vs float32 oracle", got, o32, lse.cpu().numpy(), l32.numpy(),
                     oplan)
    rows = list(range(nt)) + list(range(23 * nt, 24 * nt))
    o64, l64 = oracle.block_sparse_attention(bf16_to_f64(q), bf16_to_f64(kk), bf16_to_f64(v),
                                             oplan, rp, ci, query_rows=rows)
    compare_all_rows("heads [0, 23] vs float64 oracle", got, o64, lse.cpu().numpy(), l64, oplan,
                     heads=(0, 23))
    counts = np.diff(rp)
    for r in np.nonzero(counts == 0)[0]:
        h, i = divmod(int(r), nt)
        assert torch.all(got[0, i * 64:(i + 1) * 64, h] == 0)
    _say(f"    rows with no blocks: {int((counts == 0).sum())}; longest row {int(counts.max())}")


def test_repeat_runs_bitwise_equal_full_size():
    a = _full_forward("wan5b_k64")
    b = _full_forward("wan5b_k64")
    assert torch.equal(a[6], b[6]) and np.array_equal(a[7], b[7])
