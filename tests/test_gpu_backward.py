"""GPU parity of the block-sparse attention backward against the CPU oracle.

The forward runs through the C ABI to produce O and LSE, the backward then
produces dQ, dK and dV, which are scattered back to raster order and compared
with the fp64 oracle's gradients on the same map.  The output gradient dO is
a seeded N(0, 1) tensor.  Tolerance (bf16 tensors): the gradients are
products of bf16-rounded P and dS with bf16 operands accumulated in fp32, so
each carries a relative error of a few 2^-9; the bound used is max-abs
<= 3e-2 * max(1, max|ref|) and mean-abs <= 3e-3 * max(1, mean|ref|).
"""
import numpy as np
import pytest
import torch

import block_sparse_video_tile_amd as vsa
import oracle
from tests.gpu_common import DEV, _plan, _say, need_gpu
from vsa_inputs import WORKLOADS, bf16_to_f64, make_qkv, make_tile64_map

pytestmark = pytest.mark.gpu

MAX_REL, MEAN_REL = 3e-2, 3e-3


@pytest.fixture(autouse=True)
def _need_gpu(request):
    need_gpu(request)


def _dout(wl, dtype, seed=41):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn((wl.batch, wl.seq_len, wl.heads, wl.head_dim), generator=g).to(dtype)


def _run(plan, q, k, v, do, row_ptr, col_idx, uniform_k):
    """Forward + backward through the C ABI; returns raster (dq, dk, dv) and blocked grads."""
    et = plan.torch_dtype()
    bs, vts = plan.blocked_shape(), plan.blocked_vt_shape()
    qb, kb, vb, dob = (torch.empty(bs, dtype=et, device=DEV) for _ in range(4))
    vtb = torch.empty(vts, dtype=et, device=DEV)
    vsa.vsa_gather(plan, vsa.VSA_ROLE_Q, q.to(DEV), qb)
    vsa.vsa_gather(plan, vsa.VSA_ROLE_K, k.to(DEV), kb)
    vsa.vsa_gather(plan, vsa.VSA_ROLE_K, v.to(DEV), vb)     # token-major V for the backward
    vsa.vsa_gather(plan, vsa.VSA_ROLE_V, v.to(DEV), vtb)    # V^T for the forward
    vsa.vsa_gather(plan, vsa.VSA_ROLE_Q, do.to(DEV), dob)
    rp = None if row_ptr is None else torch.as_tensor(row_ptr, dtype=torch.int32).to(DEV)
    ci = torch.as_tensor(col_idx, dtype=torch.int32).to(DEV).contiguous()
    ob = torch.empty(bs, dtype=et, device=DEV)
    lse = torch.empty((plan.batch, plan.heads, plan.padded_len), dtype=torch.float32, device=DEV)
    vsa.vsa_block_sparse_attn_fwd(plan, qb, kb, vtb, rp, ci, uniform_k, ci.numel(), ob, lse)
    grads = [torch.full(bs, 3.0, dtype=et, device=DEV) for _ in range(3)]
    ws = torch.empty(vsa.vsa_block_sparse_attn_bwd_workspace_size(plan), dtype=torch.uint8,
                     device=DEV)
    vsa.vsa_block_sparse_attn_bwd(plan, qb, kb, vb, ob, dob, lse, rp, ci, uniform_k, ci.numel(),
                                  *grads, ws)
    raster = []
    for gb in grads:
        out = torch.empty(plan.raster_shape(), dtype=et, device=DEV)
        vsa.vsa_scatter(plan, gb, out)
        raster.append(out)
    torch.cuda.synchronize()
    return [t.cpu() for t in raster], [t.cpu() for t in grads]


def _check(name, got, want, blocked, oplan):
    for label, g, w, gb in zip(("dQ", "dK", "dV"), got, want, blocked):
        err = np.abs(g.double().numpy() - w)
        scale_max = max(1.0, np.abs(w).max())
        scale_mean = max(1.0, np.abs(w).mean())
        _say(f"    {name} {label}: max-abs {err.max():.3e} (|ref| max {np.abs(w).max():.2e}) "
             f"mean-abs {err.mean():.3e}")
        assert err.max() <= MAX_REL * scale_max and err.mean() <= MEAN_REL * scale_mean
        # pad rows of the blocked gradients are written as zero
        vol = oplan.block_volume
        gbh = gb.float().numpy()
        for beta, c in enumerate(oplan.block_counts()):
            assert np.all(gbh[:, :, beta * vol + c:(beta + 1) * vol] == 0)


@pytest.mark.parametrize("name,k", [("tiny", 4), ("tiny", 1), ("padded_tiny", 1),
                                    ("padded_tiny", 4), ("padded_tiny", 8)])
def test_backward_fed_oracle_map(name, k):
    wl = WORKLOADS[name]
    q, kk, v = make_qkv(wl)
    do = _dout(wl, torch.bfloat16)
    q64, k64, v64, do64 = (bf16_to_f64(t) for t in (q, kk, v, do))
    ref = oracle.vsa_reference(q64, k64, v64, wl.dit_seq_shape, wl.block_size, k)
    plan = _plan(wl, k)
    got, blocked = _run(plan, q, kk, v, do, None, ref["col_idx"], k)
    want = oracle.block_sparse_attention_bwd(q64, k64, v64, do64, ref["plan"], ref["row_ptr"],
                                             ref["col_idx"])
    _check(f"{name} k{k}", got, want, blocked, ref["plan"])


def test_backward_csr_with_zero_rows():
    wl = WORKLOADS["tile64_tiny"]
    q, kk, v = make_qkv(wl)
    do = _dout(wl, torch.bfloat16)
    rp, ci, _ = make_tile64_map(wl)
    assert np.any(np.diff(rp) == 0)
    plan = _plan(wl)
    oplan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size)
    got, blocked = _run(plan, q, kk, v, do, rp, ci, 0)
    want = oracle.block_sparse_attention_bwd(*(bf16_to_f64(t) for t in (q, kk, v, do)), oplan,
                                             rp, ci)
    _check("tile64_tiny", got, want, blocked, oplan)


def test_backward_repeated_ids_count_twice():
    wl = WORKLOADS["padded_tiny"]
    q, kk, v = make_qkv(wl)
    do = _dout(wl, torch.bfloat16)
    oplan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size)
    rows = wl.heads * oplan.num_blocks
    rng = np.random.default_rng(12)
    lists = [sorted(rng.choice(8, 3, replace=False).tolist()) for _ in range(rows)]
    for r in range(0, rows, 3):
        lists[r] = lists[r] + [lists[r][0]]            # one block twice
    rp = np.zeros(rows + 1, np.int64)
    rp[1:] = np.cumsum([len(x) for x in lists])
    ci = np.array(sum(lists, []), np.int32)
    plan = _plan(wl)
    got, blocked = _run(plan, q, kk, v, do, rp.astype(np.int32), ci, 0)
    want = oracle.block_sparse_attention_bwd(*(bf16_to_f64(t) for t in (q, kk, v, do)), oplan,
                                             rp, ci)
    _check("repeated ids", got, want, blocked, oplan)


def test_backward_fp16():
    wl = WORKLOADS["padded_tiny"]
    q, kk, v = make_qkv(wl, dtype=torch.float16)
    do = _dout(wl, torch.float16)
    q64, k64, v64, do64 = (bf16_to_f64(t) for t in (q, kk, v, do))
    ref = oracle.vsa_reference(q64, k64, v64, wl.dit_seq_shape, wl.block_size, 4)
    plan = _plan(wl, 4, vsa.VSA_DTYPE_FP16)
    got, blocked = _run(plan, q, kk, v, do, None, ref["col_idx"], 4)
    want = oracle.block_sparse_attention_bwd(q64, k64, v64, do64, ref["plan"], ref["row_ptr"],
                                             ref["col_idx"])
    _check("fp16", got, want, blocked, ref["plan"])


@pytest.mark.parametrize("name,heads", [("wan5b_k64", (0, 23)), ("wan5b_k64_h3", (0, 1, 2))])
def test_backward_full_size_whole_heads(name, heads):
    # the heads are independent: the oracle runs on whole heads of the
    # 27280-token layer (two of 24; all three of the 3-head shard, whose 360
    # rows and columns the balanced launches hand out with the tail split)
    # with the GPU's own selection for those heads
    wl = WORKLOADS[name]
    q, kk, v = make_qkv(wl)
    do = _dout(wl, torch.bfloat16)
    plan = _plan(wl)
    oplan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size)
    nb, k = oplan.num_blocks, wl.topk
    qb = torch.empty(plan.blocked_shape(), dtype=torch.bfloat16, device=DEV)
    kb = torch.empty_like(qb)
    qp = torch.empty(plan.pooled_shape(), dtype=torch.float32, device=DEV)
    kp = torch.empty_like(qp)
    vsa.vsa_gather(plan, vsa.VSA_ROLE_Q, q.to(DEV), qb, qp)
    vsa.vsa_gather(plan, vsa.VSA_ROLE_K, kk.to(DEV), kb, kp)
    col = torch.empty(plan.num_rows() * k, dtype=torch.int32, device=DEV)
    vsa.vsa_score_topk(plan, qp, kp, k, col)
    ci = col.cpu().numpy()
    got, blocked = _run(plan, q, kk, v, do, None, ci, k)
    for h in heads:
        hs = slice(h, h + 1)
        sub = ci.reshape(wl.heads, nb * k)[h]
        rp = np.arange(nb + 1, dtype=np.int64) * k
        want = oracle.block_sparse_attention_bwd(
            *(bf16_to_f64(t[:, :, hs]) for t in (q, kk, v, do)), oplan, rp, sub)
        for label, g, w in zip(("dQ", "dK", "dV"), got, want):
            err = np.abs(g[:, :, hs].double().numpy() - w)
            _say(f"    head {h} {label}: max-abs {err.max():.3e} (|ref| max "
                 f"{np.abs(w).max():.2e}) mean-abs {err.mean():.3e}")
            assert err.max() <= MAX_REL * max(1.0, np.abs(w).max())
            assert err.mean() <= MEAN_REL * max(1.0, np.abs(w).mean())
