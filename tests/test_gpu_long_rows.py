"""GPU parity for block maps whose lists exceed one pass of the kernels'
LDS work lists (1024 entries; 768 in the 2-wave forward kernel that 64-token
tiles use): a 1-D layout of 1100 64-token tiles where a few
query rows list every tile and every other row lists tile 0 only, so those
rows (forward and dQ) and the column of tile 0 (dK, dV) are flattened in two
passes.  Oracle rows are computed for the long rows and a sample of the short
ones; the raster kernel must equal blocked attention followed by the scatter.
"""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_common import DEV, MAX_ABS, MEAN_ABS, _attend, _gather_all, _plan, _say, need_gpu
from tests.test_gpu_backward import MAX_REL, MEAN_REL, _dout, _run
from vsa_inputs import Workload, bf16_to_f64, make_qkv

import block_sparse_video_tile_amd as vsa

pytestmark = pytest.mark.gpu

NT = 1100
WL = Workload("long_rows", (1, 1, NT * 64), (1, 1, 64), 1, 1, 128, None, seed=21)
LONG = (3, 1099)


@pytest.fixture(autouse=True)
def _need_gpu(request):
    need_gpu(request)


def _map():
    lists = [[0] for _ in range(NT)]
    for r in LONG:
        lists[r] = list(range(NT))
    rp = np.zeros(NT + 1, np.int64)
    rp[1:] = np.cumsum([len(x) for x in lists])
    return rp.astype(np.int32), np.array(sum(lists, []), np.int32)


def test_forward_rows_longer_than_one_pass():
    q, kk, v = make_qkv(WL)
    rp, ci = _map()
    plan = _plan(WL)
    oplan = oracle.make_plan(WL.seq_len, WL.dit_seq_shape, WL.block_size)
    rows = list(LONG) + [0, 1, 500, 1098]
    ref_o, ref_l = oracle.block_sparse_attention(*(bf16_to_f64(t) for t in (q, kk, v)), oplan,
                                                 rp, ci, query_rows=rows)
    qb, kb, vb, _, _ = _gather_all(plan, q, kk, v)
    ob, lse = _attend(plan, qb, kb, vb, rp, ci)
    out = torch.empty(plan.raster_shape(), dtype=torch.bfloat16, device=DEV)
    vsa.vsa_scatter(plan, ob, out)
    # the raster kernel on the same map
    out_r = torch.full(plan.raster_shape(), 7.0, dtype=torch.bfloat16, device=DEV)
    lse_r = torch.empty_like(lse)
    vsa.vsa_block_sparse_attn_fwd_raster(plan, q.to(DEV), kk.to(DEV), v.to(DEV),
                                         torch.as_tensor(rp).to(DEV), torch.as_tensor(ci).to(DEV),
                                         0, ci.size, out_r, lse_r)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), out_r.cpu()) and torch.equal(lse.cpu(), lse_r.cpu())
    oh, lh = out.cpu().double().numpy(), lse.cpu().numpy()
    errs = []
    for r in rows:
        toks = slice(r * 64, (r + 1) * 64)
        errs.append(np.abs(oh[0, toks, 0] - ref_o[0, toks, 0]).reshape(-1))
        assert np.max(np.abs(lh[0, 0, toks] - ref_l[0, toks, 0])) <= 1e-3
    e = np.concatenate(errs)
    _say(f"    {len(rows)} rows: max-abs {e.max():.3e} mean-abs {e.mean():.3e}")
    assert e.max() <= MAX_ABS and e.mean() <= MEAN_ABS


def test_backward_lists_longer_than_one_pass():
    q, kk, v = make_qkv(WL)
    do = _dout(WL, torch.bfloat16)
    rp, ci = _map()
    plan = _plan(WL)
    oplan = oracle.make_plan(WL.seq_len, WL.dit_seq_shape, WL.block_size)
    got, blocked = _run(plan, q, kk, v, do, rp, ci, 0)
    want = oracle.block_sparse_attention_bwd(*(bf16_to_f64(t) for t in (q, kk, v, do)), oplan,
                                             rp.astype(np.int64), ci)
    for label, g, w in zip(("dQ", "dK", "dV"), got, want):
        err = np.abs(g.double().numpy() - w)
        _say(f"    {label}: max-abs {err.max():.3e} (|ref| max {np.abs(w).max():.2e}) "
             f"mean-abs {err.mean():.3e}")
        assert err.max() <= MAX_REL * max(1.0, np.abs(w).max())
        assert err.mean() <= MEAN_REL * max(1.0, np.abs(w).mean())
