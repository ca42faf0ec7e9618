"""GPU parity for the block volumes beyond 256: 128 (with two batches), 192
on a padded grid (edge blocks down to 10 valid tokens) and 3-D 64-token
blocks.  These run the 4-, 6- and 2-wave instantiations of the kernels.
Same tolerances as the other parity tests.
"""
import numpy as np
import pytest
import torch

import block_sparse_video_tile_amd as vsa
import oracle
from tests.gpu_common import (DEV, MARGIN, MAX_ABS, MEAN_ABS, _attend, _compare_rows,
                              _gather_all, _host, _plan, _say, need_gpu)
from tests.test_gpu_backward import MAX_REL, MEAN_REL, _dout, _run
from vsa_inputs import WORKLOADS, bf16_to_f64, make_qkv

pytestmark = pytest.mark.gpu

NAMES = ["vol128_b2", "vol192_padded", "vol64_3d"]


@pytest.fixture(autouse=True)
def _need_gpu(request):
    need_gpu(request)


@pytest.mark.parametrize("name", NAMES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_layout_pooling_and_attention(name, dtype):
    wl = WORKLOADS[name]
    q, kk, v = make_qkv(wl, dtype=dtype)
    plan = _plan(wl, dtype=vsa.VSA_DTYPE_FP16 if dtype == torch.float16 else vsa.VSA_DTYPE_BF16)
    q64, k64, v64 = (bf16_to_f64(t) for t in (q, kk, v))
    ref = oracle.vsa_reference(q64, k64, v64, wl.dit_seq_shape, wl.block_size, wl.topk)
    oplan = ref["plan"]
    qb, kb, vb, qp, kp = _gather_all(plan, q, kk, v)
    torch.cuda.synchronize()
    vol = oplan.block_volume
    qbh = qb.cpu()
    for beta, toks in enumerate(oracle.block_token_lists(oplan)):
        c = len(toks)
        assert torch.equal(qbh[:, :, beta * vol:beta * vol + c], q[:, toks].permute(0, 2, 1, 3))
        assert torch.all(qbh[:, :, beta * vol + c:(beta + 1) * vol].view(torch.int16) == 0)
    np.testing.assert_allclose(_host(qp), ref["qbar"], rtol=0, atol=1e-5)
    # selection on the device, exact outside near-ties
    col = torch.empty(plan.num_rows() * wl.topk, dtype=torch.int32, device=DEV)
    vsa.vsa_score_topk(plan, qp, kp, wl.topk, col)
    exact = ref["margin"] >= MARGIN
    assert np.array_equal(col.cpu().numpy().reshape(ref["sel"].shape)[exact], ref["sel"][exact])
    # attention fed the oracle's map, every row
    ob, lse = _attend(plan, qb, kb, vb, None, ref["col_idx"], uniform_k=wl.topk)
    mx, mean, lerr = _compare_rows(oplan, _host(ob), _host(lse), ref["out"], ref["lse"],
                                   range(plan.num_rows()), wl.heads, vol)
    _say(f"    {name} {dtype}: max-abs {mx:.3e} mean-abs {mean:.3e} lse {lerr:.2e}")
    assert mx <= MAX_ABS and mean <= MEAN_ABS and lerr <= 1e-3


@pytest.mark.parametrize("name", NAMES)
def test_backward(name):
    wl = WORKLOADS[name]
    q, kk, v = make_qkv(wl)
    do = _dout(wl, torch.bfloat16)
    q64, k64, v64, do64 = (bf16_to_f64(t) for t in (q, kk, v, do))
    ref = oracle.vsa_reference(q64, k64, v64, wl.dit_seq_shape, wl.block_size, wl.topk)
    plan = _plan(wl)
    got, blocked = _run(plan, q, kk, v, do, None, ref["col_idx"], wl.topk)
    want = oracle.block_sparse_attention_bwd(q64, k64, v64, do64, ref["plan"], ref["row_ptr"],
                                             ref["col_idx"])
    vol = ref["plan"].block_volume
    for label, g, w, gb in zip(("dQ", "dK", "dV"), got, want, blocked):
        err = np.abs(g.double().numpy() - w)
        _say(f"    {name} {label}: max-abs {err.max():.3e} (|ref| max {np.abs(w).max():.2e})")
        assert err.max() <= MAX_REL * max(1.0, np.abs(w).max())
        assert err.mean() <= MEAN_REL * max(1.0, np.abs(w).mean())
        gbh = gb.float().numpy()
        for beta, c in enumerate(ref["plan"].block_counts()):
            assert np.all(gbh[:, :, beta * vol + c:(beta + 1) * vol] == 0)
