"""GPU parity of the balanced attention launches (vsa_block_sparse_attn_fwd_ws
and vsa_block_sparse_attn_fwd_raster_ws): workgroups claim their rows from
per-XCD queues instead of taking a fixed row, and every row is computed
exactly as before, so O and LSE must equal the plain launches bit for bit.
The plain launches are compared with the oracle elsewhere; one small case
here is also compared with the oracle directly.  Cases: every
workgroup size (2, 4, 6 and 8 waves), both element types, CSR maps with
empty rows and rows longer than one LDS list pass, raster inputs with and
without the gate, a workspace left full of junk, and repeated calls.
"""
import numpy as np
import pytest
import torch

import block_sparse_video_tile_amd as vsa
import oracle
from tests.gpu_common import (DEV, MAX_ABS, MEAN_ABS, _compare_rows, _gather_all, _host, _plan,
                              _say, need_gpu)
from vsa_inputs import WORKLOADS, Workload, bf16_to_f64, make_qkv, make_tile64_map

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(request):
    need_gpu(request)


def _junk_workspace(plan):
    """A workspace whose counters start far from zero: the launch must clear them."""
    n = vsa.vsa_attn_fwd_workspace_size(plan)
    return torch.full((n,), 0xAB, dtype=torch.uint8, device=DEV)


def _selection(plan, wl, qp, kp):
    col = torch.empty(plan.num_rows() * wl.topk, dtype=torch.int32, device=DEV)
    vsa.vsa_score_topk(plan, qp, kp, wl.topk, col)
    return col


def _both_blocked(plan, qb, kb, vb, rp, col, uk, ws):
    """Plain and balanced blocked launches on the same inputs (fresh outputs)."""
    outs = []
    for balanced in (False, True):
        ob = torch.full(plan.blocked_shape(), 3.0, dtype=plan.torch_dtype(), device=DEV)
        lse = torch.full((plan.batch, plan.heads, plan.padded_len), 5.0, dtype=torch.float32,
                         device=DEV)
        if balanced:
            vsa.vsa_block_sparse_attn_fwd_ws(plan, qb, kb, vb, rp, col, uk, col.numel(), ob, ws,
                                             lse)
        else:
            vsa.vsa_block_sparse_attn_fwd(plan, qb, kb, vb, rp, col, uk, col.numel(), ob, lse)
        outs.append((ob, lse))
    torch.cuda.synchronize()
    return outs


def _assert_same(a, b, what):
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)), f"{what}: O differs"
    assert torch.equal(a[1], b[1]), f"{what}: LSE differs"


@pytest.mark.parametrize("name,dtype", [("wan5b_k64", vsa.VSA_DTYPE_BF16),
                                        ("wan5b_k64", vsa.VSA_DTYPE_FP16),
                                        ("wan13b_long", vsa.VSA_DTYPE_BF16)])
def test_full_size_blocked_equals_plain_launch(name, dtype):
    wl = WORKLOADS[name]
    plan = _plan(wl, dtype=dtype)
    q, kk, v = make_qkv(wl, dtype=plan.torch_dtype())
    qb, kb, vb, qp, kp = _gather_all(plan, q, kk, v)
    col = _selection(plan, wl, qp, kp)
    ws = _junk_workspace(plan)
    plain, bal = _both_blocked(plan, qb, kb, vb, None, col, wl.topk, ws)
    _assert_same(plain, bal, name)
    # a second call on the same workspace (its counters now hold the last
    # call's counts) gives the same result again
    again = _both_blocked(plan, qb, kb, vb, None, col, wl.topk, ws)[1]
    _assert_same(plain, again, f"{name} repeated")
    _say(f"    {name}: balanced == plain, {plan.num_rows()} rows")


@pytest.mark.parametrize("name", ["tiny", "vol128_b2", "vol192_padded", "vol64_3d"])
def test_small_volumes_equal_plain_launch_and_oracle(name):
    wl = WORKLOADS[name]
    plan = _plan(wl)
    q, kk, v = make_qkv(wl)
    qb, kb, vb, qp, kp = _gather_all(plan, q, kk, v)
    ref = oracle.vsa_reference(*(bf16_to_f64(t) for t in (q, kk, v)), wl.dit_seq_shape,
                               wl.block_size, wl.topk)
    col = torch.as_tensor(ref["col_idx"], dtype=torch.int32).to(DEV)
    plain, bal = _both_blocked(plan, qb, kb, vb, None, col, wl.topk, _junk_workspace(plan))
    _assert_same(plain, bal, name)
    oplan = ref["plan"]
    mx, mean, lerr = _compare_rows(oplan, _host(bal[0]), _host(bal[1]), ref["out"], ref["lse"],
                                   range(plan.num_rows()), wl.heads, oplan.block_volume)
    _say(f"    {name}: max-abs {mx:.3e} mean-abs {mean:.3e} lse {lerr:.2e}")
    assert mx <= MAX_ABS and mean <= MEAN_ABS and lerr <= 1e-3


@pytest.mark.parametrize("name", ["tile64_csr", "tile64_csr_zero"])
def test_csr_maps_with_empty_rows(name):
    wl = WORKLOADS[name]
    plan = _plan(wl)
    q, kk, v = make_qkv(wl)
    qb, kb, vb, _, _ = _gather_all(plan, q, kk, v)
    rp_h, ci_h, _ = make_tile64_map(wl)
    rp = torch.as_tensor(rp_h, dtype=torch.int32).to(DEV)
    col = torch.as_tensor(ci_h, dtype=torch.int32).to(DEV)
    plain, bal = _both_blocked(plan, qb, kb, vb, rp, col, 0, _junk_workspace(plan))
    _assert_same(plain, bal, name)


def test_rows_longer_than_one_list_pass():
    nt = 1100
    wl = Workload("long_rows", (1, 1, nt * 64), (1, 1, 64), 1, 1, 128, None, seed=21)
    lists = [[0] for _ in range(nt)]
    for r in (3, 1099):
        lists[r] = list(range(nt))
    rp_h = np.zeros(nt + 1, np.int64)
    rp_h[1:] = np.cumsum([len(x) for x in lists])
    plan = _plan(wl)
    q, kk, v = make_qkv(wl)
    qb, kb, vb, _, _ = _gather_all(plan, q, kk, v)
    rp = torch.as_tensor(rp_h.astype(np.int32)).to(DEV)
    col = torch.as_tensor(np.array(sum(lists, []), np.int32)).to(DEV)
    plain, bal = _both_blocked(plan, qb, kb, vb, rp, col, 0, _junk_workspace(plan))
    _assert_same(plain, bal, "long rows")


@pytest.mark.parametrize("gated", [False, True])
def test_raster_equals_plain_raster_launch(gated):
    wl = WORKLOADS["wan5b_k64"]
    plan = _plan(wl)
    q, kk, v = (t.to(DEV) for t in make_qkv(wl))
    qp = torch.empty(plan.pooled_shape(), dtype=torch.float32, device=DEV)
    kp = torch.empty_like(qp)
    vsa.vsa_gather(plan, vsa.VSA_ROLE_Q, q, None, qp)
    vsa.vsa_gather(plan, vsa.VSA_ROLE_K, kk, None, kp)
    col = _selection(plan, wl, qp, kp)
    gate = oc = None
    if gated:
        vp = torch.empty_like(qp)
        vsa.vsa_gather(plan, vsa.VSA_ROLE_V, v, None, vp)
        oc = torch.empty_like(qp)
        vsa.vsa_compress_attn(plan, qp, kp, vp, oc)
        gen = torch.Generator("cpu").manual_seed(5)
        gate = (torch.randn(plan.raster_shape(), generator=gen) * 0.5).to(torch.bfloat16).to(DEV)
    ws = _junk_workspace(plan)
    res = []
    for balanced in (False, True):
        out = torch.full(plan.raster_shape(), 3.0, dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((plan.batch, plan.heads, plan.padded_len), dtype=torch.float32,
                          device=DEV)
        if balanced:
            vsa.vsa_block_sparse_attn_fwd_raster_ws(plan, q, kk, v, None, col, wl.topk, col.numel(),
                                                    out, ws, lse, gate=gate, o_coarse=oc)
        else:
            vsa.vsa_block_sparse_attn_fwd_raster(plan, q, kk, v, None, col, wl.topk, col.numel(),
                                                 out, lse, gate=gate, o_coarse=oc)
        res.append((out, lse))
    torch.cuda.synchronize()
    _assert_same(res[0], res[1], f"raster gated={gated}")
