"""GPU parity of the fp16 path against the same fp64 oracle.

The guide's "Verify routing and fallback" admits FP16 or BF16 tensors; the
fp16 plan runs the same kernels with fp16 MFMA operands, P and O rounded to
fp16.  The oracle takes the fp16 inputs exactly (every fp16 value is an fp64
value), and the tolerances are the same as for bf16.
"""
import numpy as np
import pytest
import torch

import block_sparse_video_tile_amd as vsa
import oracle
from tests.gpu_common import (DEV, MAX_ABS, MEAN_ABS, _attend, _compare_rows, _gather_all,
                              _host, _plan, _say, check_full_forward, need_gpu)
from vsa_inputs import WORKLOADS, bf16_to_f64 as to_f64, make_qkv, make_tile64_map

pytestmark = pytest.mark.gpu
F16 = vsa.VSA_DTYPE_FP16


@pytest.fixture(autouse=True)
def _need_gpu(request):
    need_gpu(request)


@pytest.mark.parametrize("name", ["tiny", "padded_tiny"])
def test_fp16_gather_scatter_and_pooling(name):
    wl = WORKLOADS[name]
    q, k, v = make_qkv(wl, dtype=torch.float16)
    plan = _plan(wl, dtype=F16)
    oplan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size)
    qb, kb, vb, qp, kp = _gather_all(plan, q, k, v)
    torch.cuda.synchronize()
    vol = oplan.block_volume
    qbh, vbh = qb.cpu(), vb.cpu()
    for beta, toks in enumerate(oracle.block_token_lists(oplan)):
        c = len(toks)
        assert torch.equal(qbh[:, :, beta * vol:beta * vol + c], q[:, toks].permute(0, 2, 1, 3))
        assert torch.all(qbh[:, :, beta * vol + c:(beta + 1) * vol].view(torch.int16) == 0)
        chunks = vbh[:, :, beta * (vol // 64):(beta + 1) * (vol // 64)]
        flat = chunks.permute(0, 1, 2, 4, 3).reshape(wl.batch, wl.heads, vol, wl.head_dim)
        assert torch.equal(flat[:, :, :c], v[:, toks].permute(0, 2, 1, 3))
    # block means of the exact fp16 values, accumulated in fp32
    for dev, x in ((qp, q), (kp, k)):
        np.testing.assert_allclose(_host(dev), oracle.pool_blocks(to_f64(x), oplan),
                                   rtol=0, atol=1e-5)
    out = torch.empty_like(q, device=DEV)
    vsa.vsa_scatter(plan, kb, out)
    torch.cuda.synchronize()
    assert torch.equal(out.cpu(), k)


@pytest.mark.parametrize("name,k", [("tiny", 4), ("tiny", 1), ("padded_tiny", 1),
                                    ("padded_tiny", 4)])
def test_fp16_attention_fed_oracle_map(name, k):
    wl = WORKLOADS[name]
    q, kk, v = make_qkv(wl, dtype=torch.float16)
    plan = _plan(wl, k, F16)
    ref = oracle.vsa_reference(to_f64(q), to_f64(kk), to_f64(v), wl.dit_seq_shape,
                               wl.block_size, k)
    qb, kb, vb, _, _ = _gather_all(plan, q, kk, v)
    ob, lse = _attend(plan, qb, kb, vb, None, ref["col_idx"], uniform_k=k)
    assert ob.dtype == torch.float16
    mx, mean, lerr = _compare_rows(ref["plan"], _host(ob), _host(lse), ref["out"], ref["lse"],
                                   range(plan.num_rows()), wl.heads, ref["plan"].block_volume)
    _say(f"    max-abs {mx:.3e} mean-abs {mean:.3e} lse {lerr:.2e}")
    assert mx <= MAX_ABS and mean <= MEAN_ABS and lerr <= 1e-3


def test_fp16_attention_csr_with_zero_rows():
    wl = WORKLOADS["tile64_tiny"]
    q, kk, v = make_qkv(wl, dtype=torch.float16)
    rp, ci, _ = make_tile64_map(wl)
    plan = _plan(wl, dtype=F16)
    oplan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size)
    ref_o, ref_l = oracle.block_sparse_attention(to_f64(q), to_f64(kk), to_f64(v), oplan, rp, ci)
    qb, kb, vb, _, _ = _gather_all(plan, q, kk, v)
    ob, lse = _attend(plan, qb, kb, vb, rp, ci)
    mx, mean, lerr = _compare_rows(oplan, _host(ob), _host(lse), ref_o, ref_l,
                                   range(plan.num_rows()), wl.heads, 64)
    _say(f"    max-abs {mx:.3e} mean-abs {mean:.3e} lse {lerr:.2e}")
    assert mx <= MAX_ABS and mean <= MEAN_ABS and lerr <= 1e-3


def test_fp16_full_size_forward_every_row():
    check_full_forward("wan5b_k64", dtype=F16)


def test_fp16_rejects_bf16_tensors():
    wl = WORKLOADS["tiny"]
    plan = _plan(wl, dtype=F16)
    x = torch.zeros(plan.raster_shape(), dtype=torch.bfloat16, device=DEV)
    xb = torch.empty(plan.blocked_shape(), dtype=torch.float16, device=DEV)
    with pytest.raises(ValueError):
        vsa.vsa_gather(plan, vsa.VSA_ROLE_Q, x, xb)
