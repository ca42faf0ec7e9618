"""GPU parity of the gate-compress (coarse) branch against the CPU oracle.

The branch pools values per tile, attends among the pooled tokens and adds
the gated coarse output of each token's block to the sparse output (the
oracle's readings R15 and R16).  The gate is a synthetic seeded tensor shaped
like Q: the learned to_gate_compress weights are not available.
"""
import numpy as np
import pytest
import torch

import block_sparse_video_tile_amd as vsa
import oracle
from tests.gpu_common import (DEV, MARGIN, MAX_ABS, MEAN_ABS, _gather_all, _host, _plan, _say,
                              check_selection_rows, compare_all_rows, need_gpu)
from vsa_inputs import WORKLOADS, bf16_to_f64, make_qkv

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(request):
    need_gpu(request)


def _gate(wl, dtype=torch.bfloat16, seed=77):
    g = torch.Generator("cpu").manual_seed(seed)
    x = torch.randn((wl.batch, wl.seq_len, wl.heads, wl.head_dim), generator=g) * 0.5
    return x.to(dtype).contiguous()


def _pooled_v(plan, v):
    vb = torch.empty(plan.blocked_vt_shape(), dtype=plan.torch_dtype(), device=DEV)
    vp = torch.empty(plan.pooled_shape(), dtype=torch.float32, device=DEV)
    vsa.vsa_gather(plan, vsa.VSA_ROLE_V, v.to(DEV), vb, vp)
    return vb, vp


@pytest.mark.parametrize("name", ["tiny", "padded_tiny", "wan5b_k64"])
def test_v_pooling_matches_oracle(name):
    wl = WORKLOADS[name]
    q, k, v = make_qkv(wl)
    plan = _plan(wl)
    oplan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size)
    vb, vp = _pooled_v(plan, v)
    np.testing.assert_allclose(_host(vp), oracle.pool_blocks(bf16_to_f64(v), oplan),
                               rtol=0, atol=1e-5)
    # the blocked V^T written alongside is the same as without pooling
    vb2 = torch.empty_like(vb)
    vsa.vsa_gather(plan, vsa.VSA_ROLE_V, v.to(DEV), vb2)
    assert torch.equal(vb, vb2)


@pytest.mark.parametrize("name", ["tiny", "padded_tiny", "wan5b_k64", "wan13b_long",
                                  "tile64_csr"])
def test_compress_attention_matches_oracle(name):
    wl = WORKLOADS[name]
    q, k, v = make_qkv(wl)
    plan = _plan(wl)
    oplan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size)
    _, _, _, qp, kp = _gather_all(plan, q, k, v)
    _, vp = _pooled_v(plan, v)
    oc = torch.empty(plan.pooled_shape(), dtype=torch.float32, device=DEV)
    vsa.vsa_compress_attn(plan, qp, kp, vp, oc)
    ref = oracle.compress_attention(oracle.pool_blocks(bf16_to_f64(q), oplan),
                                    oracle.pool_blocks(bf16_to_f64(k), oplan),
                                    oracle.pool_blocks(bf16_to_f64(v), oplan), wl.head_dim)
    err = np.abs(_host(oc) - ref)
    _say(f"    nb {oplan.num_blocks}: max-abs {err.max():.3e}")
    assert err.max() <= 1e-4 * max(1.0, np.abs(ref).max())


@pytest.mark.parametrize("name,dtype", [("padded_tiny", torch.bfloat16),
                                        ("padded_tiny", torch.float16),
                                        ("wan5b_k64", torch.bfloat16)])
def test_scatter_gated_matches_oracle(name, dtype):
    wl = WORKLOADS[name]
    plan = _plan(wl, dtype=vsa.VSA_DTYPE_FP16 if dtype == torch.float16 else vsa.VSA_DTYPE_BF16)
    oplan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size)
    g = torch.Generator("cpu").manual_seed(5)
    ob = torch.randn(plan.blocked_shape(), generator=g).to(dtype)
    oc = torch.randn(plan.pooled_shape(), generator=g, dtype=torch.float32)
    gate = _gate(wl, dtype)
    out = torch.full(plan.raster_shape(), 7.0, dtype=dtype, device=DEV)
    vsa.vsa_scatter_gated(plan, ob.to(DEV), oc.to(DEV), gate.to(DEV), out)
    # oracle: the blocked sparse output back in raster order, then R16
    vol = oplan.block_volume
    o_sparse = np.zeros((wl.batch, wl.seq_len, wl.heads, wl.head_dim))
    obh = ob.double().numpy()
    for beta, toks in enumerate(oracle.block_token_lists(oplan)):
        o_sparse[:, toks] = np.swapaxes(obh[:, :, beta * vol:beta * vol + len(toks)], 1, 2)
    want = oracle.gated_combine(o_sparse, oc.double().numpy(), gate.double().numpy(), oplan)
    got = out.cpu().double().numpy()
    # one rounding of an fp32 result to the element type
    ulp = 2.0 ** -8 if dtype == torch.bfloat16 else 2.0 ** -11
    assert np.all(np.abs(got - want) <= ulp * np.abs(want) + 1e-6)


def _gated_forward(wl, k, gate, dtype=torch.bfloat16):
    plan = _plan(wl, k, vsa.VSA_DTYPE_FP16 if dtype == torch.float16 else vsa.VSA_DTYPE_BF16)
    q, kk, v = make_qkv(wl, dtype=dtype)
    ws = torch.empty(vsa.vsa_forward_workspace_size(plan), dtype=torch.uint8, device=DEV)
    out = torch.empty(plan.raster_shape(), dtype=dtype, device=DEV)
    col = torch.empty(plan.num_rows() * k, dtype=torch.int32, device=DEV)
    vsa.vsa_forward(plan, q.to(DEV), kk.to(DEV), v.to(DEV), out, ws, col,
                    gate=None if gate is None else gate.to(DEV))
    torch.cuda.synchronize()
    return plan, q, kk, v, out.cpu(), col.cpu().numpy()


@pytest.mark.parametrize("name,dtype", [("tiny", torch.bfloat16), ("padded_tiny", torch.bfloat16),
                                        ("padded_tiny", torch.float16)])
def test_forward_gated_end_to_end(name, dtype):
    wl = WORKLOADS[name]
    gate = _gate(wl, dtype)
    plan, q, kk, v, out, col = _gated_forward(wl, wl.topk, gate, dtype)
    ref = oracle.vsa_gated_reference(bf16_to_f64(q), bf16_to_f64(kk), bf16_to_f64(v),
                                     bf16_to_f64(gate), wl.dit_seq_shape, wl.block_size, wl.topk)
    exact = ref["margin"] >= MARGIN
    assert np.array_equal(col.reshape(ref["sel"].shape)[exact], ref["sel"][exact])
    assert exact.all()
    err = np.abs(out.double().numpy() - ref["gated_out"])
    _say(f"    max-abs {err.max():.3e} mean-abs {err.mean():.3e}")
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS
    # without a gate the output is the sparse branch alone, bit for bit
    _, _, _, _, out_plain, _ = _gated_forward(wl, wl.topk, None, dtype)
    _, _, _, _, out_zero, _ = _gated_forward(wl, wl.topk, torch.zeros_like(gate), dtype)
    assert torch.equal(out_plain, out_zero)


def test_forward_gated_full_size_every_row():
    wl = WORKLOADS["wan5b_k64"]
    gate = _gate(wl)
    plan, q, kk, v, out, col = _gated_forward(wl, wl.topk, gate)
    oplan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size, wl.topk)
    q64, k64, v64 = bf16_to_f64(q), bf16_to_f64(kk), bf16_to_f64(v)
    qbar, kbar, vbar = (oracle.pool_blocks(x, oplan) for x in (q64, k64, v64))
    gsel = col.reshape(wl.batch, wl.heads, oplan.num_blocks, wl.topk)
    check_selection_rows(gsel, oracle.block_scores(qbar, kbar), wl.topk)
    rp, ci = oracle.selection_to_csr(gsel)
    # every row: the float32 block loop for the sparse branch, the float64
    # coarse branch and gated combination
    o_sparse, _ = oracle.block_sparse_attention_f32(q, kk, v, oplan, rp, ci)
    oc = oracle.compress_attention(qbar, kbar, vbar, wl.head_dim)
    want = oracle.gated_combine(o_sparse.double().numpy(), oc, bf16_to_f64(gate), oplan)
    compare_all_rows("gated, all rows vs oracle", out, want)
