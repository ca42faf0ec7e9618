"""GPU parity of the gather-free path against the CPU oracle: block-sparse
attention on raster [B,S,NH,D] tensors (tokens located by block index
arithmetic inside the kernel, O written straight to raster rows) and the fused
forward (block means read from the raster tensors; no gather or scatter
pass).  Besides the oracle comparison (same tolerances as the other parity
tests) the raster output is compared with the blocked kernel followed by the
scatter: bit for bit for block volumes below 256, where both run the same
interleaved step and form the same products in the same order; for 256-token
blocks the blocked kernel runs the alternating (two-group) pipeline, whose
row sums and key halves of blocks with at most 4 query groups are added in
another order, so there the two agree to within rounding of the last bit of
the element type (and the LSE to 1e-4).
"""
import numpy as np
import pytest
import torch

import block_sparse_video_tile_amd as vsa
import oracle
from tests.gpu_common import (DEV, MARGIN, MAX_ABS, MEAN_ABS, _attend, _gather_all, _plan, _say,
                              check_full_forward, need_gpu)
from tests.test_gpu_coarse import _gate
from vsa_inputs import WORKLOADS, bf16_to_f64, make_qkv, make_tile64_map

pytestmark = pytest.mark.gpu

CASES = [("tiny", 4), ("tiny", 1), ("padded_tiny", 1), ("padded_tiny", 4), ("padded_tiny", 8),
         ("vol128_b2", 5), ("vol192_padded", 5), ("vol64_3d", 6)]


@pytest.fixture(autouse=True)
def _need_gpu(request):
    need_gpu(request)


def _dt(dtype):
    return vsa.VSA_DTYPE_FP16 if dtype == torch.float16 else vsa.VSA_DTYPE_BF16


def _raster_attend(plan, q, k, v, row_ptr, col_idx, uniform_k, gate=None, oc=None):
    et = plan.torch_dtype()
    out = torch.full(plan.raster_shape(), 7.0, dtype=et, device=DEV)  # every row is overwritten
    lse = torch.empty((plan.batch, plan.heads, plan.padded_len), dtype=torch.float32, device=DEV)
    rp = None if row_ptr is None else torch.as_tensor(row_ptr, dtype=torch.int32).to(DEV)
    ci = torch.as_tensor(col_idx, dtype=torch.int32).to(DEV).contiguous()
    vsa.vsa_block_sparse_attn_fwd_raster(plan, q.to(DEV), k.to(DEV), v.to(DEV), rp, ci, uniform_k,
                                         ci.numel(), out, lse, gate=gate, o_coarse=oc)
    torch.cuda.synchronize()
    return out, lse


def _blocked_then_scatter(plan, q, k, v, row_ptr, col_idx, uniform_k):
    qb, kb, vb, _, _ = _gather_all(plan, q, k, v)
    ob, lse = _attend(plan, qb, kb, vb, row_ptr, col_idx, uniform_k)
    out = torch.empty(plan.raster_shape(), dtype=plan.torch_dtype(), device=DEV)
    vsa.vsa_scatter(plan, ob, out)
    torch.cuda.synchronize()
    return out.cpu(), lse.cpu()


def _same_as_blocked(plan, out, o2, lse=None, l2=None):
    """Raster vs blocked + scatter: bitwise below 256-token blocks, else to the
    last bit of the element type (relative 2^-7 of max(1, |x|)) and LSE 1e-4."""
    if plan.info["block_volume"] < 256:
        assert torch.equal(out, o2)
        if lse is not None:
            assert torch.equal(lse, l2)
        return
    a, b = out.double(), o2.double()
    assert torch.all((a - b).abs() <= 2.0 ** -7 * torch.clamp(b.abs(), min=1.0))
    if lse is not None:
        assert torch.equal(torch.isinf(lse), torch.isinf(l2))
        fin = torch.isfinite(l2)
        assert torch.all((lse[fin] - l2[fin]).abs() <= 1e-4)


def _check_oracle(oplan, out, lse, ref_out, ref_lse, label):
    err = np.abs(out.double().numpy() - ref_out)
    vol = oplan.block_volume
    lerr = 0.0
    lh = lse.numpy()
    for beta, toks in enumerate(oracle.block_token_lists(oplan)):
        c = len(toks)
        got = lh[:, :, beta * vol:beta * vol + c]
        want = np.swapaxes(ref_lse[:, toks, :], 1, 2)
        assert np.array_equal(np.isinf(got), np.isinf(want))
        fin = np.isfinite(want)
        if fin.any():
            lerr = max(lerr, float(np.abs(got[fin] - want[fin]).max()))
        assert np.all(np.isneginf(lh[:, :, beta * vol + c:(beta + 1) * vol]))
    _say(f"    {label}: max-abs {err.max():.3e} mean-abs {err.mean():.3e} lse {lerr:.2e}")
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS and lerr <= 1e-3


@pytest.mark.parametrize("name,k", CASES)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_raster_attention(name, k, dtype):
    wl = WORKLOADS[name]
    q, kk, v = make_qkv(wl, dtype=dtype)
    plan = _plan(wl, k, _dt(dtype))
    q64, k64, v64 = (bf16_to_f64(t) for t in (q, kk, v))
    ref = oracle.vsa_reference(q64, k64, v64, wl.dit_seq_shape, wl.block_size, k)
    out, lse = _raster_attend(plan, q, kk, v, None, ref["col_idx"], k)
    out, lse = out.cpu(), lse.cpu()
    _check_oracle(ref["plan"], out, lse, ref["out"], ref["lse"], f"{name} k{k} {dtype}")
    o2, l2 = _blocked_then_scatter(plan, q, kk, v, None, ref["col_idx"], k)
    _same_as_blocked(plan, out, o2, lse, l2)


@pytest.mark.parametrize("name,dtype", [("padded_tiny", torch.bfloat16),
                                        ("padded_tiny", torch.float16),
                                        ("vol128_b2", torch.bfloat16)])
def test_raster_attention_gated_epilogue_equals_gated_scatter(name, dtype):
    wl = WORKLOADS[name]
    q, kk, v = make_qkv(wl, dtype=dtype)
    gate = _gate(wl, dtype).to(DEV)
    plan = _plan(wl, dtype=_dt(dtype))
    ref = oracle.vsa_reference(*(bf16_to_f64(t) for t in (q, kk, v)), wl.dit_seq_shape,
                               wl.block_size, wl.topk)
    g = torch.Generator("cpu").manual_seed(5)
    oc = torch.randn(plan.pooled_shape(), generator=g, dtype=torch.float32).to(DEV)
    out, _ = _raster_attend(plan, q, kk, v, None, ref["col_idx"], wl.topk, gate, oc)
    qb, kb, vb, _, _ = _gather_all(plan, q, kk, v)
    ob, _ = _attend(plan, qb, kb, vb, None, ref["col_idx"], wl.topk)
    out2 = torch.empty(plan.raster_shape(), dtype=dtype, device=DEV)
    vsa.vsa_scatter_gated(plan, ob, oc, gate, out2)
    torch.cuda.synchronize()
    _same_as_blocked(plan, out.cpu(), out2.cpu())


def test_raster_attention_csr_with_zero_rows():
    wl = WORKLOADS["tile64_tiny"]
    q, kk, v = make_qkv(wl)
    rp, ci, _ = make_tile64_map(wl)
    assert np.any(np.diff(rp) == 0)
    plan = _plan(wl)
    oplan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size)
    q64, k64, v64 = (bf16_to_f64(t) for t in (q, kk, v))
    ref_o, ref_l = oracle.block_sparse_attention(q64, k64, v64, oplan, rp, ci)
    out, lse = _raster_attend(plan, q, kk, v, rp, ci, 0)
    out, lse = out.cpu(), lse.cpu()
    # rows without blocks: O = 0, LSE = -inf
    _check_oracle(oplan, out, lse, np.nan_to_num(ref_o), ref_l, "tile64_tiny CSR")
    o2, l2 = _blocked_then_scatter(plan, q, kk, v, rp, ci, 0)
    _same_as_blocked(plan, out, o2, lse, l2)


def test_raster_attention_full_size_csr_map():
    # 1-D 64-token tiles with the non-uniform map at full size (2-wave kernel)
    wl = WORKLOADS["tile64_csr"]
    q, kk, v = make_qkv(wl)
    rp, ci, _ = make_tile64_map(wl)
    plan = _plan(wl)
    out, lse = _raster_attend(plan, q, kk, v, rp, ci, 0)
    o2, l2 = _blocked_then_scatter(plan, q, kk, v, rp, ci, 0)
    _same_as_blocked(plan, out.cpu(), o2, lse.cpu(), l2)
    # sampled rows against the oracle
    oplan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size)
    nb = oplan.num_blocks
    rows = [0, 7, nb - 1, 5 * nb + 300, 23 * nb + 519, 11 * nb + 8]
    q64, k64, v64 = (bf16_to_f64(t) for t in (q, kk, v))
    ref_o, ref_l = oracle.block_sparse_attention(q64, k64, v64, oplan, rp, ci, query_rows=rows)
    lists = oracle.block_token_lists(oplan)
    oh = out.cpu()
    errs = []
    for r in rows:
        h, i = divmod(r, nb)
        toks = lists[i]
        errs.append(np.abs(oh[0, toks, h].double().numpy() - np.nan_to_num(ref_o[0, toks, h])))
    e = np.concatenate([x.reshape(-1) for x in errs])
    _say(f"    {len(rows)} rows: max-abs {e.max():.3e} mean-abs {e.mean():.3e}")
    assert e.max() <= MAX_ABS and e.mean() <= MEAN_ABS


def _forward(plan, q, k, v, gate=None, fused=False):
    size = (vsa.vsa_forward_fused_workspace_size if fused else vsa.vsa_forward_workspace_size)(plan)
    ws = torch.empty(size, dtype=torch.uint8, device=DEV)
    out = torch.empty(plan.raster_shape(), dtype=plan.torch_dtype(), device=DEV)
    col = torch.empty(plan.num_rows() * plan.topk, dtype=torch.int32, device=DEV)
    lse = torch.empty((plan.batch, plan.heads, plan.padded_len), dtype=torch.float32, device=DEV)
    vsa.vsa_forward(plan, q.to(DEV), k.to(DEV), v.to(DEV), out, ws, col, lse,
                    gate=None if gate is None else gate.to(DEV), fused=fused)
    torch.cuda.synchronize()
    return out.cpu(), col.cpu().numpy(), lse.cpu()


@pytest.mark.parametrize("name", ["tiny", "padded_tiny", "vol128_b2", "vol192_padded",
                                  "vol64_3d"])
def test_fused_forward(name):
    wl = WORKLOADS[name]
    q, kk, v = make_qkv(wl)
    plan = _plan(wl)
    out, col, lse = _forward(plan, q, kk, v, fused=True)
    ref = oracle.vsa_reference(*(bf16_to_f64(t) for t in (q, kk, v)), wl.dit_seq_shape,
                               wl.block_size, wl.topk)
    exact = ref["margin"] >= MARGIN
    assert exact.all()
    assert np.array_equal(col.reshape(ref["sel"].shape), ref["sel"])
    _check_oracle(ref["plan"], out, lse, ref["out"], ref["lse"], f"fused {name}")
    # the means are the gather's, so the map is the unfused path's, and the
    # output too (to the last bit for 256-token blocks, as above)
    o2, c2, l2 = _forward(plan, q, kk, v, fused=False)
    assert np.array_equal(col, c2)
    _same_as_blocked(plan, out, o2, lse, l2)


@pytest.mark.parametrize("name,dtype", [("tiny", torch.bfloat16), ("padded_tiny", torch.bfloat16),
                                        ("padded_tiny", torch.float16),
                                        ("vol192_padded", torch.bfloat16)])
def test_fused_forward_gated(name, dtype):
    wl = WORKLOADS[name]
    q, kk, v = make_qkv(wl, dtype=dtype)
    gate = _gate(wl, dtype)
    plan = _plan(wl, dtype=_dt(dtype))
    out, col, _ = _forward(plan, q, kk, v, gate, fused=True)
    ref = oracle.vsa_gated_reference(*(bf16_to_f64(t) for t in (q, kk, v, gate)),
                                     wl.dit_seq_shape, wl.block_size, wl.topk)
    assert (ref["margin"] >= MARGIN).all()
    assert np.array_equal(col.reshape(ref["sel"].shape), ref["sel"])
    err = np.abs(out.double().numpy() - ref["gated_out"])
    _say(f"    gated fused {name} {dtype}: max-abs {err.max():.3e} mean-abs {err.mean():.3e}")
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS


@pytest.mark.parametrize("name", ["wan5b_k64", "wan13b_long", "wan5b_k64_h3"])
def test_fused_forward_full_size_every_row(name):
    check_full_forward(name, fused=True)
