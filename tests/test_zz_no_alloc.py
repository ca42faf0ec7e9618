"""The no-allocation attention entry point against the workspace one.

vsa_block_sparse_attn_fwd_noalloc runs the balanced launch with its row
queues in the library's static device scratch; vsa_block_sparse_attn_fwd_ws
runs the same kernels with a caller workspace.  Both must write the same O
and LSE bit for bit, and match the oracle, on two calls in a row (the second
on a smaller input, after the first has left its counters in the scratch),
in uniform-k and in CSR mode.  The entry point allocates nothing and clears
its counters with a kernel, so it can be recorded into a HIP graph: replays,
with eager work and synchronisations between them, must equal eager calls on
the inputs the buffers hold at replay time.
"""
import numpy as np
import pytest
import torch

import block_sparse_video_tile_amd as vsa
import oracle
from tests.gpu_common import (DEV, _gather_all, _plan, _say, blocked_positions,
                              compare_all_rows, need_gpu)
from vsa_inputs import WORKLOADS, bf16_to_f64, make_qkv, make_tile64_map

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(request):
    need_gpu(request)


def _both(name):
    wl = WORKLOADS[name]
    q, kk, v = make_qkv(wl)
    plan = _plan(wl)
    oplan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size)
    if wl.topk:
        sc = oracle.block_scores(oracle.pool_blocks(bf16_to_f64(q), oplan),
                                 oracle.pool_blocks(bf16_to_f64(kk), oplan))
        sel, _ = oracle.select_topk(sc, wl.topk)
        rp, ci = oracle.selection_to_csr(sel)
        rp_dev, uk = None, wl.topk
    else:
        rp, ci, _ = make_tile64_map(wl)
        rp_dev, uk = torch.as_tensor(rp, dtype=torch.int32).to(DEV), 0
    ci_dev = torch.as_tensor(ci, dtype=torch.int32).to(DEV).contiguous()
    qb, kb, vb, _, _ = _gather_all(plan, q, kk, v)
    outs = []
    for noalloc in (False, True):
        ob = torch.full(plan.blocked_shape(), 7.0, dtype=torch.bfloat16, device=DEV)
        lse = torch.full((plan.batch, plan.heads, plan.padded_len), 7.0, dtype=torch.float32,
                         device=DEV)
        if noalloc:
            vsa.vsa_block_sparse_attn_fwd_noalloc(plan, qb, kb, vb, rp_dev, ci_dev, uk,
                                                  ci_dev.numel(), ob, lse)
        else:
            ws = torch.empty(vsa.vsa_attn_fwd_workspace_size(plan), dtype=torch.uint8,
                             device=DEV)
            vsa.vsa_block_sparse_attn_fwd_ws(plan, qb, kb, vb, rp_dev, ci_dev, uk,
                                             ci_dev.numel(), ob, ws, lse)
        torch.cuda.synchronize()
        outs.append((ob.cpu(), lse.cpu()))
    (o_ws, l_ws), (o_na, l_na) = outs
    assert torch.equal(o_ws, o_na), name
    assert torch.equal(l_ws, l_na), name
    # and the oracle, every row (float32 block loop on the same map)
    o32, l32 = oracle.block_sparse_attention_f32(q, kk, v, oplan, rp, ci)
    slots, toks, _ = blocked_positions(oplan)
    got = torch.zeros(plan.raster_shape(), dtype=torch.bfloat16)
    got[:, toks] = o_na[:, :, slots].permute(0, 2, 1, 3)
    compare_all_rows(f"{name} no-alloc vs float32 oracle", got, o32, l_na.numpy(), l32.numpy(),
                     oplan)


def test_noalloc_equals_workspace_entry_two_calls_second_smaller():
    for name in ("wan5b_k64", "padded_tiny"):
        _say(f"    call on {name}")
        _both(name)


def test_noalloc_equals_workspace_entry_csr_map():
    for name in ("tile64_csr", "tile64_tiny"):
        _say(f"    call on {name}")
        _both(name)


def _graph_case(name):
    wl = WORKLOADS[name]
    q, kk, v = make_qkv(wl)
    plan = _plan(wl)
    if wl.topk:
        oplan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size)
        sc = oracle.block_scores(oracle.pool_blocks(bf16_to_f64(q), oplan),
                                 oracle.pool_blocks(bf16_to_f64(kk), oplan))
        sel, _ = oracle.select_topk(sc, wl.topk)
        _, ci = oracle.selection_to_csr(sel)
        rp_dev, uk = None, wl.topk
    else:
        rp, ci, _ = make_tile64_map(wl)
        rp_dev, uk = torch.as_tensor(rp, dtype=torch.int32).to(DEV), 0
    ci_dev = torch.as_tensor(ci, dtype=torch.int32).to(DEV).contiguous()
    nnz = ci_dev.numel()
    qb, kb, vb, _, _ = _gather_all(plan, q, kk, v)
    # a second query tensor, copied into qb between replays
    q2 = (q.float() * -0.75).to(torch.bfloat16)
    qb2, _, _, _, _ = _gather_all(plan, q2, kk, v)

    def outputs():
        return (torch.full(plan.blocked_shape(), 7.0, dtype=torch.bfloat16, device=DEV),
                torch.full((plan.batch, plan.heads, plan.padded_len), 7.0, dtype=torch.float32,
                           device=DEV))

    def eager(qsrc):
        ob, lse = outputs()
        ws = torch.empty(vsa.vsa_attn_fwd_workspace_size(plan), dtype=torch.uint8, device=DEV)
        vsa.vsa_block_sparse_attn_fwd_ws(plan, qsrc, kb, vb, rp_dev, ci_dev, uk, nnz, ob, ws, lse)
        torch.cuda.synchronize()
        return ob.clone(), lse.clone()

    want1 = eager(qb.clone())
    want2 = eager(qb2)
    q_live = qb.clone()
    ob, lse = outputs()
    # one eager call first: the library's one-time scratch lookup stays out of the capture
    vsa.vsa_block_sparse_attn_fwd_noalloc(plan, q_live, kb, vb, rp_dev, ci_dev, uk, nnz, ob, lse)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        vsa.vsa_block_sparse_attn_fwd_noalloc(plan, q_live, kb, vb, rp_dev, ci_dev, uk, nnz, ob,
                                              lse)
    torch.cuda.synchronize()
    for rep, (src, want) in enumerate([(qb, want1), (qb2, want2), (qb, want1), (qb2, want2)]):
        q_live.copy_(src)          # eager work between the replays
        ob.fill_(3.0)
        lse.fill_(3.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(ob, want[0]), f"{name}: replay {rep} O"
        assert torch.equal(lse, want[1]), f"{name}: replay {rep} LSE"
    _say(f"    {name}: 4 graph replays equal the eager calls")
    del graph


def test_noalloc_replays_in_a_hip_graph():
    for name in ("padded_tiny", "tile64_tiny", "wan5b_k64"):
        _say(f"    graph on {name}")
        _graph_case(name)
