"""Host-side tests of the C ABI: no GPU needed.

The library must load, export every function include/vsa.h declares, and
reject every malformed request with the documented status before any HIP
call (mirroring host-side route checks that need no device).
"""
import os

import numpy as np
import pytest

import block_sparse_video_tile_amd as vsa
import oracle
from tests.test_oracle_pins import _golden_fields, _line_fields

FAKE = 1 << 20   # a non-NULL address; every call below fails validation before using it


@pytest.fixture(scope="module")
def lib():
    return vsa.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = vsa.exported_symbols()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) <= set(vsa.__all__)


def test_status_strings(lib):
    assert vsa.vsa_status_string(0) == "VSA_OK"
    assert vsa.vsa_status_string(3) == "VSA_ERR_HIP"


def test_describe_matches_page_worked_example(golden_dir):
    page = _golden_fields(os.path.join(golden_dir, "routing_line.txt"))
    plan = vsa.vsa_plan(27280, (31, 22, 40), (4, 8, 8), batch=1, num_heads=24, topk=64)
    ours = _line_fields(vsa.vsa_plan_describe(plan))
    for key in page:
        if key != "checkpoint_mode":
            assert ours[key] == page[key], key


def test_describe_all_blocks_and_map_mode():
    p = vsa.vsa_plan(27280, (31, 22, 40), (4, 8, 8), topk=120)
    assert vsa.vsa_plan_describe(p).endswith("keep_ratio=100.0%, route=VSA_ALL_BLOCKS")
    p = vsa.vsa_plan(33280, (1, 1, 33280), (1, 1, 64), topk=0)
    assert vsa.vsa_plan_describe(p) == ("seq_len=33280, dit_seq_shape=(1, 1, 33280), "
                                        "block_size=(1, 1, 64), num_blocks=520")


def test_describe_small_buffer_is_rejected():
    p = vsa.vsa_plan(2048, (8, 16, 16), (4, 8, 8), topk=4)
    with pytest.raises(vsa.VsaError) as e:
        vsa.vsa_plan_describe(p, buf_len=10)
    assert e.value.status == vsa.VSA_ERR_INVALID_ARGUMENT


@pytest.mark.parametrize("shape,block", [((31, 22, 40), (4, 8, 8)), ((81, 30, 52), (4, 8, 8)),
                                         ((7, 13, 10), (4, 8, 8)), ((1, 1, 33280), (1, 1, 64)),
                                         ((5, 9, 17), (2, 8, 8)), ((3, 5, 70), (1, 4, 48))])
def test_plan_geometry_agrees_with_oracle(shape, block):
    s = int(np.prod(shape))
    p = vsa.vsa_plan(s, shape, block, batch=2, num_heads=3)
    o = oracle.make_plan(s, shape, block)
    assert p.info["block_grid"] == o.block_grid
    assert p.num_blocks == o.num_blocks
    assert p.padded_len == o.num_blocks * o.block_volume
    assert vsa.vsa_plan_block_counts(p) == o.block_counts().tolist()
    assert p.info["num_rows"] == 2 * 3 * o.num_blocks
    assert p.info["blocked_elems"] == 2 * 3 * p.padded_len * 128


@pytest.mark.parametrize("kwargs,status", [
    (dict(seq_len=27281), vsa.VSA_ERR_INVALID_ARGUMENT),             # S != T*H*W
    (dict(topk=121), vsa.VSA_ERR_INVALID_ARGUMENT),                  # topk > num_blocks
    (dict(topk=-1), vsa.VSA_ERR_INVALID_ARGUMENT),
    (dict(batch=0), vsa.VSA_ERR_INVALID_ARGUMENT),
    (dict(num_heads=0), vsa.VSA_ERR_INVALID_ARGUMENT),
    (dict(dit_seq_shape=(0, 22, 40), seq_len=0), vsa.VSA_ERR_INVALID_ARGUMENT),
    (dict(block_size=(4, 8, 0)), vsa.VSA_ERR_INVALID_ARGUMENT),
    (dict(head_dim=64), vsa.VSA_ERR_UNSUPPORTED),
    (dict(dtype=2), vsa.VSA_ERR_UNSUPPORTED),                        # neither bf16 nor fp16
    (dict(block_size=(2, 4, 4)), vsa.VSA_ERR_UNSUPPORTED),           # V = 32
    (dict(block_size=(4, 8, 16)), vsa.VSA_ERR_UNSUPPORTED),          # V = 512
    (dict(dit_seq_shape=(2**31 - 1,) * 3, seq_len=1), vsa.VSA_ERR_INVALID_ARGUMENT),  # T*H*W > 2^63
    (dict(block_size=(2**31 - 1,) * 3), vsa.VSA_ERR_UNSUPPORTED),    # block volume > 2^63
])
def test_plan_rejects(kwargs, status):
    args = dict(seq_len=27280, dit_seq_shape=(31, 22, 40), block_size=(4, 8, 8), batch=1,
                num_heads=24, head_dim=128, topk=64, dtype=vsa.VSA_DTYPE_BF16)
    args.update(kwargs)
    with pytest.raises(vsa.VsaError) as e:
        vsa.vsa_plan(**args)
    assert e.value.status == status
    assert vsa.vsa_last_error()            # a reason is always given


@pytest.fixture
def plan():
    return vsa.vsa_plan(2048, (8, 16, 16), (4, 8, 8), batch=1, num_heads=2, topk=4)


def _raw(fn_name, *args):
    return getattr(vsa.load_library(), fn_name)(*args)


def test_null_and_range_checks_before_any_device_call(plan):
    h = plan.handle
    bad = vsa.VSA_ERR_INVALID_ARGUMENT
    assert _raw("vsa_gather", h, 0, None, FAKE, None, None) == bad
    assert _raw("vsa_gather", h, 0, FAKE, None, None, None) == bad
    assert _raw("vsa_gather", h, 7, FAKE, FAKE, None, None) == bad          # unknown role
    assert _raw("vsa_scatter", h, None, FAKE, None) == bad
    assert _raw("vsa_score_topk", h, FAKE, FAKE, 0, FAKE, None, None) == bad   # topk < 1
    assert _raw("vsa_score_topk", h, FAKE, FAKE, 9, FAKE, None, None) == bad   # topk > nb
    assert _raw("vsa_score_topk", h, None, FAKE, 4, FAKE, None, None) == bad
    f = "vsa_block_sparse_attn_fwd"
    assert _raw(f, h, FAKE, FAKE, FAKE, None, FAKE, 9, 9 * 16, FAKE, None, None) == bad  # k > nb
    assert _raw(f, h, FAKE, FAKE, FAKE, None, FAKE, 4, 63, FAKE, None, None) == bad      # nnz short
    assert _raw(f, h, FAKE, FAKE, FAKE, FAKE, FAKE, 0, -1, FAKE, None, None) == bad      # nnz < 0
    assert _raw(f, h, FAKE, FAKE, FAKE, FAKE, None, 0, 5, FAKE, None, None) == bad       # col NULL
    assert _raw(f, h, None, FAKE, FAKE, None, FAKE, 4, 64, FAKE, None, None) == bad
    assert _raw(f, h, FAKE, FAKE, FAKE, None, FAKE, 4, 64, None, None, None) == bad
    assert _raw("vsa_plan_block_counts", h, None, 8) == bad


def test_forward_checks(plan):
    h = plan.handle
    bad = vsa.VSA_ERR_INVALID_ARGUMENT
    need = vsa.vsa_forward_workspace_size(plan)
    assert need > 0 and need % 256 == 0
    f = "vsa_forward"   # (plan, q, k, v, gate, out, ws, ws_bytes, col_out, lse, stream)
    assert _raw(f, h, FAKE, FAKE, FAKE, None, FAKE, FAKE, need - 1, None, None, None) == bad
    assert _raw(f, h, FAKE, FAKE, FAKE, None, FAKE, FAKE + 16, need, None, None, None) == bad
    assert _raw(f, h, FAKE, None, FAKE, None, FAKE, FAKE, need, None, None, None) == bad
    mp = vsa.vsa_plan(2048, (8, 16, 16), (4, 8, 8), topk=0)
    assert _raw(f, mp.handle, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1 << 30, None, None, None) == bad
    assert "map mode" in vsa.vsa_last_error()


def test_binding_rejects_host_tensors(plan):
    import torch
    x = torch.zeros(plan.raster_shape(), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        vsa.vsa_gather(plan, vsa.VSA_ROLE_Q, x, x)


def test_fp16_plan_is_accepted_and_sets_the_binding_dtype():
    import torch
    p16 = vsa.vsa_plan(27280, (31, 22, 40), (4, 8, 8), num_heads=24, topk=64,
                       dtype=vsa.VSA_DTYPE_FP16)
    assert p16.dtype == vsa.VSA_DTYPE_FP16 and p16.torch_dtype() == torch.float16
    p16b = vsa.vsa_plan(27280, (31, 22, 40), (4, 8, 8), num_heads=24, topk=64)
    assert p16b.torch_dtype() == torch.bfloat16
    # geometry does not depend on the element type
    assert p16.info == p16b.info


def test_coarse_branch_checks(plan):
    h = plan.handle
    bad = vsa.VSA_ERR_INVALID_ARGUMENT
    f = "vsa_compress_attn"   # (plan, q_pooled, k_pooled, v_pooled, o_coarse, stream)
    assert _raw(f, h, None, FAKE, FAKE, FAKE, None) == bad
    assert _raw(f, h, FAKE, FAKE, FAKE, None, None) == bad
    assert _raw(f, h, FAKE, FAKE + 4, FAKE, FAKE, None) == bad          # k_pooled alignment
    big = vsa.vsa_plan(1025 * 64, (1, 1, 1025 * 64), (1, 1, 64), topk=1)
    assert _raw(f, big.handle, FAKE, FAKE, FAKE, FAKE, None) == vsa.VSA_ERR_UNSUPPORTED
    g = "vsa_scatter_gated"   # (plan, o_blk, o_coarse, gate, o_raster, stream)
    assert _raw(g, h, FAKE, FAKE, None, FAKE, None) == bad
    assert _raw(g, h, FAKE, None, FAKE, FAKE, None) == bad
    assert _raw(g, h, FAKE, FAKE + 8, FAKE, FAKE, None) == bad          # o_coarse alignment
    # the workspace of vsa_forward holds pooled V and the coarse output too
    info = plan.info
    assert vsa.vsa_forward_workspace_size(plan) >= (4 * info["blocked_elems"] * 2
                                                    + 4 * info["pooled_elems"] * 4)


def test_backward_checks(plan):
    h = plan.handle
    bad = vsa.VSA_ERR_INVALID_ARGUMENT
    need = vsa.vsa_block_sparse_attn_bwd_workspace_size(plan)
    info = plan.info
    # rowsum and the transposed map (nb x nb per head)
    assert need >= (info["num_rows"] // info["num_blocks"]) * (
        info["padded_len"] * 4 + info["num_blocks"] ** 2 * 4)
    f = "vsa_block_sparse_attn_bwd"
    # (plan, q, k, v, o, do, lse, row_ptr, col, uniform_k, nnz, dq, dk, dv, ws, ws_bytes, stream)
    args = [h, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 4, 64, FAKE, FAKE, FAKE, FAKE,
            need, None]
    for idx in (1, 5, 6, 11, 14):                      # null inputs, outputs, workspace
        a = list(args)
        a[idx] = None
        assert _raw(f, *a) == bad
    a = list(args); a[9] = 9                            # uniform_k > nb
    assert _raw(f, *a) == bad
    a = list(args); a[10] = 63                          # nnz short for uniform rows
    assert _raw(f, *a) == bad
    a = list(args); a[15] = need - 1                    # short workspace
    assert _raw(f, *a) == bad
    a = list(args); a[14] = FAKE + 64                   # misaligned workspace
    assert _raw(f, *a) == bad
    big = vsa.vsa_plan(4097 * 64, (1, 1, 4097 * 64), (1, 1, 64), topk=1)
    a = list(args); a[0] = big.handle; a[9] = 1; a[10] = 4097; a[15] = 1 << 40
    assert _raw(f, *a) == vsa.VSA_ERR_UNSUPPORTED


def test_raster_attention_and_fused_forward_checks(plan):
    h = plan.handle
    bad = vsa.VSA_ERR_INVALID_ARGUMENT
    f = "vsa_block_sparse_attn_fwd_raster"
    # (plan, q, k, v, row_ptr, col, uniform_k, nnz, gate, o_coarse, o, lse, stream)
    n0 = (None, None)
    assert _raw(f, h, FAKE, FAKE, FAKE, None, FAKE, 9, 9 * 16, *n0, FAKE, None, None) == bad
    assert _raw(f, h, FAKE, FAKE, FAKE, None, FAKE, 4, 63, *n0, FAKE, None, None) == bad
    assert _raw(f, h, FAKE, FAKE, FAKE, FAKE, FAKE, 0, -1, *n0, FAKE, None, None) == bad
    assert _raw(f, h, FAKE, FAKE, FAKE, FAKE, None, 0, 5, *n0, FAKE, None, None) == bad
    assert _raw(f, h, FAKE, FAKE, None, None, FAKE, 4, 64, *n0, FAKE, None, None) == bad
    assert _raw(f, h, FAKE, FAKE, FAKE, None, FAKE, 4, 64, *n0, None, None, None) == bad
    # gate and o_coarse come together; o_coarse is read as float4
    assert _raw(f, h, FAKE, FAKE, FAKE, None, FAKE, 4, 64, FAKE, None, FAKE, None, None) == bad
    assert _raw(f, h, FAKE, FAKE, FAKE, None, FAKE, 4, 64, None, FAKE, FAKE, None, None) == bad
    assert _raw(f, h, FAKE, FAKE, FAKE, None, FAKE, 4, 64, FAKE, FAKE + 8, FAKE, None,
                None) == bad
    # descriptors hold a block's origin token in 21 bits
    n = 1 << 21
    big = vsa.vsa_plan(n, (1, 1, n), (1, 1, 64), topk=1)
    rows = big.num_rows()
    assert _raw(f, big.handle, FAKE, FAKE, FAKE, None, FAKE, 1, rows, None, None, FAKE, None,
                None) == vsa.VSA_ERR_UNSUPPORTED
    assert "2^21" in vsa.vsa_last_error()
    # the gather-free forward needs no blocked copies: pooled tensors and ids only
    need = vsa.vsa_forward_fused_workspace_size(plan)
    info = plan.info
    assert need % 256 == 0
    assert 4 * info["pooled_elems"] * 4 <= need < info["blocked_elems"] * 2 + _split_region_bytes(plan)
    g = "vsa_forward_fused"   # (plan, q, k, v, gate, out, ws, ws_bytes, col_out, lse, stream)
    assert _raw(g, h, FAKE, FAKE, FAKE, None, FAKE, FAKE, need - 1, None, None, None) == bad
    assert _raw(g, h, FAKE, FAKE, FAKE, None, FAKE, FAKE + 16, need, None, None, None) == bad
    assert _raw(g, h, FAKE, FAKE, None, None, FAKE, FAKE, need, None, None, None) == bad
    mp = vsa.vsa_plan(2048, (8, 16, 16), (4, 8, 8), topk=0)
    assert _raw(g, mp.handle, FAKE, FAKE, FAKE, None, FAKE, FAKE, 1 << 30, None, None,
                None) == bad
    # pooling alone: x_blk NULL needs `pooled`
    assert _raw("vsa_gather", h, 2, FAKE, None, None, None) == bad


def _a256(n):
    return (n + 255) // 256 * 256


def _split_region_bytes(p):
    """Tail-split part of a balanced launch's workspace, from its rule: the
    last min(rows of the queue, 16) rows of each of the 8 queues are split,
    under either queue cut; a counter and a row id per slot, and two halves
    of (O^T, m, l) per slot (waves x 66 x 64 fp32)."""
    rows, nb, heads = p.num_rows(), p.num_blocks, p.batch * p.heads
    per, rem = divmod(rows, 8)
    plain = rem * min(16, per + 1) + (8 - rem) * min(16, per)
    strided = sum(min(16, (nb // 8 + (x < nb % 8)) * heads) for x in range(8))
    slots = max(plain, strided)
    vol = p.padded_len // nb
    waves = 4 if vol == 64 else vol // 32
    return _a256(2 * _a256(slots * 4) + slots * 2 * waves * 66 * 64 * 4)


def test_balanced_attention_workspace_checks(plan):
    """The balanced (queued) attention launches: a fixed small workspace, the
    same argument checks as the plain entry points, and a null, short or
    misaligned workspace rejected before any device call."""
    h = plan.handle
    bad = vsa.VSA_ERR_INVALID_ARGUMENT
    need = vsa.vsa_attn_fwd_workspace_size(plan)
    # 9 row-queue counters (256 bytes), then one int32 per row for the claim
    # order of a block map, then the tail split: a counter and a row per
    # split slot, and two halves of (O^T, m, l) per slot (waves x 66 x 64
    # fp32), each part 256-byte aligned.  A queue splits min(its rows, 16).
    rows = plan.num_rows()
    assert need == 256 + _a256(rows * 4) + _split_region_bytes(plan)
    big = vsa.vsa_plan(27280, (31, 22, 40), (4, 8, 8), batch=1, num_heads=24, topk=64)
    # 2880 rows: 128 split slots of 8-wave halves
    assert vsa.vsa_attn_fwd_workspace_size(big) == 256 + 11520 + 1024 + 128 * 2 * 135168
    f = "vsa_block_sparse_attn_fwd_ws"
    # (plan, q, k, v, row_ptr, col, uniform_k, nnz, o, lse, ws, ws_bytes, stream)
    ok_args = (FAKE, FAKE, FAKE, None, FAKE, 4, rows * 4, FAKE, None)
    assert _raw(f, h, *ok_args, None, need, None) == bad
    assert "null workspace" in vsa.vsa_last_error()
    assert _raw(f, h, *ok_args, FAKE, need - 1, None) == bad
    assert _raw(f, h, *ok_args, FAKE + 16, need, None) == bad
    assert "256-byte" in vsa.vsa_last_error()
    assert _raw(f, h, FAKE, FAKE, FAKE, None, FAKE, 9, 9 * rows, FAKE, None, FAKE, need,
                None) == bad   # uniform_k > nb, as the plain entry point
    assert _raw(f, h, FAKE, FAKE, None, None, FAKE, 4, rows * 4, FAKE, None, FAKE, need,
                None) == bad
    g = "vsa_block_sparse_attn_fwd_raster_ws"
    # (plan, q, k, v, row_ptr, col, uniform_k, nnz, gate, o_coarse, o, lse, ws, ws_bytes, stream)
    r_args = (FAKE, FAKE, FAKE, None, FAKE, 4, rows * 4)
    assert _raw(g, h, *r_args, None, None, FAKE, None, None, need, None) == bad
    assert _raw(g, h, *r_args, None, None, FAKE, None, FAKE, need - 4, None) == bad
    assert _raw(g, h, *r_args, FAKE, None, FAKE, None, FAKE, need, None) == bad
    assert "gate and o_coarse" in vsa.vsa_last_error()
    # the layer entry points carry the queues in their own workspaces
    assert vsa.vsa_forward_workspace_size(plan) % 256 == 0
    assert vsa.vsa_forward_fused_workspace_size(plan) % 256 == 0


def test_alignment_checks_before_any_device_call(plan):
    """Element tensors are moved as 16-byte units and fp32/int32 arrays as
    4-byte words: an offset pointer is rejected before any device call."""
    h = plan.handle
    bad = vsa.VSA_ERR_INVALID_ARGUMENT
    m16, m4 = FAKE + 8, FAKE + 2
    rows = plan.num_rows()
    assert _raw("vsa_gather", h, 0, m16, FAKE, None, None) == bad
    assert _raw("vsa_gather", h, 0, FAKE, m16, None, None) == bad
    assert _raw("vsa_gather", h, 0, FAKE, None, m4, None) == bad
    assert _raw("vsa_scatter", h, m16, FAKE, None) == bad
    assert _raw("vsa_scatter", h, FAKE, m16, None) == bad
    assert _raw("vsa_score_topk", h, FAKE, FAKE + 4, 4, FAKE, None, None) == bad   # float4 reads
    assert _raw("vsa_score_topk", h, m4, FAKE, 4, FAKE, None, None) == bad
    assert _raw("vsa_score_topk", h, FAKE, FAKE, 4, m4, None, None) == bad
    assert _raw("vsa_score_topk", h, FAKE, FAKE, 4, FAKE, m4, None) == bad
    assert "aligned" in vsa.vsa_last_error()
    assert _raw("vsa_scatter_gated", h, FAKE, FAKE, m16, FAKE, None) == bad
    assert _raw("vsa_compress_attn", h, m4, FAKE, FAKE, FAKE, None) == bad
    # attention: (plan, q, k, v, row_ptr, col, uniform_k, nnz, o, lse, stream)
    f = "vsa_block_sparse_attn_fwd"
    for idx in (1, 2, 3, 8):
        a = [h, FAKE, FAKE, FAKE, None, FAKE, 4, rows * 4, FAKE, None, None]
        a[idx] = m16
        assert _raw(f, *a) == bad, idx
    assert _raw(f, h, FAKE, FAKE, FAKE, m4, FAKE, 0, 8, FAKE, None, None) == bad
    assert _raw(f, h, FAKE, FAKE, FAKE, None, m4, 4, rows * 4, FAKE, None, None) == bad
    assert _raw(f, h, FAKE, FAKE, FAKE, None, FAKE, 4, rows * 4, FAKE, m4, None) == bad
    assert "lse" in vsa.vsa_last_error()
    g = "vsa_block_sparse_attn_fwd_ws"
    assert _raw(g, h, m16, FAKE, FAKE, None, FAKE, 4, rows * 4, FAKE, None, FAKE, 256, None) == bad
    r = "vsa_block_sparse_attn_fwd_raster"
    assert _raw(r, h, FAKE, FAKE, FAKE, None, FAKE, 4, rows * 4, m16, FAKE, FAKE, None,
                None) == bad   # gate
    assert _raw(r, h, FAKE, m16, FAKE, None, FAKE, 4, rows * 4, None, None, FAKE, None,
                None) == bad
    rw = "vsa_block_sparse_attn_fwd_raster_ws"
    assert _raw(rw, h, FAKE, FAKE, FAKE, None, FAKE, 4, rows * 4, None, None, m16, None, FAKE,
                256, None) == bad
    # backward: (plan, q, k, v, o, do, lse, row_ptr, col, uk, nnz, dq, dk, dv, ws, ws_bytes, s)
    need = vsa.vsa_block_sparse_attn_bwd_workspace_size(plan)
    base = [h, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE, 4, 64, FAKE, FAKE, FAKE, FAKE,
            need, None]
    for idx, val in ((2, m16), (5, m16), (6, m4), (8, m4), (13, m16)):
        a = list(base)
        a[idx] = val
        assert _raw("vsa_block_sparse_attn_bwd", *a) == bad, idx
    # whole-path entry points: (plan, q, k, v, gate, out, ws, ws_bytes, col_out, lse, stream)
    for fn, size in (("vsa_forward", vsa.vsa_forward_workspace_size(plan)),
                     ("vsa_forward_fused", vsa.vsa_forward_fused_workspace_size(plan))):
        assert _raw(fn, h, FAKE, FAKE, m16, None, FAKE, FAKE, size, None, None, None) == bad
        assert _raw(fn, h, FAKE, FAKE, FAKE, m16, FAKE, FAKE, size, None, None, None) == bad
        assert _raw(fn, h, FAKE, FAKE, FAKE, None, FAKE, FAKE, size, m4, None, None) == bad
        assert _raw(fn, h, FAKE, FAKE, FAKE, None, FAKE, FAKE, size, None, m4, None) == bad


def test_measurement_kernel_checks():
    import ctypes
    bad = vsa.VSA_ERR_INVALID_ARGUMENT
    hz = ctypes.c_int64()
    f = "vsa_bench_mfma_peak"   # (num_workgroups, iters, timing, wall_clock_hz, stream)
    assert _raw(f, 0, 10, FAKE, ctypes.byref(hz), None) == bad
    assert _raw(f, (1 << 20) + 1, 10, FAKE, ctypes.byref(hz), None) == bad
    assert _raw(f, 4, 0, FAKE, ctypes.byref(hz), None) == bad
    assert _raw(f, 4, 10, None, ctypes.byref(hz), None) == bad
    assert _raw(f, 4, 10, FAKE, None, None) == bad
    assert _raw(f, 4, 10, FAKE + 4, ctypes.byref(hz), None) == bad
    g = "vsa_bench_hbm_copy"    # (src, dst, bytes, stream)
    assert _raw(g, None, FAKE, 64, None) == bad
    assert _raw(g, FAKE, FAKE, 0, None) == bad
    assert _raw(g, FAKE, FAKE, 40, None) == bad
    assert _raw(g, FAKE + 8, FAKE, 64, None) == bad
    assert "16-byte" in vsa.vsa_last_error()


def test_noalloc_attention_map_rows_limit():
    """The fixed scratch holds the longest-first order of at most 2^16 rows of
    a block map: a larger map-mode plan is UNSUPPORTED (uniform rows need no
    order and have no such limit)."""
    bad = vsa.VSA_ERR_UNSUPPORTED
    f = "vsa_block_sparse_attn_fwd_noalloc"
    big = vsa.vsa_plan(33280, (1, 1, 33280), (1, 1, 64), batch=1, num_heads=127, topk=0)
    assert big.num_rows() == 127 * 520 > 65536
    assert _raw(f, big.handle, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 10, FAKE, None, None) == bad
    assert "65536" in vsa.vsa_last_error()
    ok = vsa.vsa_plan(33280, (1, 1, 33280), (1, 1, 64), batch=1, num_heads=126, topk=0)
    assert ok.num_rows() == 65520 <= 65536


def test_noalloc_attention_checks(plan):
    """The no-allocation balanced launch: the argument checks of the workspace
    entry point, before any device call (no workspace argument to check)."""
    h = plan.handle
    bad = vsa.VSA_ERR_INVALID_ARGUMENT
    f = "vsa_block_sparse_attn_fwd_noalloc"
    # (plan, q, k, v, row_ptr, col, uniform_k, nnz, o, lse, stream)
    rows = plan.num_rows()
    assert _raw(f, h, None, FAKE, FAKE, None, FAKE, 4, rows * 4, FAKE, None, None) == bad
    assert _raw(f, h, FAKE, FAKE, FAKE, None, FAKE, 9, rows * 9, FAKE, None, None) == bad
    assert _raw(f, h, FAKE, FAKE, FAKE, None, FAKE, 4, rows * 4 - 1, FAKE, None, None) == bad
    assert _raw(f, h, FAKE, FAKE, FAKE, None, FAKE, 4, rows * 4, FAKE + 8, None, None) == bad
    assert _raw(f, h, FAKE, FAKE, FAKE, None, FAKE, 4, rows * 4, FAKE, FAKE + 2, None) == bad
    assert _raw(f, None, FAKE, FAKE, FAKE, None, FAKE, 4, rows * 4, FAKE, None, None) == bad
