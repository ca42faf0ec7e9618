"""GPU parity of the balanced attention launches (vsa_block_sparse_attn_fwd_ws
and vsa_block_sparse_attn_fwd_raster_ws): workgroups claim their rows from
per-XCD queues instead of taking a fixed row.  Every row the queues hand
out whole is computed exactly as before, so its O and LSE must equal the
plain launches bit for bit; the rows split in halves at the end of each
queue (the tail split, for launches of at most 256 rows per queue: each
half computed by its own workgroup over half of the row's entries, then
merged) sum in another order, so theirs must
agree to within the last bit of the element type (|a - b| <= 2^-7 max(1,
|b|)) and LSE to 1e-4.  The split rows are read from the workspace, where
each merge records its row; their number must be the launch's split slot
count.  The plain launches are compared with the oracle elsewhere; the
small cases here are also compared with the oracle directly.  Cases: every
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


# Byte offset of the claim order in the balanced launch's workspace (after
# the 256 bytes of row-queue counters).
_ORDER_OFFSET = 256


def _expected_claim_order(rp_h, nb):
    """The claim order of a block map's rows, written from its rule: the rows
    cut into 8 ranges as the queues cut them; in each range first the long
    rows (entry count times the range's row count at least 4 times the
    range's entries) in ascending order, then the others head by head (nb
    rows per head), by entry count descending (counts of 2047 and more count
    as 2047), equal counts ascending."""
    lens = np.diff(np.asarray(rp_h, np.int64))
    n = len(lens)
    per, rem = n // 8, n % 8
    out = []
    for x in range(8):
        start = x * (per + 1) if x < rem else rem * (per + 1) + (x - rem) * per
        count = per + (1 if x < rem else 0)
        rows = np.arange(start, start + count)
        total = int(lens[rows].sum()) if count else 0
        is_long = lens[rows] * count >= 4 * total
        out += [int(r) for r in rows[is_long]]
        rest = rows[~is_long]
        out += sorted((int(r) for r in rest), key=lambda r: (r // nb, -min(lens[r], 2047), r))
    return np.array(out, np.int64)


def _check_claim_order(ws, rp_h, nb, what):
    rows = len(rp_h) - 1
    got = ws[_ORDER_OFFSET:_ORDER_OFFSET + 4 * rows].cpu().view(torch.int32).numpy()
    exp = _expected_claim_order(rp_h, nb)
    assert np.array_equal(np.sort(got), np.arange(rows)), f"{what}: claim order is no permutation"
    bad = np.flatnonzero(got != exp)
    assert bad.size == 0, f"{what}: claim order differs at {bad.size} positions, first {bad[:5]}"
    _say(f"    {what}: claim order of {rows} rows as expected")


_SPLIT_PER_QUEUE = 16


def _a256(n):
    return (n + 255) & ~255


_SPLIT_MAX_QUEUE_ROWS = 256


def _split_slots(plan, strided):
    """Split slots of a launch, from the rule: the last min(count, 16) rows of
    each of the 8 queues; the queues cut the rows as the XCD ranges do, or
    (heads interleaved) queue x holds heads * ceil((nb - x) / 8) rows; none
    when the longest queue holds more than 256 rows."""
    heads, nb = plan.batch * plan.heads, plan.num_blocks
    if strided:
        counts = [(nb // 8 + (1 if x < nb % 8 else 0)) * heads for x in range(8)]
    else:
        per, rem = divmod(heads * nb, 8)
        counts = [per + (1 if x < rem else 0) for x in range(8)]
    if max(counts) > _SPLIT_MAX_QUEUE_ROWS:
        return 0
    return sum(min(_SPLIT_PER_QUEUE, c) for c in counts)


def _split_cap(plan):
    """Slots the workspace holds (either queue cut, no length limit)."""
    heads, nb = plan.batch * plan.heads, plan.num_blocks
    per, rem = divmod(heads * nb, 8)
    plain = sum(min(_SPLIT_PER_QUEUE, per + (1 if x < rem else 0)) for x in range(8))
    strided = sum(min(_SPLIT_PER_QUEUE, (nb // 8 + (1 if x < nb % 8 else 0)) * heads)
                  for x in range(8))
    return max(plain, strided)


def _split_rows(ws, plan, strided=False):
    """Rows the last launch on `ws` split (recorded by their merges), checked
    against the slot count of the rule."""
    rows = plan.num_rows()
    cap = _split_cap(plan)
    off = _ORDER_OFFSET + _a256(rows * 4) + _a256(cap * 4)
    got = ws[off:off + 4 * cap].cpu().view(torch.int32).numpy().astype(np.int64)
    n = _split_slots(plan, strided)
    used = got[:n]
    assert np.all((used >= 0) & (used < rows)), "split slot without a valid row"
    assert len(np.unique(used)) == n, "a row split twice"
    return used


def _expected_split_rows(order, n):
    """The rows the tail split takes, from its rule: in queue x (the rows
    xcd_remap gives XCD x, in claim order `order`), the last min(16, count)
    positions, slots numbered queue by queue in claim order; none when a
    queue holds more than 256 rows."""
    per, rem = divmod(n, 8)
    counts = [per + (1 if x < rem else 0) for x in range(8)]
    if max(counts) > _SPLIT_MAX_QUEUE_ROWS:
        return np.zeros(0, np.int64)
    out, start = [], 0
    for c in counts:
        s = min(_SPLIT_PER_QUEUE, c)
        out += [int(r) for r in order[start + c - s:start + c]]
        start += c
    return np.array(out, np.int64)


def _uniform_claim_order(wl):
    """Claim order of uniform rows (queues cut as xcd_remap cuts the rows),
    from its rule: within each head the blocks grouped by edge class (bit 2,
    1, 0: the block is the last along T, H, W, where the grid edge may cut
    it), the classes by descending valid-token count, then class number, the
    blocks of a class ascending."""
    (T, H, W), (bt, bh, bw) = wl.dit_seq_shape, wl.block_size
    nbt, nbh, nbw = -(-T // bt), -(-H // bh), -(-W // bw)
    keys = []
    for b in range(nbt * nbh * nbw):
        it, rem = divmod(b, nbh * nbw)
        ih, iw = divmod(rem, nbw)
        cls = (4 if it == nbt - 1 else 0) | (2 if ih == nbh - 1 else 0) | (1 if iw == nbw - 1 else 0)
        cnt = min(bt, T - it * bt) * min(bh, H - ih * bh) * min(bw, W - iw * bw)
        keys.append((-cnt, cls, b))
    head = [b for _, _, b in sorted(keys)]
    nb = len(head)
    heads = wl.batch * wl.heads
    return np.array([h * nb + head[p] for h in range(heads) for p in range(nb)], np.int64)


def _assert_same(a, b, what, split_rows=(), plan=None):
    """a: plain launch, b: balanced; blocked O [B,NH,Npad,D] and LSE [B,NH,Npad]."""
    oa, ob = a[0].view(torch.int16), b[0].view(torch.int16)
    la, lb = a[1], b[1]
    if len(split_rows) == 0:
        assert torch.equal(oa, ob), f"{what}: O differs"
        assert torch.equal(la, lb), f"{what}: LSE differs"
        return
    nb, heads = plan.num_blocks, plan.heads
    vol = plan.padded_len // nb
    mask = torch.zeros((plan.batch, heads, plan.padded_len), dtype=torch.bool)
    for r in split_rows:
        bb, rem = divmod(int(r), heads * nb)
        h, i = divmod(rem, nb)
        mask[bb, h, i * vol:(i + 1) * vol] = True
    mask = mask.to(oa.device)
    assert torch.equal(oa[~mask], ob[~mask]), f"{what}: O of a whole row differs"
    assert torch.equal(la[~mask], lb[~mask]), f"{what}: LSE of a whole row differs"
    fa, fb = a[0][mask].float(), b[0][mask].float()
    tol = 2.0 ** -7 * torch.clamp(fb.abs(), min=1.0)
    assert bool(((fa - fb).abs() <= tol).all()), f"{what}: O of a split row beyond the last bit"
    sa, sb = la[mask], lb[mask]
    assert torch.equal(torch.isinf(sa), torch.isinf(sb)), f"{what}: LSE -inf differs"
    fin = torch.isfinite(sb)
    if bool(fin.any()):
        assert float((sa[fin] - sb[fin]).abs().max()) <= 1e-4, f"{what}: LSE of a split row"
    _say(f"    {what}: {len(split_rows)} split rows within the last bit, the rest bitwise")


@pytest.mark.parametrize("name,dtype", [("wan5b_k64", vsa.VSA_DTYPE_BF16),
                                        ("wan5b_k64", vsa.VSA_DTYPE_FP16),
                                        ("wan13b_long", vsa.VSA_DTYPE_BF16),
                                        ("wan5b_k64_h3", vsa.VSA_DTYPE_BF16)])
def test_full_size_blocked_equals_plain_launch(name, dtype):
    wl = WORKLOADS[name]
    plan = _plan(wl, dtype=dtype)
    q, kk, v = make_qkv(wl, dtype=plan.torch_dtype())
    qb, kb, vb, qp, kp = _gather_all(plan, q, kk, v)
    col = _selection(plan, wl, qp, kp)
    ws = _junk_workspace(plan)
    plain, bal = _both_blocked(plan, qb, kb, vb, None, col, wl.topk, ws)
    strided = name == "wan13b_long"   # its heads' K and V outgrow the memory-side cache
    split = _split_rows(ws, plan, strided)
    _assert_same(plain, bal, name, split, plan)
    if not strided:
        # the split rows are those the rule names: the last 16 of each queue
        # in cost order (none for queues of more than 256 rows)
        want = _expected_split_rows(_uniform_claim_order(wl), plan.num_rows())
        assert np.array_equal(split, want), f"{name}: split rows differ from the rule"
    # a second call on the same workspace (its counters now hold the last
    # call's counts) gives the same result again, bit for bit
    again = _both_blocked(plan, qb, kb, vb, None, col, wl.topk, ws)[1]
    assert np.array_equal(_split_rows(ws, plan, strided), split)
    _assert_same(bal, again, f"{name} repeated")
    _say(f"    {name}: balanced == plain, {plan.num_rows()} rows")


def test_interleaved_heads_with_split_rows():
    """One head of the (81,30,52) layer (a 12-way head shard): its K and V
    times 8 outgrow the memory-side cache, so the queues interleave the
    head's blocks (queue x takes positions x, x+8, ... of the cost order: 74
    or 73 rows), and with at most 256 rows per queue the last 16 of each are
    split: 128 split slots numbered queue by queue over unequal queues."""
    wl = Workload("long_h1", (81, 30, 52), (4, 8, 8), 1, 1, 128, 64, seed=4)
    plan = _plan(wl)
    q, kk, v = make_qkv(wl)
    qb, kb, vb, qp, kp = _gather_all(plan, q, kk, v)
    col = _selection(plan, wl, qp, kp)
    ws = _junk_workspace(plan)
    plain, bal = _both_blocked(plan, qb, kb, vb, None, col, wl.topk, ws)
    split = _split_rows(ws, plan, strided=True)
    assert len(split) == 128
    _assert_same(plain, bal, "long_h1", split, plan)


@pytest.mark.parametrize("name", ["tiny", "vol128_b2", "vol192_padded", "vol64_3d"])
def test_small_volumes_equal_plain_launch_and_oracle(name):
    wl = WORKLOADS[name]
    plan = _plan(wl)
    q, kk, v = make_qkv(wl)
    qb, kb, vb, qp, kp = _gather_all(plan, q, kk, v)
    ref = oracle.vsa_reference(*(bf16_to_f64(t) for t in (q, kk, v)), wl.dit_seq_shape,
                               wl.block_size, wl.topk)
    col = torch.as_tensor(ref["col_idx"], dtype=torch.int32).to(DEV)
    ws = _junk_workspace(plan)
    plain, bal = _both_blocked(plan, qb, kb, vb, None, col, wl.topk, ws)
    _assert_same(plain, bal, name, _split_rows(ws, plan), plan)
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
    ws = _junk_workspace(plan)
    plain, bal = _both_blocked(plan, qb, kb, vb, rp, col, 0, ws)
    _assert_same(plain, bal, name, _split_rows(ws, plan), plan)
    _check_claim_order(ws, rp_h, plan.info["num_blocks"], name)


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
    col = torch.as_tensor(np.array([c for x in lists for c in x], np.int32)).to(DEV)
    ws = _junk_workspace(plan)
    plain, bal = _both_blocked(plan, qb, kb, vb, rp, col, 0, ws)
    _assert_same(plain, bal, "long rows", _split_rows(ws, plan), plan)
    _check_claim_order(ws, rp_h, nt, "long rows")


def test_claim_order_across_heads():
    """Queue ranges that start and end inside heads (5 heads of 300 tiles
    over 8 ranges), rows of every length from 0 to 300 in random order."""
    nt, heads = 300, 5
    wl = Workload("order_heads", (1, 1, nt * 64), (1, 1, 64), 1, heads, 128, None, seed=22)
    rng = np.random.default_rng(22)
    lists = []
    for h in range(heads):
        for i in range(nt):
            k = int(rng.integers(0, nt + 1))
            lists.append(sorted(rng.choice(nt, size=k, replace=False).tolist()))
    rp_h = np.zeros(len(lists) + 1, np.int64)
    rp_h[1:] = np.cumsum([len(x) for x in lists])
    plan = _plan(wl)
    q, kk, v = make_qkv(wl)
    qb, kb, vb, _, _ = _gather_all(plan, q, kk, v)
    rp = torch.as_tensor(rp_h.astype(np.int32)).to(DEV)
    col = torch.as_tensor(np.array([c for x in lists for c in x], np.int32)).to(DEV)
    ws = _junk_workspace(plan)
    plain, bal = _both_blocked(plan, qb, kb, vb, rp, col, 0, ws)
    split = _split_rows(ws, plan)
    _assert_same(plain, bal, "order across heads", split, plan)
    _check_claim_order(ws, rp_h, nt, "order across heads")
    # 1500 rows, queues of 188 and 187: the split rows are the last 16 of
    # each queue's claim order, slot by slot
    want = _expected_split_rows(_expected_claim_order(rp_h, nt), len(rp_h) - 1)
    assert len(want) == 128 and np.array_equal(split, want)


def test_claim_order_of_ranges_longer_than_the_length_cache():
    """Queue ranges of 4125 rows (33000 one-tile rows of one head), more than
    the 4096 row lengths the order kernel keeps in LDS, so it reads them from
    the map at every pass.  Seeded Q, K, V drawn on the device (the check is
    the claim order and the balanced launch equal to the plain one)."""
    nt = 33000
    wl = Workload("order_long", (1, 1, nt * 64), (1, 1, 64), 1, 1, 128, None, seed=23)
    rng = np.random.default_rng(23)
    lens = rng.integers(0, 9, size=nt)
    lists = [sorted(rng.choice(nt, size=int(k), replace=False).tolist()) for k in lens]
    rp_h = np.zeros(nt + 1, np.int64)
    rp_h[1:] = np.cumsum(lens)
    plan = _plan(wl)
    gen = torch.Generator(DEV).manual_seed(23)
    q, kk, v = (torch.randn((1, nt * 64, 1, 128), generator=gen, device=DEV).to(torch.bfloat16)
                for _ in range(3))
    qb, kb, vb, _, _ = _gather_all(plan, q, kk, v)
    rp = torch.as_tensor(rp_h.astype(np.int32)).to(DEV)
    col = torch.as_tensor(np.array([c for x in lists for c in x], np.int32)).to(DEV)
    ws = _junk_workspace(plan)
    plain, bal = _both_blocked(plan, qb, kb, vb, rp, col, 0, ws)
    _assert_same(plain, bal, "long ranges", _split_rows(ws, plan), plan)
    _check_claim_order(ws, rp_h, nt, "long ranges")


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
    split = _split_rows(ws, plan)
    # O is raster [B,S,NH,D]: the tokens of the split rows' query blocks may
    # differ in the last bit, every other token must be equal bit for bit
    lists = oracle.block_token_lists(oracle.make_plan(wl.seq_len, wl.dit_seq_shape,
                                                      wl.block_size))
    nb = plan.num_blocks
    mask = torch.zeros((plan.batch, wl.seq_len, plan.heads), dtype=torch.bool)
    for r in split:
        bb, rem = divmod(int(r), plan.heads * nb)
        h, i = divmod(rem, nb)
        mask[bb, torch.as_tensor(lists[i]), h] = True
    mask = mask.to(DEV)
    oa, ob = res[0][0], res[1][0]
    assert torch.equal(oa[~mask], ob[~mask]), f"raster gated={gated}: O of a whole row differs"
    fa, fb = oa[mask].float(), ob[mask].float()
    assert bool(((fa - fb).abs() <= 2.0 ** -7 * torch.clamp(fb.abs(), min=1.0)).all())
    # LSE keeps the blocked row order
    rows_mask = torch.zeros(plan.num_rows(), dtype=torch.bool)
    rows_mask[torch.as_tensor(split)] = True
    vol = plan.padded_len // nb
    tok_mask = rows_mask.repeat_interleave(vol).view(plan.batch, plan.heads, plan.padded_len)
    tok_mask = tok_mask.to(DEV)
    la, lb = res[0][1], res[1][1]
    assert torch.equal(la[~tok_mask], lb[~tok_mask])
    sa, sb = la[tok_mask], lb[tok_mask]
    assert torch.equal(torch.isinf(sa), torch.isinf(sb))
    fin = torch.isfinite(sb)
    if bool(fin.any()):
        assert float((sa[fin] - sb[fin]).abs().max()) <= 1e-4
    _say(f"    raster gated={gated}: {len(split)} split rows within the last bit, the rest bitwise")
