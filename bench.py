"""Benchmark of the VSA hot path on one MI355X.

A step is one pass of the whole hot path over one layer's synthetic input
(inputs resident in HBM): gather Q, K (with block mean-pooling) and V into
block-major form, score the pooled blocks and pick the top-k per query block,
run the block-sparse attention, scatter O back to raster order.  Every stage is
a kernel of libvsa_amd.so launched through the C ABI on torch's current
stream; HIP events on that stream bracket each stage of every timed step.
The attention stage is the balanced launch (vsa_block_sparse_attn_fwd_ws:
workgroups claim rows from per-XCD queues; a one-block counter reset kernel
runs first and is inside the stage's time); --fixed-order times the launch
with one workgroup per row in a fixed order instead (same results).

Metric: effective TFLOP/s counting the selected blocks' valid tokens only
(4 * D * sum over query blocks i of c_i * sum_{j in row i} c_j, from the map
the step produced), divided by the whole step time; ms/layer is reported
alongside.  The attention kernel's own rate against the dense MFMA peak is the
roofline object, with the MFMA rate, engine clock and copy bandwidth measured
on the same machine beside the published figures (measure_denominators).
Unless --no-cpu-baseline is given, the step's block ids are checked against
the float64 oracle (map_check: near-tie rows counted) and the float32 CPU
oracle is timed over the same layer on the host's cores (cpu_baseline).

Default workload: the 27280-token (31, 22, 40) layer, block (4, 8, 8),
24 heads, head_dim 128, topk 64, bf16 -- the shape of the routing example in
the "FastVideo VSA" user guide ("Choose top-k").

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--no-cpu-baseline] [--cpu-seconds S]

Two helper modes serve the HBM traffic record of the attention kernel:
  python bench.py --copy-calibration MIB
      runs the library's plain device copy (vsa_bench_hbm_copy, hbm_copy_kernel)
      of MIB MiB a few times, so that rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE
      can be read for a kernel whose byte count is known;
  python bench.py --record-traffic FETCH.csv WRITE.csv CAL_FETCH.csv CAL_WRITE.csv
                  --cal-mib MIB [--workload NAME] [--traffic-json PATH]
      turns the four counter_collection.csv files (attention runs, then the
      calibration copy) into the JSON record that the default mode reads:
      bytes per attention launch = FETCH_SIZE and WRITE_SIZE per dispatch,
      each scaled by the ratio of the copy's known bytes to what the same
      counter read for it, tagged with the sha256 of the kernel source.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import block_sparse_video_tile_amd as vsa  # noqa: E402
from vsa_inputs import WORKLOADS, make_qkv, make_tile64_map  # noqa: E402

# MI355X published figures: dense bf16/fp16 MFMA 256 CUs x 2.4 GHz x 4096
# flop/clock = 2516.6 TFLOP/s ("2.5 PFLOP/s"), HBM3E 8 TB/s.
MFMA_16BIT_PEAK_TFLOPS = 2516.6
HBM_PEAK_GBS = 8000.0
MFMA_FLOPS_PER_INSTR = 32 * 32 * 16 * 2   # v_mfma_f32_32x32x16_bf16
COPY_KERNEL = "hbm_copy_kernel"

STAGES = ["gather_q", "gather_k", "gather_v", "score_topk", "attention", "scatter"]
GATED_STAGES = ["gather_q", "gather_k", "gather_v", "score_topk", "attention", "coarse",
                "scatter"]
# gather-free path: block means read from the raster tensors, raster attention
FUSED_STAGES = ["pool_q", "pool_k", "score_topk", "attention"]
FUSED_GATED_STAGES = ["pool_q", "pool_k", "score_topk", "pool_v", "coarse", "attention"]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def step_flops(plan, col_host, row_ptr_host, uniform_k):
    counts = np.asarray(vsa.vsa_plan_block_counts(plan), dtype=np.int64)
    nb = plan.num_blocks
    rows = plan.num_rows()
    if row_ptr_host is None:
        keys = counts[col_host.reshape(rows, uniform_k)].sum(axis=1)
        nnz = rows * uniform_k
    else:
        keys = np.zeros(rows, np.int64)
        cnt = np.diff(row_ptr_host)
        nz = np.nonzero(cnt)[0]
        sums = np.add.reduceat(counts[col_host], row_ptr_host[:-1][nz]) if len(nz) else []
        keys[nz] = sums
        nnz = int(row_ptr_host[-1])
    qc = np.tile(counts, rows // nb)
    f_valid = 4 * plan.head_dim * int(np.sum(qc * keys))
    f_nominal = 4 * plan.head_dim * plan.info["block_volume"] ** 2 * nnz
    return f_valid, f_nominal


def attention_source_digest():
    """sha256 over the sources the forward attention kernel is compiled from."""
    h = hashlib.sha256()
    for name in ("attention.hip", "attn_common.h"):
        with open(os.path.join(ROOT, "block_sparse_video_tile_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(path, workload, dtype, variant="blocked"):
    """HBM bytes per attention launch from the committed PMC record, or None.

    The record is only used when it was taken on this workload and on the
    attention kernel source as it is now (same sha256); otherwise the counters
    describe a different kernel and traffic is reported as null.
    """
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if (rec.get("workload") != workload or rec.get("dtype", "bf16") != dtype
            or rec.get("variant", "blocked") != variant
            or rec.get("kernel_source_sha256") != attention_source_digest()):
        return None
    return rec.get("bytes_per_launch")


def copy_calibration(mib, reps=5):
    """The library's plain device copy (vsa_bench_hbm_copy) of a known size,
    for counter calibration."""
    n = mib * (1 << 20)
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        vsa.vsa_bench_hbm_copy(src, dst, n)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    print(json.dumps({"copy_calibration_bytes_read": n, "bytes_written": n, "reps": reps,
                      "kernel": COPY_KERNEL}))


def measure_denominators(dev, mfma_iters=4000, copy_mib=2048, reps=3):
    """Roofline denominators measured on this machine.

    Dense bf16 MFMA rate: vsa_bench_mfma_peak with two 4-wave workgroups per
    CU (the attention kernel's two waves per SIMD); flops = waves x iters x 16
    x 32768 over the launch's HIP-event time, best of `reps`; the engine clock
    is each wave's shader-clock cycles over its wall-clock time, averaged.
    Copy bandwidth: vsa_bench_hbm_copy of `copy_mib` MiB, 2 x bytes over the
    event time, best of `reps`.
    """
    props = torch.cuda.get_device_properties(dev)
    wgs = 2 * props.multi_processor_count
    timing = torch.zeros(16 * wgs, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)
    vsa.vsa_bench_mfma_peak(wgs, 100, timing)          # warm-up
    best_tf, clocks = 0.0, []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        hz = vsa.vsa_bench_mfma_peak(wgs, mfma_iters, timing)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        flops = wgs * 4 * mfma_iters * 16 * MFMA_FLOPS_PER_INSTR
        best_tf = max(best_tf, flops / (ms * 1e-3) / 1e12)
        t = timing.view(-1, 4).cpu().numpy().astype(np.float64)
        clocks.append(float(np.mean(t[:, 0] / (t[:, 1] / hz))) / 1e9)
    n = copy_mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(7)
    dst = torch.empty_like(src)
    vsa.vsa_bench_hbm_copy(src, dst, n)
    best_gbs = 0.0
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        vsa.vsa_bench_hbm_copy(src, dst, n)
        e1.record(stream)
        torch.cuda.synchronize()
        best_gbs = max(best_gbs, 2 * n / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del src, dst
    return {"mfma_bf16_tflops": round(best_tf, 1), "mfma_clock_ghz": round(float(np.mean(clocks)), 3),
            "mfma_loop": f"{wgs} workgroups x 4 waves x {mfma_iters} x 16 "
                         "v_mfma_f32_32x32x16_bf16, best of 3",
            "hbm_copy_gbs": round(best_gbs, 1),
            "hbm_copy": f"{copy_mib} MiB device copy (read + write), best of 3",
            "compute_units": props.multi_processor_count}


def _counter_means(path, name_filter):
    """Mean Counter_Value per counter over the dispatches whose kernel name matches."""
    import csv
    import collections
    acc = collections.defaultdict(list)
    with open(path) as f:
        for row in csv.DictReader(f):
            if name_filter in row["Kernel_Name"]:
                acc[row["Counter_Name"]].append(float(row["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def _short_kernel_name(name):
    """Kernel name without namespace and argument list, template arguments kept."""
    if name.startswith("void "):
        name = name[5:]
    return name.replace("vsa::(anonymous namespace)::", "").split("(")[0]


def _calibration_factors(cal_fetch_csv, cal_write_csv, cal_mib):
    cal_bytes = cal_mib * (1 << 20)
    f = _counter_means(cal_fetch_csv, COPY_KERNEL)["FETCH_SIZE"][0]
    w = _counter_means(cal_write_csv, COPY_KERNEL)["WRITE_SIZE"][0]
    return cal_bytes / (f * 1024.0), cal_bytes / (w * 1024.0)


def stage_traffic(args):
    """HBM bytes and rates of every kernel of a layer run (markdown rows).

    FETCH_SIZE and WRITE_SIZE per dispatch (KiB) of each kernel, scaled by the
    calibration copy's factors, against the mean duration of the same kernel in
    a --kernel-trace --stats run of the same command; the algorithmic bytes of
    the gathers and the scatter (B*S*NH*D*2 read, B*NH*Npad*D*2 written, or the
    reverse) are given for the 27280-token layer.
    """
    import csv
    import collections
    fetch_csv, write_csv, cal_fetch_csv, cal_write_csv, stats_csv = args.stage_traffic
    kf, kw = _calibration_factors(cal_fetch_csv, cal_write_csv, args.cal_mib)
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    for path, counter in ((fetch_csv, "FETCH_SIZE"), (write_csv, "WRITE_SIZE")):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row["Counter_Name"] == counter:
                    vals[_short_kernel_name(row["Kernel_Name"])][counter].append(
                        float(row["Counter_Value"]))
    dur = {}
    with open(stats_csv) as f:
        for row in csv.DictReader(f):
            dur[_short_kernel_name(row["Name"])] = float(row["AverageNs"]) * 1e-9
    print("| kernel | mean duration (us) | fetched (MB) | written (MB) | measured GB/s | % of 8 TB/s |")
    print("|---|---|---|---|---|---|")
    for name, c in sorted(vals.items()):
        if name not in dur or not c.get("FETCH_SIZE") or not c.get("WRITE_SIZE"):
            continue
        fb = np.mean(c["FETCH_SIZE"]) * 1024.0 * kf
        wb = np.mean(c["WRITE_SIZE"]) * 1024.0 * kw
        rate = (fb + wb) / dur[name] / 1e9
        print(f"| {name} | {dur[name] * 1e6:.1f} | {fb / 1e6:.1f} | {wb / 1e6:.1f} | {rate:.0f} | "
              f"{100 * rate / HBM_PEAK_GBS:.1f} |")


def mfma_utilisation(args):
    """MFMA busy fraction and sustained clock of the attention kernel.

    From a rocprofv3 --pmc GRBM_GUI_ACTIVE SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_MFMA
    --kernel-trace run: GRBM_GUI_ACTIVE is summed over the 8 XCDs, so the
    kernel's cycles are GRBM_GUI_ACTIVE / 8; SQ_VALU_MFMA_BUSY_CYCLES is summed
    over the 1024 SIMDs.  busy = MFMA busy cycles / (cycles * 1024); clock =
    cycles / duration (duration from the same run's kernel trace).
    """
    import csv
    import collections
    pmc_csv, trace_csv = args.mfma_util
    per = collections.defaultdict(dict)
    names = {}
    with open(pmc_csv) as f:
        for row in csv.DictReader(f):
            if "attn_fwd_kernel" in row["Kernel_Name"]:
                per[row["Dispatch_Id"]][row["Counter_Name"]] = float(row["Counter_Value"])
                names[row["Dispatch_Id"]] = _short_kernel_name(row["Kernel_Name"])
    durs = {}
    with open(trace_csv) as f:
        for row in csv.DictReader(f):
            durs[row["Dispatch_Id"]] = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) * 1e-9
    rows = []
    for d, c in per.items():
        cycles = c["GRBM_GUI_ACTIVE"] / 8
        busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * 1024)
        rows.append((busy, cycles / durs[d] / 1e9, c["SQ_VALU_MFMA_BUSY_CYCLES"] / c["SQ_INSTS_MFMA"],
                     durs[d] * 1e3, c["SQ_INSTS_MFMA"]))
    r = np.array(rows)
    print(json.dumps({"kernel": sorted(set(names.values())), "dispatches": len(rows),
                      "mfma_busy": round(float(r[:, 0].mean()), 4),
                      "clock_ghz": round(float(r[:, 1].mean()), 3),
                      "busy_cycles_per_mfma": round(float(r[:, 2].mean()), 2),
                      "duration_ms": round(float(r[:, 3].mean()), 3),
                      "mfma_instructions": float(r[:, 4].mean())}))


def record_traffic(args):
    fetch_csv, write_csv, cal_fetch_csv, cal_write_csv = args.record_traffic
    cal_bytes = args.cal_mib * (1 << 20)
    out = {}
    for label, att_csv, cal_csv, counter in (("fetch", fetch_csv, cal_fetch_csv, "FETCH_SIZE"),
                                              ("write", write_csv, cal_write_csv, "WRITE_SIZE")):
        att, n_att = _counter_means(att_csv, "attn_fwd_kernel")[counter]
        cal, n_cal = _counter_means(cal_csv, COPY_KERNEL)[counter]
        factor = cal_bytes / (cal * 1024.0)   # counter reads KiB
        out[label] = {"counter": counter, "kib_per_dispatch": att, "dispatches": n_att,
                      "calibration_kib": cal, "calibration_dispatches": n_cal,
                      "calibration_factor": factor, "bytes_per_launch": att * 1024.0 * factor}
    rec = {"workload": args.workload, "dtype": args.dtype,
           "variant": "raster" if args.fused else "blocked",
           "kernel_source_sha256": attention_source_digest(),
           "bytes_per_launch": out["fetch"]["bytes_per_launch"] + out["write"]["bytes_per_launch"],
           "fetch": out["fetch"], "write": out["write"], "calibration_copy_bytes": cal_bytes}
    with open(args.traffic_json, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def _cpu_model():
    """The host CPU's model name (lscpu, else /proc/cpuinfo)."""
    import subprocess
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except (OSError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, q, k, v, budget_s):
    """The float32 CPU oracle over one layer of the same workload.

    vsa_reference_f32 (pool, score, top-k, then the per-row block loop: one
    product against the row's concatenated valid keys, softmax, one product
    with the values) in torch-CPU ops on the host's cores; map workloads run
    block_sparse_attention_f32 on the given map.  One head is run first as a
    warm-up; then the whole layer is timed if the warm-up says it fits in
    about `budget_s`, else as many whole heads as fit, and the layer time is
    extrapolated from them (said in `sample`).  value = F_valid of the rows
    computed (the CPU's own map) / their time.
    """
    import oracle
    threads = torch.get_num_threads()
    plan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size, wl.topk)

    def run(heads):
        if wl.topk:
            ref = oracle.vsa_reference_f32(q, k, v, wl.dit_seq_shape, wl.block_size, wl.topk,
                                           heads=heads)
            return ref["row_ptr"], ref["col_idx"]
        rp, ci, _ = make_tile64_map(wl)
        oracle.block_sparse_attention_f32(q, k, v, plan, rp, ci, heads=heads)
        return rp, ci

    t0 = time.perf_counter()
    run([0])
    t_head = time.perf_counter() - t0
    n = wl.heads if t_head * wl.heads <= budget_s else max(1, int(budget_s / t_head))
    t0 = time.perf_counter()
    rp, ci = run(list(range(n)))
    t = time.perf_counter() - t0
    nb = plan.num_blocks
    rows = n * nb   # batch 1: the first n heads' rows
    rp = np.asarray(rp, np.int64)
    flops = oracle.valid_flops(plan, rp[:rows + 1], np.asarray(ci, np.int64)[:rp[rows]],
                               wl.head_dim)
    s_layer = t * wl.heads / n
    return {"value": round(flops / t / 1e12, 4), "unit": "TFLOP/s", "cores": int(threads),
            "kind": "oracle", "s_per_layer": round(s_layer, 2),
            "sample": (f"float32 torch-CPU oracle, whole path (pool, score, top-k, block-loop "
                       f"attention), {'the whole layer' if n == wl.heads else f'{n} of {wl.heads} heads, layer time extrapolated'}"
                       f" ({wl.name}), {t:.1f} s after a one-head warm-up; {threads} threads"),
            "nproc": os.cpu_count(), "cpu_model": _cpu_model()}


def map_check(wl, q, k, col_host):
    """The step's block ids against the float64 oracle's selection: rows equal
    bit for bit outside near-ties (k-th vs (k+1)-th score gap < 1e-3), and
    the number of near-tie rows excluded from that check."""
    import oracle
    plan = oracle.make_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size, wl.topk)
    q64, k64 = (x.to(torch.float64).numpy() for x in (q, k))
    sc = oracle.block_scores(oracle.pool_blocks(q64, plan), oracle.pool_blocks(k64, plan))
    sel, margin = oracle.select_topk(sc, wl.topk)
    got = col_host.reshape(sel.shape)
    exact = margin >= 1e-3
    same = np.all(got == sel, axis=-1)
    return {"rows": int(exact.size), "bit_exact": int((same & exact).sum()),
            "near_tie_excluded": int((~exact).sum()),
            "mismatch_outside_near_ties": int((~same & exact).sum())}


def bench_backward(args, wl, plan, elem, dq, dk, dv):
    """Time vsa_block_sparse_attn_bwd on the workload (the forward runs once for O and LSE).

    Work counted: the five products of the attention backward (S recompute,
    dP, dV, dK, dQ) on valid (query, key) pairs of the selected blocks, i.e.
    2.5 x the forward's F_valid.
    """
    dev = dq.device
    bs = plan.blocked_shape()
    qb, kb, vb, ob, dob = (torch.empty(bs, dtype=elem, device=dev) for _ in range(5))
    vtb = torch.empty(plan.blocked_vt_shape(), dtype=elem, device=dev)
    qp = torch.empty(plan.pooled_shape(), dtype=torch.float32, device=dev)
    kp = torch.empty_like(qp)
    vsa.vsa_gather(plan, vsa.VSA_ROLE_Q, dq, qb, qp)
    vsa.vsa_gather(plan, vsa.VSA_ROLE_K, dk, kb, kp)
    vsa.vsa_gather(plan, vsa.VSA_ROLE_K, dv, vb)
    vsa.vsa_gather(plan, vsa.VSA_ROLE_V, dv, vtb)
    gen = torch.Generator("cpu").manual_seed(41)
    vsa.vsa_gather(plan, vsa.VSA_ROLE_Q,
                   torch.randn(plan.raster_shape(), generator=gen).to(elem).to(dev), dob)
    col = torch.empty(plan.num_rows() * wl.topk, dtype=torch.int32, device=dev)
    vsa.vsa_score_topk(plan, qp, kp, wl.topk, col)
    lse = torch.empty((plan.batch, plan.heads, plan.padded_len), dtype=torch.float32, device=dev)
    vsa.vsa_block_sparse_attn_fwd(plan, qb, kb, vtb, None, col, wl.topk, col.numel(), ob, lse)
    grads = [torch.empty(bs, dtype=elem, device=dev) for _ in range(3)]
    ws = torch.empty(vsa.vsa_block_sparse_attn_bwd_workspace_size(plan), dtype=torch.uint8,
                     device=dev)

    def step():
        vsa.vsa_block_sparse_attn_bwd(plan, qb, kb, vb, ob, dob, lse, None, col, wl.topk,
                                      col.numel(), *grads, ws)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for s in range(args.steps):
        step()
        ev[s + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [ev[s].elapsed_time(ev[s + 1]) for s in range(args.steps)]
    ms = max(float(np.mean(per)), wall * 1e3 / args.steps)
    f_valid, _ = step_flops(plan, col.cpu().numpy().astype(np.int64), None, wl.topk)
    f_bwd = 2.5 * f_valid
    tf = f_bwd / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "attention backward effective TFLOP/s (5 products on selected valid pairs)",
        "value": round(tf, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": args.dtype,
        "data": "synthetic: seeded inputs and output gradient, " + args.dtype,
        "config": {"workload": wl.name, "topk": wl.topk, "heads": wl.heads,
                   "seq_len": wl.seq_len, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_16BIT_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / MFMA_16BIT_PEAK_TFLOPS, 4),
                     "traffic": None},
        "flops_backward": f_bwd,
    }), flush=True)


def stage_bandwidth(plan, wl, stage_ms, fused):
    """Algorithmic GB/s of the data-movement stages at their mean times: a
    gather reads the raster tensor and writes the padded blocked copy (the
    fused path's pooling passes read the raster tensor only); the scatter
    reads the blocked output and writes the raster one (16-bit elements; the
    fp32 means and the selected ids are negligible)."""
    raster = wl.batch * wl.seq_len * wl.heads * wl.head_dim * 2
    blocked = wl.batch * wl.heads * plan.padded_len * wl.head_dim * 2
    moved = {"gather_q": raster + blocked, "gather_k": raster + blocked,
             "gather_v": raster + blocked, "scatter": raster + blocked}
    if fused:
        moved = {"pool_q": raster, "pool_k": raster, "pool_v": raster}
    return {n: round(b / (float(np.mean(stage_ms[n])) * 1e-3) / 1e9, 1)
            for n, b in moved.items() if n in stage_ms}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan5b_k64", choices=sorted(WORKLOADS))
    ap.add_argument("--dtype", default="bf16", choices=["bf16", "fp16"],
                    help="element type of Q, K, V and O (the headline is bf16)")
    ap.add_argument("--backward", action="store_true",
                    help="time the attention backward (dQ, dK, dV) instead of the forward layer")
    ap.add_argument("--gated", action="store_true",
                    help="also run the gate-compress branch (pooled V, coarse attention, "
                         "gated scatter) with a synthetic gate")
    ap.add_argument("--fixed-order", action="store_true",
                    help="attention with one workgroup per row in a fixed order instead of "
                         "the balanced launch (rows claimed from per-XCD queues)")
    ap.add_argument("--fused", action="store_true",
                    help="gather-free path: pool Q and K from the raster tensors, score/top-k, "
                         "raster attention writing the raster output (no gather or scatter)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=30.0)
    ap.add_argument("--traffic-json", default=None,
                    help="PMC traffic record of the attention kernel (default: the one in "
                         "profiles/ for the blocked or, with --fused, the raster kernel)")
    ap.add_argument("--copy-calibration", type=int, metavar="MIB")
    ap.add_argument("--record-traffic", nargs=4, metavar="CSV")
    ap.add_argument("--cal-mib", type=int, default=1024)
    ap.add_argument("--stage-traffic", nargs=5, metavar="CSV",
                    help="FETCH.csv WRITE.csv CAL_FETCH.csv CAL_WRITE.csv KERNEL_STATS.csv: "
                         "HBM bytes and GB/s of every kernel of the layer")
    ap.add_argument("--mfma-util", nargs=2, metavar="CSV",
                    help="COUNTER_COLLECTION.csv KERNEL_TRACE.csv of one --pmc --kernel-trace "
                         "run: MFMA busy fraction and clock of the attention kernel")
    args = ap.parse_args()
    if args.traffic_json is None:
        args.traffic_json = os.path.join(
            ROOT, "profiles", "attention_raster_wan5b_k64_traffic.json" if args.fused
            else "attention_wan5b_k64_traffic.json")

    if args.record_traffic:
        record_traffic(args)
        return
    if args.stage_traffic:
        stage_traffic(args)
        return
    if args.mfma_util:
        mfma_utilisation(args)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on exactly one GPU; "
                          f"--gpus {args.gpus} is not supported (no multi-GPU path)"}))
        sys.exit(2)
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    wl = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    log(f"[bench] workload {wl.name}: generating inputs")
    elem = torch.float16 if args.dtype == "fp16" else torch.bfloat16
    q, k, v = make_qkv(wl, dtype=elem)
    dq, dk, dv = (t.to(dev) for t in (q, k, v))
    plan = vsa.vsa_plan(wl.seq_len, wl.dit_seq_shape, wl.block_size, batch=wl.batch,
                        num_heads=wl.heads, head_dim=wl.head_dim, topk=wl.topk or 0,
                        dtype=vsa.VSA_DTYPE_FP16 if args.dtype == "fp16" else vsa.VSA_DTYPE_BF16)
    if args.backward:
        if not wl.topk:
            sys.exit("--backward runs on a top-k workload")
        bench_backward(args, wl, plan, elem, dq, dk, dv)
        return
    log(f"[bench] {vsa.vsa_plan_describe(plan)}")
    if not args.fused:   # the gather-free path keeps no blocked copies
        qb = torch.empty(plan.blocked_shape(), dtype=elem, device=dev)
        kb = torch.empty_like(qb)
        ob = torch.empty_like(qb)
        vb = torch.empty(plan.blocked_vt_shape(), dtype=elem, device=dev)
    qp = torch.empty(plan.pooled_shape(), dtype=torch.float32, device=dev)
    kp = torch.empty_like(qp)
    out = torch.empty(plan.raster_shape(), dtype=elem, device=dev)
    if args.fused:
        stages = FUSED_GATED_STAGES if args.gated else FUSED_STAGES
    else:
        stages = GATED_STAGES if args.gated else STAGES
    if args.gated:
        vp = torch.empty_like(qp)
        oc = torch.empty_like(qp)
        gen = torch.Generator("cpu").manual_seed(77)
        gate = (torch.randn(plan.raster_shape(), generator=gen) * 0.5).to(elem).to(dev)
    if wl.topk:
        col = torch.empty(plan.num_rows() * wl.topk, dtype=torch.int32, device=dev)
        rp_dev, rp_host, uk = None, None, wl.topk
        nnz = col.numel()
    else:
        rp_host, ci_host, _ = make_tile64_map(wl)
        rp_dev = torch.as_tensor(rp_host).to(dev)
        col = torch.as_tensor(ci_host).to(dev)
        uk, nnz = 0, col.numel()
    stream = torch.cuda.current_stream(dev)
    # row queues of the balanced attention launch
    attn_ws = torch.empty(vsa.vsa_attn_fwd_workspace_size(plan), dtype=torch.uint8, device=dev)

    def raster_attention(**gated):
        if args.fixed_order:
            vsa.vsa_block_sparse_attn_fwd_raster(plan, dq, dk, dv, rp_dev, col, uk, nnz, out,
                                                 **gated)
        else:
            vsa.vsa_block_sparse_attn_fwd_raster_ws(plan, dq, dk, dv, rp_dev, col, uk, nnz, out,
                                                    attn_ws, **gated)

    def fused_step(ev=None):
        def mark(n):
            if ev is not None:
                ev[n].record(stream)
        mark(0)
        vsa.vsa_gather(plan, vsa.VSA_ROLE_Q, dq, None, qp)
        mark(1)
        vsa.vsa_gather(plan, vsa.VSA_ROLE_K, dk, None, kp)
        mark(2)
        if wl.topk:
            vsa.vsa_score_topk(plan, qp, kp, wl.topk, col)
        mark(3)
        if args.gated:
            vsa.vsa_gather(plan, vsa.VSA_ROLE_V, dv, None, vp)
            mark(4)
            vsa.vsa_compress_attn(plan, qp, kp, vp, oc)
            mark(5)
            raster_attention(gate=gate, o_coarse=oc)
        else:
            raster_attention()
        mark(len(stages))

    def step(ev=None):
        if args.fused:
            return fused_step(ev)

        def mark(n):
            if ev is not None:
                ev[n].record(stream)
        mark(0)
        vsa.vsa_gather(plan, vsa.VSA_ROLE_Q, dq, qb, qp)
        mark(1)
        vsa.vsa_gather(plan, vsa.VSA_ROLE_K, dk, kb, kp)
        mark(2)
        vsa.vsa_gather(plan, vsa.VSA_ROLE_V, dv, vb, vp if args.gated else None)
        mark(3)
        if wl.topk:
            vsa.vsa_score_topk(plan, qp, kp, wl.topk, col)
        mark(4)
        if args.fixed_order:
            vsa.vsa_block_sparse_attn_fwd(plan, qb, kb, vb, rp_dev, col, uk, nnz, ob)
        else:
            vsa.vsa_block_sparse_attn_fwd_ws(plan, qb, kb, vb, rp_dev, col, uk, nnz, ob, attn_ws)
        mark(5)
        if args.gated:
            vsa.vsa_compress_attn(plan, qp, kp, vp, oc)
            mark(6)
            vsa.vsa_scatter_gated(plan, ob, oc, gate, out)
        else:
            vsa.vsa_scatter(plan, ob, out)
        mark(len(stages))

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
              for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage_ms = {name: [] for name in stages}
    for ev in events:
        for n, name in enumerate(stages):
            stage_ms[name].append(ev[n].elapsed_time(ev[n + 1]))
    gpu_ms = events[0][0].elapsed_time(events[-1][len(stages)]) / args.steps
    ms_per_step = max(wall * 1e3 / args.steps, gpu_ms)
    col_host = col.cpu().numpy().astype(np.int64)
    f_valid, f_nominal = step_flops(plan, col_host, None if rp_host is None else rp_host.astype(np.int64), uk)
    t_attn = float(np.mean(stage_ms["attention"]))
    attn_tflops = f_valid / (t_attn * 1e-3) / 1e12
    value = f_valid / (ms_per_step * 1e-3) / 1e12
    traffic = recorded_traffic(args.traffic_json, wl.name, args.dtype,
                               "raster" if args.fused else "blocked")
    log("[bench] measuring the MFMA loop and the copy bandwidth")
    den = measure_denominators(dev)
    result = {
        "metric": "effective TFLOP/s (selected blocks) + ms/layer, 27280 tok, topk=64, 1 GPU",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic: seeded N(0,1) tokens plus a per-block N(0,0.25) mean vector, "
                + args.dtype,
        "config": {"workload": wl.name, "dit_seq_shape": list(wl.dit_seq_shape),
                   "block_size": list(wl.block_size), "seq_len": wl.seq_len,
                   "heads": wl.heads, "head_dim": wl.head_dim, "batch": wl.batch,
                   "topk": wl.topk, "num_blocks": plan.num_blocks,
                   "gate_compress": bool(args.gated), "gather_free": bool(args.fused),
                   "attention_launch": "fixed order" if args.fixed_order else "balanced",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(attn_tflops, 2),
                     "peak": MFMA_16BIT_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(attn_tflops / MFMA_16BIT_PEAK_TFLOPS, 4),
                     "traffic": traffic,
                     "peak_measured": den["mfma_bf16_tflops"],
                     "frac_measured": round(attn_tflops / den["mfma_bf16_tflops"], 4),
                     "clock_ghz": den["mfma_clock_ghz"],
                     "kernel": "attn_fwd_kernel (balanced launch)" if not args.fixed_order
                               else "attn_fwd_kernel (fixed order)"},
        "measured_denominators": den,
        "stage_ms": {n: round(float(np.mean(v)), 4) for n, v in stage_ms.items()},
        "stage_ms_median": {n: round(float(np.median(v)), 4) for n, v in stage_ms.items()},
        "stage_ms_min": {n: round(float(np.min(v)), 4) for n, v in stage_ms.items()},
        "stage_gbs": stage_bandwidth(plan, wl, stage_ms, args.fused),
        "flops_valid": f_valid,
        "flops_nominal": f_nominal,
        "attention_tflops_nominal": round(f_nominal / (t_attn * 1e-3) / 1e12, 2),
    }
    if not args.no_cpu_baseline:
        if wl.topk:
            log("[bench] checking the block ids against the float64 oracle")
            result["map_check"] = map_check(wl, q, k, col_host)
        log("[bench] timing the CPU oracle")
        result["cpu_baseline"] = cpu_baseline(wl, q, k, v, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
