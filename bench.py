#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

One step = one kvattn_decode call (the forward stage over every planned item,
then the merge stage) on one synthetic decode batch whose q / KV pools are
already resident in HBM.  The plan (host pack scheduler) is built and uploaded
once before timing: one plan serves every layer of a decode step, and its host
time is reported separately as plan_ms.

A default run measures all five workloads, one after the other, and prints one
JSON line: the headline fields are those of the largest single-GPU workload,
the stateful streaming sessions (16 sessions x 131072 tokens, 8 registered
queries each, 64/8 heads, d 128); "per_config" holds the same measurements for
every workload.  --config N measures workload N alone (profiler runs).

So that the 256 MB Infinity Cache cannot serve a whole batch from a previous
step, the steps rotate over enough HBM-resident copies of the KV pools that
each step reads data last touched several hundred MB earlier.

Metric: effective HBM GB/s counting unique KV bytes (each physical block of the
paged cache once, K and V, all KV heads), and microseconds per call.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config all|1..5]
       python bench.py --copy-calibration BYTES   (plain device copy, for counter scaling)
       python bench.py --summarize-trace DIR --config N        (rocprofv3 kernel-trace summary)
       python bench.py --summarize-counters FETCH_DIR WRITE_DIR CAL_FETCH_DIR CAL_WRITE_DIR --config N
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode-attn effective HBM GB/s (unique KV bytes) + us/call, % of MI355X HBM peak"
PEAK_HBM_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "decode_attention_prefix_amd", "csrc", "kvattn_kernels.hip")
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_src_sha():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def describe(c, wl):
    d = {"workload": wl.name, "batch": int(wl.num_queries), "q_heads": wl.num_q_heads, "kv_heads": wl.num_kv_heads,
         "head_dim": wl.head_dim, "block_tokens": 16, "unique_kv_bytes": int(wl.unique_kv_bytes),
         "query_centric_kv_bytes": int(wl.query_centric_kv_bytes), "prefix_ratio": round(wl.prefix_ratio, 4),
         "mean_seq_len": round(float(wl.seq_lens.mean()), 1), "parallelism": "single GPU"}
    d["structure"] = {
        1: "256-token shared prefix + uniform 32-96 suffixes",
        2: "2048-token shared system prefix + uniform 128-1024 suffixes",
        3: "4096 root + 8 x 1024 children (uniform choice) + uniform 64-2048 leaves",
        4: "16 sessions x 131072 tokens, 8 registered queries per session",
        5: "independent lengths log-uniform in [16, 32768]",
    }[c]
    return d


def traffic_from_counters(c):
    """HBM bytes per forward launch from committed rocprofv3 FETCH_SIZE / WRITE_SIZE summaries.

    Each counter (KiB per dispatch) is scaled by what the same counter reads for a
    plain device copy of known size (fetch_scale, write_scale in the summary).
    Returns (read + written bytes, read bytes, bytes the merge launch reads), all
    None when no summary exists for this workload or the kernel source changed
    since the counters were taken.
    """
    path = os.path.join(PROFILES, "counters_c%d.json" % c)
    if not os.path.exists(path):
        return None, None, None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_src_sha") != kernel_src_sha():
        return None, None, None
    fetch = rec["forward_fetch_kib"] * 1024.0 * rec["fetch_scale"]
    write = rec["forward_write_kib"] * 1024.0 * rec["write_scale"]
    merge_fetch = (rec.get("merge_fetch_kib") or 0.0) * 1024.0 * rec["fetch_scale"]
    return fetch + write, fetch, merge_fetch


def cpu_baseline(wl, budget_s=8.0, threads=None):
    """The fp64 oracle on the host cores, on a bounded sample of (query, head) rows.

    When the whole batch costs less than the budget, the sample is the whole
    batch, repeated until the budget is spent; otherwise it is a random subset
    of rows sized to the budget, and the full-batch time is extrapolated by the
    subset's share of the token-row work.  threads: OpenMP threads (None: all
    the host's cores, the oracle's default).
    """
    import oracle
    default_threads = oracle.threads()
    if threads is not None:
        oracle.set_threads(threads)
    try:
        return _cpu_baseline(oracle, wl, budget_s)
    finally:
        oracle.set_threads(default_threads)


def _cpu_baseline(oracle, wl, budget_s):
    B, Hq = wl.num_queries, wl.num_q_heads
    rng = np.random.default_rng(1234)
    rows = rng.permutation(B * Hq).astype(np.int64)
    cost = wl.seq_lens.astype(np.float64)[rows // Hq]
    total_cost = float(cost.sum())
    n0 = max(1, min(len(rows), 64))
    t0 = time.perf_counter()
    oracle.decode_workload(wl, rows=rows[:n0])
    dt0 = max(time.perf_counter() - t0, 1e-6)
    est_full = dt0 * total_cost / float(cost[:n0].sum())
    threads = oracle.threads()
    if est_full <= budget_s:
        reps, t0 = 0, time.perf_counter()
        while True:
            oracle.decode_workload(wl, rows=rows)
            reps += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
        full_s = dt / reps
        sample = "all %d (query, head) rows, %d repetitions in %.2f s wall on %d OpenMP threads" % (
            B * Hq, reps, dt, threads)
    else:
        csum = np.cumsum(cost)
        n = int(min(len(rows), max(n0, np.searchsorted(csum, total_cost * budget_s / est_full) + 1)))
        t0 = time.perf_counter()
        oracle.decode_workload(wl, rows=rows[:n])
        dt = time.perf_counter() - t0
        frac = float(cost[:n].sum()) / total_cost
        full_s = dt / frac
        sample = ("%d of %d (query, head) rows chosen at random (%.1f%% of the token-row work), %.2f s wall on %d "
                  "OpenMP threads; the full batch extrapolates to %.1f s" % (n, B * Hq, 100 * frac, dt, threads,
                                                                             full_s))
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((line.split(":", 1)[1].strip() for line in f if line.startswith("model name")), cpu)
    except OSError:
        pass
    return {"value": round(wl.unique_kv_bytes / full_s / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "sample": sample, "full_batch_seconds": float("%.4g" % full_s), "cpu_model": cpu,
            "host_cpus": os.cpu_count()}


def copy_calibration(nbytes):
    import torch
    n = nbytes // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n * 4, "dispatches": 3}))


def plan_update_timing(K, wl, opts):
    """Host time of kvattn_plan_update for one decode step: a plan at every
    query's length minus one token, brought to the workload's lengths (the
    path taken: 1 patched in place, 2 re-serialized, 3 rebuilt)."""
    lens = (wl.seq_lens - 1).astype(np.int32)
    bt = wl.block_tables.copy()
    for b, T in enumerate(lens):
        bt[b, (int(T) + 15) // 16:] = -1
    plan = K.kvattn_plan(wl.shape_tuple(), bt, lens, None, opts)
    t0 = time.perf_counter()
    K.kvattn_plan_update(plan, wl.block_tables, wl.seq_lens)
    ms = (time.perf_counter() - t0) * 1e3
    return ms, int(K.kvattn_plan_stats(plan)["update_path"])


def append_timing(K, torch, W, wl, dec, pools, q, outs, steps, warmup):
    """The decode step with its KV append fused in (kvattn_decode_append over a
    new-token plan) against the unfused step (the new K/V written with a torch
    index_copy_ per cache, then kvattn_decode over the full lengths), both as
    HIP-graph replays over the rotated KV copies.  Both write the same slots."""
    try:
        fused = K.Decoder(wl.shape_tuple(), wl.block_tables, wl.seq_lens, options=K.make_options(new_token=1))
    except K.KvattnError as e:
        return {"applicable": False, "reason": str(e)}
    B, Hkv, D = wl.num_queries, wl.num_kv_heads, wl.head_dim
    rng = np.random.default_rng(5)

    def bf16_dev(shape):
        return torch.from_numpy(W.f32_to_bf16_bits(rng.standard_normal(shape).astype(np.float32)).view(np.int16)).cuda()

    kn, vn = bf16_dev((B, Hkv, D)), bf16_dev((B, Hkv, D))
    pos = wl.seq_lens.astype(np.int64) - 1
    blk = wl.block_tables[np.arange(B), pos // 16].astype(np.int64)
    rows = ((blk[:, None] * Hkv + np.arange(Hkv)[None, :]) * 16 + (pos % 16)[:, None]).reshape(-1)
    rows = torch.from_numpy(rows).cuda()
    copies = len(pools)

    def fused_call(i):
        kk, vv = pools[i % copies]
        K.kvattn_decode_append(q, kn, vn, kk, vv, fused.plan, outs[i % copies])

    def unfused_call(i):
        kk, vv = pools[i % copies]
        kk.view(-1, D).index_copy_(0, rows, kn.view(-1, D))
        vv.view(-1, D).index_copy_(0, rows, vn.view(-1, D))
        K.kvattn_decode(q, kk, vv, dec.plan, outs[i % copies])

    # the two steps agree (same slots written, same attention)
    fused_call(0)
    torch.cuda.synchronize()
    a = outs[0].clone()
    unfused_call(0)
    torch.cuda.synchronize()
    agree = float((a - outs[0]).abs().max())
    assert agree <= 2e-3, "fused and unfused append steps disagree: %.3e" % agree
    res = {"applicable": True, "max_abs_diff_fused_vs_unfused": agree}
    best = graph_best_us(torch, {"fused": fused_call, "unfused": unfused_call}, copies, steps, warmup)
    for name, us in best.items():
        res[name + "_us_per_call"] = us
    return res


def graph_best_us(torch, fns, copies, steps, warmup):
    """Each step function captured as one HIP graph of `steps` consecutive calls
    (call i on KV copy i mod copies, as the main timing does), replayed once per
    round between HIP events after warm-up replays, in two alternating rounds;
    the best round of each.  Launch-bound sizes are sensitive to what ran just before, hence the
    alternation."""
    graphs = {}
    for name, fn in fns.items():
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                fn(i)
        graphs[name] = g
    best = {}
    for _ in range(2):
        for name, g in graphs.items():
            for _ in range(max(1, warmup // 5)):
                g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / steps * 1e3
            best[name] = min(best.get(name, us), us)
    return {name: round(us, 2) for name, us in best.items()}


def multi_stream_timing(K, torch, wl, dec, pools, q, outs, steps, warmup):
    """The PAT review's multi-stream forward (MFMA launches on a side stream,
    kvattn_decode_streams over a multi_stream plan) against the single-launch
    plan of the main measurement, both as graph replays."""
    ms = K.Decoder(wl.shape_tuple(), wl.block_tables, wl.seq_lens, options=K.make_options(multi_stream=1))
    side = torch.cuda.Stream()
    copies = len(pools)

    def single(i):
        K.kvattn_decode(q, pools[i % copies][0], pools[i % copies][1], dec.plan, outs[i % copies])

    def multi(i):
        K.kvattn_decode_streams(q, pools[i % copies][0], pools[i % copies][1], ms.plan, outs[i % copies], side)

    multi(0)
    torch.cuda.synchronize()
    a = outs[0].clone()
    single(0)
    torch.cuda.synchronize()
    diff = float((a - outs[0]).abs().max())
    assert diff <= 2e-3, "multi-stream and single-launch decodes disagree: %.3e" % diff
    best = graph_best_us(torch, {"single_launch": single, "multi_stream": multi}, copies, steps, warmup)
    st = ms.stats()
    return {"us_per_call_single_launch": best["single_launch"], "us_per_call_multi_stream": best["multi_stream"],
            "multi_stream_launches": st["num_launches"], "max_abs_diff": diff}


# (workgroups per CU, loads in flight per lane, threads): the best of these is the plain-read
# ceiling; a sweep over 2-8 loads, 256-1024 threads and 1-16 workgroups per CU found one of them
# best at every pool size from 169 MB to 8.6 GB
PROBE_CONFIGS = ((2, 4, 256), (1, 2, 1024), (2, 8, 512), (2, 8, 1024))


def plain_read(K, torch, pools, stream, n_ev):
    """A plain streaming read of the same K/V pools (kvattn_read_probe, one contiguous share
    per workgroup), median of HIP-event timed launches, for a few launch shapes: what the
    memory system delivers for those bytes at that size, as context beside the peak."""
    copies = len(pools)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(2 * cus * 1024, dtype=torch.int32, device="cuda")
    nbytes = pools[0][0].numel() * 2 + pools[0][1].numel() * 2
    best = None
    for per_cu, depth, threads in PROBE_CONFIGS:
        grid = per_cu * cus
        for i in range(3):
            K.kvattn_read_probe(pools[i % copies][0], pools[i % copies][1], sink, grid, stream, depth, threads)
        pev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_ev)]
        for i in range(n_ev):
            pev[i][0].record(stream)
            K.kvattn_read_probe(pools[i % copies][0], pools[i % copies][1], sink, grid, stream, depth, threads)
            pev[i][1].record(stream)
        torch.cuda.synchronize()
        us = float(np.median([e[0].elapsed_time(e[1]) for e in pev])) * 1e3
        r = {"GB/s": round(nbytes / (us * 1e-6) / 1e9, 1), "bytes": int(nbytes), "us": round(us, 2), "grid": grid,
             "threads": threads, "loads_in_flight": depth}
        if best is None or r["GB/s"] > best["GB/s"]:
            best = r
    best["what"] = ("kvattn_read_probe: one contiguous share per workgroup of the K and V pools, median of HIP-event "
                    "timed launches, best of %d launch shapes" % len(PROBE_CONFIGS))
    return best


# ---- rocprofv3 summaries (profiles/) -------------------------------------------------------------
WORKLOAD_NAMES = {1: "c1_tiny", 2: "c2_llama3_8b_layer", 3: "c3_two_level_tree", 4: "c4_streaming_sessions",
                  5: "c5_no_sharing"}


def _csv_rows(directory, suffix):
    """Rows of every rocprofv3 CSV file named *<suffix> under directory (any depth)."""
    import csv
    rows = []
    for root, _, files in os.walk(directory):
        for name in sorted(files):
            if name.endswith(suffix):
                with open(os.path.join(root, name), newline="") as f:
                    rows.extend(csv.DictReader(f))
    if not rows:
        raise SystemExit("no *%s under %s" % (suffix, directory))
    return rows


def _short(name):
    name = name.replace("void kvattn::(anonymous namespace)::", "").replace("kvattn::(anonymous namespace)::", "")
    return name.split("(")[0][:60]


def trace_summary(directory, c, command):
    """Text summary of a rocprofv3 --kernel-trace --stats run: calls and durations per kernel."""
    rows = _csv_rows(directory, "kernel_stats.csv")
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    lines = ["rocprofv3 kernel-trace summary: %s" % WORKLOAD_NAMES[c],
             "command: %s" % command,
             "kernel source sha256[:16]: %s" % kernel_src_sha(), "",
             "%-60s %8s %12s %10s %10s %8s" % ("kernel", "calls", "avg_ns", "min_ns", "max_ns", "pct")]
    for r in rows:
        lines.append("%-60s %8s %12.1f %10s %10s %8.2f" % (_short(r["Name"]), r["Calls"], float(r["AverageNs"]),
                                                             r["MinNs"], r["MaxNs"], float(r["Percentage"])))
    return "\n".join(lines)


def _counter_by_kernel(directory, counter):
    """Mean counter value per dispatch, by kernel name (first dispatch of each kernel dropped when
    several exist: it runs cold)."""
    per = {}
    for r in _csv_rows(directory, "counter_collection.csv"):
        if r.get("Counter_Name", counter) != counter:
            continue
        per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return {k: (float(np.mean(v[1:])) if len(v) > 2 else float(np.mean(v)), len(v)) for k, v in per.items()}


def counters_summary(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, c, command):
    """profiles/counters_c<c>.json from four rocprofv3 --pmc runs: FETCH_SIZE and WRITE_SIZE (KiB per
    dispatch) of the decode, and of a plain 1 GiB device copy that scales each counter to bytes."""
    import workloads as W
    fetch = _counter_by_kernel(fetch_dir, "FETCH_SIZE")
    write = _counter_by_kernel(write_dir, "WRITE_SIZE")
    cal_f = max(v for v, _ in _counter_by_kernel(cal_fetch_dir, "FETCH_SIZE").values())
    cal_w = max(v for v, _ in _counter_by_kernel(cal_write_dir, "WRITE_SIZE").values())
    copy_kib = 1024.0 * 1024.0
    fwd = next(k for k in fetch if "fwd_kernel" in k)
    mrg = next((k for k in fetch if "merge_kernel" in k), None)
    wl = W.WORKLOADS[c]()
    uniq = wl.unique_kv_bytes
    rec = {
        "workload": wl.name, "kernel": fwd, "kernel_src_sha": kernel_src_sha(),
        "forward_fetch_kib": fetch[fwd][0], "forward_write_kib": write[fwd][0],
        "merge_fetch_kib": fetch[mrg][0] if mrg else None, "merge_write_kib": write[mrg][0] if mrg else None,
        "fetch_scale": round(copy_kib / cal_f, 6), "write_scale": round(copy_kib / cal_w, 6),
        "dispatches_averaged": fetch[fwd][1] - (1 if fetch[fwd][1] > 2 else 0),
        "unique_kv_bytes": int(uniq),
    }
    rec["forward_fetch_bytes"] = int(rec["forward_fetch_kib"] * 1024 * rec["fetch_scale"])
    rec["forward_write_bytes"] = int(rec["forward_write_kib"] * 1024 * rec["write_scale"])
    rec["fetch_over_unique"] = round(rec["forward_fetch_bytes"] / uniq, 4)
    rec["commands"] = command
    rec["scale_note"] = ("a 1 GiB device copy reads %.1f KiB by FETCH_SIZE and writes %.1f KiB by WRITE_SIZE per "
                         "dispatch; scale = 1 GiB / counter" % (cal_f, cal_w))
    path = os.path.join(PROFILES, "counters_c%d.json" % c)
    with open(path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


# timed steps of the workloads that are not the headline (the headline takes --steps exactly)
OTHER_STEPS = {1: 400, 2: 200, 3: 100, 4: 30, 5: 30}
HEADLINE = 4
SINGLE_CORE_CONFIGS = (1, 2, 3)


def measure(c, args, torch, K, W, steps, warmup, extras_on):
    """Every measurement of workload c; returns (record, workload description)."""
    t_gen = time.perf_counter()
    wl = W.WORKLOADS[c]().materialize()
    log("bench: %s generated in %.1f s; unique KV %.1f MB" % (wl.name, time.perf_counter() - t_gen,
                                                              wl.unique_kv_bytes / 1e6))
    opts = K.make_options(pack_mode=args.pack_mode, split_tokens=args.split_tokens, fused_merge=args.fused_merge,
                          force_variant=args.force_variant, num_cus=args.num_cus)
    # the device is initialised before this point: plan_upload_ms covers planning,
    # the workspace allocation and the upload copy only
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    dec = K.Decoder(wl.shape_tuple(), wl.block_tables, wl.seq_lens, options=opts)
    torch.cuda.synchronize()
    plan_upload_ms = (time.perf_counter() - t0) * 1e3
    st = dec.stats()
    log("bench: plan %s" % json.dumps(st))
    upd_ms, upd_path = plan_update_timing(K, wl, opts)
    log("bench: plan update (one decode step) %.3f ms, path %d" % (upd_ms, upd_path))

    pool_bytes = wl.k_pool.nbytes + wl.v_pool.nbytes
    copies = args.copies or max(1, min(8, math.ceil(3 * 256e6 / pool_bytes) + 1))
    q = torch.from_numpy(wl.q.view(np.int16)).cuda()
    k0 = torch.from_numpy(wl.k_pool.view(np.int16)).cuda()
    v0 = torch.from_numpy(wl.v_pool.view(np.int16)).cuda()
    pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(copies - 1)]
    outs = [torch.empty((wl.num_queries, wl.num_q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
            for _ in range(copies)]
    stream = torch.cuda.current_stream()

    parity = None
    if not args.no_check:
        import oracle
        K.kvattn_decode(q, k0, v0, dec.plan, outs[0], stream)
        torch.cuda.synchronize()
        rng = np.random.default_rng(0)
        rows = rng.choice(wl.num_queries * wl.num_q_heads, size=min(64, wl.num_queries * wl.num_q_heads),
                          replace=False).astype(np.int64)
        ref = oracle.decode_workload(wl, rows=rows)
        got = outs[0].cpu().numpy().reshape(-1, wl.head_dim)[rows]
        err = float(np.abs(got - ref).max())
        log("bench: parity on %d sampled rows: max abs err %.3e" % (len(rows), err))
        assert err <= 2e-3, "parity check failed"
        parity = {"rows_checked": int(len(rows)), "max_abs_err": float("%.3g" % err), "tolerance": 2e-3}

    def eager_step(i):
        kk, vv = pools[i % copies]
        K.kvattn_decode(q, kk, vv, dec.plan, outs[i % copies], stream)

    for i in range(warmup):
        eager_step(i)
    torch.cuda.synchronize()

    # one HIP graph per KV copy: a replay is one decode call (forward + merge launches)
    # HIP graphs of consecutive decode calls, rotating over the KV copies: a model's
    # decode step runs its layers' attention calls back to back inside one graph,
    # so the timed region replays one graph holding exactly `steps` calls
    # ("graph"); "graph-per-call" replays a one-call graph per step instead.
    graphs, per_call = [], []
    timing = "eager launches"
    if not args.no_graph:
        for i in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                K.kvattn_decode(q, pools[i][0], pools[i][1], dec.plan, outs[i])
            per_call.append(g)
        for i in range(warmup):
            per_call[i % copies].replay()
        torch.cuda.synchronize()
        if args.timing == "graph":
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(steps):
                    K.kvattn_decode(q, pools[i % copies][0], pools[i % copies][1], dec.plan, outs[i % copies])
            graphs.append(g)
            timing = "one HIP graph of %d consecutive calls (rotating over %d KV copies), replayed once" % (steps,
                                                                                                         copies)
        else:
            timing = "HIP graph replay per call"

    def step(i):
        if per_call:
            per_call[i % copies].replay()
        else:
            eager_step(i)

    # Untimed pre-warm by time, before the counted warm-up steps: short calls
    # (tens of microseconds) need ~0.1 s of work before the GPU's clocks settle,
    # more than a few warm-up steps give.  The timed region below is unchanged.
    t_warm = time.perf_counter()
    i = 0
    while time.perf_counter() - t_warm < args.prewarm_s:
        for _ in range(16):
            step(i)
            i += 1
        torch.cuda.synchronize()
    for i in range(warmup):
        step(i)
    if graphs:
        graphs[0].replay()   # the timed graph itself, once untimed
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps, synchronised on both sides
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graphs:
        graphs[0].replay()
    else:
        for i in range(steps):
            step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / steps * 1e3

    # Per-stage GPU time with HIP events on the launch stream.  With graphs: one
    # graph of n_ev consecutive forward launches and one of n_ev merge launches
    # (over the partials the last forward wrote), each replay bracketed by events:
    # the average duration of each kernel as it runs back to back, without launch
    # latency.  Eagerly: an event pair around each launch.
    n_ev = min(max(steps, 30), 100)
    if graphs:
        merges = st["num_merge_rows"] > 0   # one-launch plans have no merge launch
        gf, gm = torch.cuda.CUDAGraph(), torch.cuda.CUDAGraph()
        with torch.cuda.graph(gf):
            for i in range(n_ev):
                kk, vv = pools[i % copies]
                K.kvattn_forward(q, kk, vv, dec.plan, outs[i % copies])
        if merges:
            with torch.cuda.graph(gm):
                for i in range(n_ev):
                    K.kvattn_merge(dec.plan, outs[(n_ev - 1) % copies])
        gf.replay()
        if merges:
            gm.replay()
        torch.cuda.synchronize()
        fwd_ms, mrg_ms = [], []
        for _ in range(3):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            ev[0].record(stream)
            gf.replay()
            ev[1].record(stream)
            if merges:
                gm.replay()
            ev[2].record(stream)
            torch.cuda.synchronize()
            fwd_ms.append(ev[0].elapsed_time(ev[1]) / n_ev)
            mrg_ms.append(ev[1].elapsed_time(ev[2]) / n_ev)
        fwd_ms, mrg_ms = np.array(fwd_ms), np.array(mrg_ms)
        stage_timing = "graphs of %d consecutive forward launches, then %d merge launches, events around each" % (
            n_ev, n_ev)
        del gf, gm
    else:
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_ev)]
        for i in range(n_ev):
            kk, vv = pools[i % copies]
            evs[i][0].record(stream)
            K.kvattn_forward(q, kk, vv, dec.plan, outs[i % copies], stream)
            evs[i][1].record(stream)
            K.kvattn_merge(dec.plan, outs[i % copies], stream)
            evs[i][2].record(stream)
        torch.cuda.synchronize()
        fwd_ms = np.array([evs[i][0].elapsed_time(evs[i][1]) for i in range(n_ev)])
        mrg_ms = np.array([evs[i][1].elapsed_time(evs[i][2]) for i in range(n_ev)])
        stage_timing = "an event pair around each eager launch"
    call_ms = fwd_ms + mrg_ms

    plain = plain_read(K, torch, pools, stream, n_ev)
    append = multi = None
    if extras_on:
        append = append_timing(K, torch, W, wl, dec, pools, q, outs, min(steps, 100), warmup)
        log("bench: decode step with KV append %s" % json.dumps(append))
        multi = multi_stream_timing(K, torch, wl, dec, pools, q, outs, min(steps, 100), warmup)
        log("bench: multi-stream forward %s" % json.dumps(multi))

    uniq = wl.unique_kv_bytes
    value = uniq / (ms_per_step * 1e-3) / 1e9
    fwd_avg = float(fwd_ms.mean())
    achieved = uniq / (fwd_avg * 1e-3) / 1e9
    traffic, fetched, merge_fetched = traffic_from_counters(c)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None if traffic is None else int(traffic),
                "kernel": "fwd_kernel (persistent; %d MFMA + %d VALU items)" % (st["num_items_mfma"],
                                                                                 st["num_items_valu"]),
                "algorithmic_bytes_per_launch": int(uniq),
                "avg_forward_us": round(fwd_avg * 1e3, 2),
                # plans without merge rows (one-launch plans) have no merge launch
                "avg_merge_us": round(float(mrg_ms.mean()) * 1e3, 2) if st["num_merge_rows"] > 0 else None,
                "stage_timing": stage_timing,
                "plain_read": dict(plain, forward_over_plain_read=round(achieved / plain["GB/s"], 4))}
    rec = {
        "value": round(value, 1), "unit": "GB/s", "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_call": round(ms_per_step * 1e3, 2),
        "us_per_call_gpu_events_median": round(float(np.median(call_ms)) * 1e3, 2),
        "pct_of_peak_hbm": round(100 * value / PEAK_HBM_GBS, 2),
        "redundancy_fetch_over_unique": None if fetched is None else round(fetched / uniq, 4),
        "redundancy_fetch_over_unique_with_merge": None if fetched is None else round((fetched + merge_fetched) / uniq,
                                                                                      4),
        "plan_ms": round(st["plan_seconds"] * 1e3, 3), "plan_upload_ms": round(plan_upload_ms, 3),
        "plan_update_ms": round(upd_ms, 3), "plan_update_path": upd_path,
        "parity_sample": parity,
        "decode_with_kv_append": append,
        "multi_stream_forward": multi,
        "plan": {k: st[k] for k in ("num_items", "num_items_valu", "num_items_mfma", "num_packed_nodes",
                                    "num_folded_leaves", "num_merge_rows", "num_launches", "split_tokens",
                                    "planned_kv_bytes", "partial_bytes")},
        "kv_copies_rotated": copies,
        "timing": timing,
        "roofline": roofline,
    }
    desc = describe(c, wl)
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget_s)
        log("bench: cpu baseline %s" % json.dumps(rec["cpu_baseline"]))
        if c in SINGLE_CORE_CONFIGS:
            rec["cpu_baseline_single_core"] = cpu_baseline(wl, args.cpu_budget_s / 2, threads=1)
            log("bench: cpu baseline, one core %s" % json.dumps(rec["cpu_baseline_single_core"]))
    del dec, graphs, per_call, pools, outs, q, k0, v0
    wl.release_values()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec, desc


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30, help="timed steps of the headline workload")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="all", choices=["all", "1", "2", "3", "4", "5"])
    ap.add_argument("--pack-mode", type=int, default=0)
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--num-cus", type=int, default=0,
                    help="plan option num_cus (0: a whole MI355X); more than the device's CUs leaves lists to run-time claims")
    ap.add_argument("--force-variant", type=int, default=-1, choices=[-1, 0, 1, 2],
                    help="plan option force_variant: -1 auto, 0 VALU, 1 MFMA, 2 VALU_SPLIT tile for every item")
    ap.add_argument("--fused-merge", type=int, default=-1, choices=[-1, 0, 1],
                    help="plan option fused_merge: -1 auto, 0 merge launch, 1 merge inside the forward launch")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=8.0, help="wall seconds of oracle work per workload")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--copies", type=int, default=0)
    ap.add_argument("--copy-calibration", type=int, default=0)
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--timing", default="graph", choices=["graph", "graph-per-call"],
                    help="graph: one HIP graph of the timed steps' consecutive calls; graph-per-call: one replay per call")
    ap.add_argument("--prewarm-s", type=float, default=0.2,
                    help="seconds of untimed calls before the counted warm-up steps (GPU clocks settle)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the fused-append and multi-stream timings (profiler runs of the decode alone)")
    ap.add_argument("--summarize-trace", default=None, metavar="DIR")
    ap.add_argument("--summarize-counters", nargs=4, default=None,
                    metavar=("FETCH_DIR", "WRITE_DIR", "CAL_FETCH_DIR", "CAL_WRITE_DIR"))
    ap.add_argument("--command", default="", help="the profiling command, recorded in a summary")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this decode-attention library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.summarize_trace or args.summarize_counters:
        c = HEADLINE if args.config == "all" else int(args.config)
        if args.summarize_trace:
            print(trace_summary(args.summarize_trace, c, args.command))
        else:
            counters_summary(*args.summarize_counters, c, args.command)
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import torch
    import workloads as W
    from decode_attention_prefix_amd import kvattn as K

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    # device, allocator and pageable host-to-device copy path initialised before any timing:
    # plan_upload_ms then covers planning, the workspace allocation and the upload copy only
    torch.cuda.init()
    torch.from_numpy(np.zeros(1 << 20, dtype=np.uint8)).cuda()
    torch.cuda.synchronize()
    configs = [1, 2, 3, 4, 5] if args.config == "all" else [int(args.config)]
    headline = HEADLINE if args.config == "all" else int(args.config)
    per_config, desc = {}, {}
    for c in configs:
        steps = args.steps if c == headline else max(args.steps, OTHER_STEPS[c])
        rec, d = measure(c, args, torch, K, W, steps, args.warmup, extras_on=not args.no_extras)
        per_config[d["workload"]] = dict(rec, config=d)
        desc[c] = d
        log("bench: %s %.2f us/call, %.1f GB/s (%.1f %% of peak), forward frac %.4f" % (
            d["workload"], rec["us_per_call"], rec["value"], rec["pct_of_peak_hbm"], rec["roofline"]["frac"]))
    head = per_config[desc[headline]["workload"]]
    result = {
        "metric": METRIC, "value": head["value"], "unit": "GB/s", "n_gpus": 1, "steps": head["steps"],
        "warmup": head["warmup"], "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic", "config": desc[headline],
    }
    for k in ("us_per_call", "us_per_call_gpu_events_median", "pct_of_peak_hbm", "redundancy_fetch_over_unique",
              "redundancy_fetch_over_unique_with_merge", "plan_ms", "plan_upload_ms", "plan_update_ms",
              "plan_update_path", "parity_sample", "plan", "kv_copies_rotated", "timing", "roofline"):
        result[k] = head[k]
    if "cpu_baseline" in head:
        result["cpu_baseline"] = head["cpu_baseline"]
    if len(per_config) > 1:
        summary_keys = ("us_per_call", "value", "pct_of_peak_hbm", "redundancy_fetch_over_unique",
                        "redundancy_fetch_over_unique_with_merge", "plan_ms", "plan_upload_ms", "plan_update_ms",
                        "parity_sample", "decode_with_kv_append", "multi_stream_forward", "plan", "steps",
                        "kv_copies_rotated", "cpu_baseline", "cpu_baseline_single_core")
        result["per_config"] = {}
        for name, rec in per_config.items():
            r = {k: rec[k] for k in summary_keys if k in rec}
            rf = rec["roofline"]
            r["forward"] = {"avg_us": rf["avg_forward_us"], "merge_avg_us": rf["avg_merge_us"],
                            "frac": rf["frac"], "achieved_GB/s": rf["achieved"], "traffic": rf["traffic"],
                            "plain_read_GB/s": rf["plain_read"]["GB/s"],
                            "forward_over_plain_read": rf["plain_read"]["forward_over_plain_read"]}
            r["config"] = {k: rec["config"][k] for k in ("batch", "q_heads", "kv_heads", "head_dim",
                                                         "unique_kv_bytes", "prefix_ratio", "structure")}
            result["per_config"][name] = r
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
