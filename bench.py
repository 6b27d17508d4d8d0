#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

One step = one kvattn_decode call (the forward stage over every planned item,
then the merge stage) on one synthetic decode batch whose q / KV pools are
already resident in HBM.  The plan (host pack scheduler) is built and uploaded
once before timing: one plan serves every layer of a decode step, and its host
time is reported separately as plan_ms.

So that the 256 MB Infinity Cache cannot serve a whole batch from a previous
step, the steps rotate over enough HBM-resident copies of the KV pools that
each step reads data last touched several hundred MB earlier.

Metric: effective HBM GB/s counting unique KV bytes (each physical block of the
paged cache once, K and V, all KV heads), and microseconds per call.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]
       python bench.py --copy-calibration BYTES   (plain device copy, for counter scaling)
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


def cpu_baseline(wl, budget_s=12.0):
    """The fp64 oracle on the host cores, on a bounded sample of (query, head) rows.

    When the whole batch costs less than the budget, the sample is the whole
    batch, repeated until the budget is spent; otherwise it is a random subset
    of rows sized to the budget, and the full-batch time is extrapolated by the
    subset's share of the token-row work.
    """
    import oracle
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
    """HIP-graph replays of each step function (one graph per KV copy), timed in two
    alternating rounds; the best round of each.  Launch-bound sizes are sensitive to
    what ran just before, hence the alternation."""
    graphs = {}
    for name, fn in fns.items():
        graphs[name] = []
        for i in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn(i)
            graphs[name].append(g)
    best = {}
    for _ in range(2):
        for name, gs in graphs.items():
            for i in range(warmup):
                gs[i % copies].replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for i in range(steps):
                gs[i % copies].replay()
            torch.cuda.synchronize()
            us = (time.perf_counter() - t0) / steps * 1e6
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


def extras(K, torch, W, wl, dec, pools, q, outs, stream, n_ev, pool_bytes, args):
    """Context beside the roofline: a plain streaming read of the same K/V pools
    (kvattn_read_probe, same grid), and the decode step with its KV append fused in."""
    copies = len(pools)
    grid = 2 * torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(grid * 256, dtype=torch.int32, device="cuda")
    for i in range(3):
        K.kvattn_read_probe(pools[i % copies][0], pools[i % copies][1], sink, grid, stream)
    pev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_ev)]
    for i in range(n_ev):
        pev[i][0].record(stream)
        K.kvattn_read_probe(pools[i % copies][0], pools[i % copies][1], sink, grid, stream)
        pev[i][1].record(stream)
    torch.cuda.synchronize()
    probe_us = float(np.median([e[0].elapsed_time(e[1]) for e in pev])) * 1e3
    attainable = pool_bytes / (probe_us * 1e-6) / 1e9

    append = append_timing(K, torch, W, wl, dec, pools, q, outs, min(args.steps, 100), args.warmup)
    log("bench: decode step with KV append %s" % json.dumps(append))
    multi = multi_stream_timing(K, torch, wl, dec, pools, q, outs, min(args.steps, 100), args.warmup)
    log("bench: multi-stream forward %s" % json.dumps(multi))
    plain = {"GB/s": round(attainable, 1), "bytes": int(pool_bytes), "us": round(probe_us, 2), "grid": grid,
                     "what": "kvattn_read_probe: one contiguous share per workgroup of the K and V pools, "
                             "median of HIP-event timed launches"}
    return plain, append, multi


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--pack-mode", type=int, default=0)
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-check", action="store_true")
    ap.add_argument("--copies", type=int, default=0)
    ap.add_argument("--copy-calibration", type=int, default=0)
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying HIP graphs")
    ap.add_argument("--prewarm-s", type=float, default=0.2,
                    help="seconds of untimed calls before the counted warm-up steps (GPU clocks settle)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the plain-read probe and the fused-append timing (profiler runs of the decode alone)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: this decode-attention library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import torch
    import workloads as W
    from decode_attention_prefix_amd import kvattn as K

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    t_gen = time.perf_counter()
    wl = W.WORKLOADS[args.config]().materialize()
    log("bench: %s generated in %.1f s; unique KV %.1f MB" % (wl.name, time.perf_counter() - t_gen,
                                                              wl.unique_kv_bytes / 1e6))
    opts = K.make_options(pack_mode=args.pack_mode, split_tokens=args.split_tokens)
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

    def eager_step(i):
        kk, vv = pools[i % copies]
        K.kvattn_decode(q, kk, vv, dec.plan, outs[i % copies], stream)

    for i in range(args.warmup):
        eager_step(i)
    torch.cuda.synchronize()

    # one HIP graph per KV copy: a replay is one decode call (forward + merge launches)
    graphs = []
    if not args.no_graph:
        for i in range(copies):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                K.kvattn_decode(q, pools[i][0], pools[i][1], dec.plan, outs[i])
            graphs.append(g)
        for i in range(args.warmup):
            graphs[i % copies].replay()
        torch.cuda.synchronize()

    def step(i):
        if graphs:
            graphs[i % copies].replay()
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
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: exactly K steps, synchronised on both sides
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall / args.steps * 1e3

    # per-stage GPU time with HIP events on the launch stream
    n_ev = min(args.steps, 100)
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
    call_ms = fwd_ms + mrg_ms

    # a plain streaming read of the same pools (same bytes, same grid) for context beside the peak
    plain_read = append = multi = None
    if not args.no_extras:
        plain_read, append, multi = extras(K, torch, W, wl, dec, pools, q, outs, stream, n_ev, pool_bytes, args)

    uniq = wl.unique_kv_bytes
    value = uniq / (ms_per_step * 1e-3) / 1e9
    fwd_avg = float(fwd_ms.mean())
    achieved = uniq / (fwd_avg * 1e-3) / 1e9
    traffic, fetched, merge_fetched = traffic_from_counters(args.config)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": None if traffic is None else int(traffic),
                "kernel": "fwd_kernel (persistent; %d MFMA + %d VALU items)" % (st["num_items_mfma"],
                                                                                 st["num_items_valu"]),
                "algorithmic_bytes_per_launch": int(uniq),
                "avg_forward_us": round(fwd_avg * 1e3, 2), "avg_merge_us": round(float(mrg_ms.mean()) * 1e3, 2),
                "plain_read": None if plain_read is None else
                dict(plain_read, forward_over_plain_read=round(achieved / plain_read["GB/s"], 4))}
    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": describe(args.config, wl),
        "us_per_call": round(ms_per_step * 1e3, 2),
        "us_per_call_gpu_events_median": round(float(np.median(call_ms)) * 1e3, 2),
        "pct_of_peak_hbm": round(100 * value / PEAK_HBM_GBS, 2),
        "redundancy_fetch_over_unique": None if fetched is None else round(fetched / uniq, 4),
        "redundancy_fetch_over_unique_with_merge": None if fetched is None else round((fetched + merge_fetched) / uniq, 4),
        "plan_ms": round(st["plan_seconds"] * 1e3, 3), "plan_upload_ms": round(plan_upload_ms, 3),
        "plan_update_ms": round(upd_ms, 3), "plan_update_path": upd_path,
        "decode_with_kv_append": append,
        "multi_stream_forward": multi,
        "plan": {k: st[k] for k in ("num_items", "num_items_valu", "num_items_mfma", "num_packed_nodes",
                                    "num_folded_leaves", "num_merge_rows", "num_launches", "split_tokens",
                                    "planned_kv_bytes", "partial_bytes")},
        "kv_copies_rotated": copies,
        "timing": "HIP graph replay per call" if graphs else "eager launches",
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
