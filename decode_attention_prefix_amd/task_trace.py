"""Per-task traces of the forward launch: a diagnostic, not part of the decode path.

Loads the trace build of the library (_build/trace/libkvattn.so, made by build.py: the same
planner and runtime, the kernels compiled with -DKVATTN_TASK_TRACE), decodes a workload as a
HIP graph of consecutive calls, and keeps the records the last call's forward launch wrote:
per workgroup slot, when its list started, when each MFMA task started and ended, when each
wave's VALU stream ended, and on which XCD, SE and CU it ran.  Prints a summary: end times of
the workgroups (overall, per XCD, per workgroup slot), MFMA time per 32-token tile, VALU time
per block and wave, and how evenly each XCD's CUs stream.

Usage: python -m decode_attention_prefix_amd.task_trace --config N [--calls 12] [--reps 3]
"""
from __future__ import annotations

import argparse
import ctypes
import os
import sys
import time

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
TRACE_LIB = os.path.join(ROOT, "_build", "trace", "libkvattn.so")
EVENTS = 64          # records per workgroup slot (kTraceEvents in the kernels)
WAVE_END = 40        # record index of wave 0's VALU stream end
SLOTS = 4096         # workgroup slots the buffer holds


def _ensure_trace_library():
    """Point the binding at the trace build before it loads a library."""
    if not os.path.exists(TRACE_LIB):
        raise SystemExit("no %s: run decode_attention_prefix_amd.build first" % TRACE_LIB)
    if "decode_attention_prefix_amd.kvattn" in sys.modules:
        raise SystemExit("the library is already loaded; run task_trace in a fresh process")
    os.environ["KVATTN_LIBRARY"] = TRACE_LIB


def record(config, calls, reps):
    """Trace buffers of `reps` graph replays of `calls` consecutive decodes of workload `config`."""
    _ensure_trace_library()
    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import torch
    import workloads as W
    from decode_attention_prefix_amd import kvattn as K

    lib = ctypes.CDLL(TRACE_LIB)
    lib.kvattn_trace_set.argtypes = [ctypes.c_void_p]
    lib.kvattn_trace_set.restype = ctypes.c_int
    wl = W.WORKLOADS[config]().materialize()
    dec = K.Decoder(wl.shape_tuple(), wl.block_tables, wl.seq_lens)
    q = torch.from_numpy(wl.q.view(np.int16)).cuda()
    k0 = torch.from_numpy(wl.k_pool.view(np.int16)).cuda()
    v0 = torch.from_numpy(wl.v_pool.view(np.int16)).cuda()
    copies = max(2, min(6, int(3 * 256e6 / (wl.k_pool.nbytes * 2)) + 2))
    pools = [(k0, v0)] + [(k0.clone(), v0.clone()) for _ in range(copies - 1)]
    out = torch.empty((wl.num_queries, wl.num_q_heads, wl.head_dim), device="cuda")
    buf = torch.zeros(SLOTS * EVENTS * 4, dtype=torch.int32, device="cuda")
    if lib.kvattn_trace_set(ctypes.c_void_p(buf.data_ptr())) != 0:
        raise SystemExit("kvattn_trace_set failed")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            K.kvattn_decode(q, pools[i % copies][0], pools[i % copies][1], dec.plan, out)
    recs, per_call = [], []
    t_end = time.perf_counter() + 0.3   # untimed replays first: the clocks settle
    while time.perf_counter() < t_end:
        g.replay()
        torch.cuda.synchronize()
    for _ in range(reps):
        g.replay()
        torch.cuda.synchronize()
        buf.zero_()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        per_call.append(e0.elapsed_time(e1) * 1e3 / calls)
        recs.append(buf.cpu().numpy().reshape(SLOTS, EVENTS, 4).view(np.uint32).copy())
    lib.kvattn_trace_set(ctypes.c_void_p(0))
    return wl.name, recs, per_call


def kernel_src_sha():
    import hashlib
    with open(os.path.join(PKG, "csrc", "kvattn_kernels.hip"), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def summarize(name, recs, per_call, command=""):
    """Text summary of the traces (times in microseconds from the first list start)."""
    lines = ["per-task trace: %s (last call of a graph of consecutive decodes; %d replays)" % (name, len(recs)),
             "command: %s" % command, "kernel source sha256[:16]: %s" % kernel_src_sha(),
             "us per call over the graphs: %s" % ", ".join("%.2f" % x for x in per_call)]
    for rep, r in enumerate(recs):
        typ = r[:, :, 0] & 0xFF
        xcc = (r[:, :, 0] >> 8) & 0xF
        valid = r[:, :, 1] != 0
        n = int(valid[:, 0].sum())
        t = r[:, :, 1].astype(np.int64)
        t0 = t[valid].min()
        T = (t - t0) / 100.0
        end = np.array([T[w][valid[w]].max() for w in range(n)])
        x = xcc[:n, 0]
        lines.append("")
        lines.append("replay %d: %d workgroups; end p10 %.1f p50 %.1f p90 %.1f max %.1f" % (
            rep, n, *np.percentile(end, [10, 50, 90, 100])))
        lines.append("  per XCD (p50 / max end): " + "  ".join(
            "%d: %.1f/%.1f" % (xx, np.median(end[x == xx]), end[x == xx].max()) for xx in range(8) if (x == xx).any()))
        if n >= 512:
            lines.append("  first-slot lists end p50 %.1f, second-slot lists p50 %.1f" % (
                np.median(end[:n // 2]), np.median(end[n // 2:])))
        mt = []
        for w in range(n):
            ev = [(int(typ[w, i]), T[w, i], int(r[w, i, 3])) for i in range(WAVE_END) if valid[w, i]]
            for a, b in zip(ev, ev[1:]):
                if a[0] == 1 and b[0] == 2:
                    tiles = max(1, ((a[2] & 0xFFFFF) + 31) // 32)
                    mt.append(((b[1] - a[1]) / tiles, a[2] >> 20))
        if mt:
            mt = np.array(mt)
            lines.append("  MFMA tasks %d: us per 32-token tile p10 %.2f p50 %.2f p90 %.2f (rows %s)" % (
                len(mt), *np.percentile(mt[:, 0], [10, 50, 90]), sorted(set(int(v) for v in mt[:, 1]))))
        vs = []
        for w in range(n):
            ready = [T[w, i] for i in range(WAVE_END) if valid[w, i] and typ[w, i] == 3]
            for k in range(4):
                if ready and valid[w, WAVE_END + k] and r[w, WAVE_END + k, 3]:
                    vs.append((T[w, WAVE_END + k] - ready[0]) / r[w, WAVE_END + k, 3])
        if vs:
            lines.append("  VALU waves %d: us per block p10 %.2f p50 %.2f p90 %.2f" % (
                len(vs), *np.percentile(vs, [10, 50, 90])))
        if n >= 512:
            cu_end = np.maximum(end[:256], end[256:512])
            spread = ["%d: %.1f-%.1f" % (xx, cu_end[x[:256] == xx].min(), cu_end[x[:256] == xx].max()) for xx in range(8)]
            lines.append("  CU end range per XCD: " + "  ".join(spread))
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--config", type=int, required=True, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--calls", type=int, default=12)
    ap.add_argument("--reps", type=int, default=3)
    args = ap.parse_args()
    command = "python -m decode_attention_prefix_amd.task_trace --config %d --calls %d --reps %d" % (
        args.config, args.calls, args.reps)
    print(summarize(*record(args.config, args.calls, args.reps), command=command), flush=True)


if __name__ == "__main__":
    main()
