#!/usr/bin/env python3
"""Benchmark of one attention layer's mixed prefill/decode varlen paged attention on one
MI355X.

A step is one ``varlen_attn_run`` of the whole planned iteration (every kernel of the hot
path) over inputs already resident in HBM.  The timed steps are issued as a model's
forward issues them: consecutive runs read and write the buffers of consecutive layers
(32 copies of Q, K, V and the output), all captured in one HIP graph that is launched
once; the time per step with one graph launch per run and the eager time are reported
beside it, and per-kernel times come from eager runs with the library's events.  The
headline workload is the ORCA-style mixed iteration: a 4096-token uncached prefill plus decodes at 1500 and 1700 cached positions,
32 query / 32 KV heads, head_dim 128, 16-token pages in a seeded random permutation, bf16.
It is MFMA-bound, so ``value`` is TFLOP/s of algorithmic attention work (4·head_dim FLOPs
per visible (query, key) pair per query head).  Secondary lines time the decode-heavy,
chunked-prefill-mix and shared-prefix workloads (HBM GB/s of algorithmic bytes, µs/step).

Prints progress on stderr and ONE JSON line on stdout.
"""
import argparse
import hashlib
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "varlen paged attn: decode HBM GB/s + prefill TFLOP/s, % of MI355X peak"
PEAK_HBM = 8.0e12          # B/s, MI355X HBM3E
PEAK_BF16 = 2.5e15         # FLOP/s, MI355X dense bf16 MFMA
STAGES = ("prefill", "split_kv", "combine")
KERNEL_NAMES = {"prefill": "prefill_bf16_kernel", "split_kv": "split_kv_bf16_kernel", "combine": "combine_kernel"}
KERNEL_NAMES_FP8 = {**KERNEL_NAMES, "split_kv": "split_kv_fp8_kernel"}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")


def kernel_source_hash():
    """sha256 (first 16 hex digits) over the library sources, in name order."""
    csrc = os.path.join(ROOT, "varlen_paged_attention_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".hip", ".cpp", ".h")):
            h.update(name.encode())
            h.update(open(os.path.join(csrc, name), "rb").read())
    return h.hexdigest()[:16]


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` on `workload` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE passes (already scaled by the copy-kernel calibration), or None when the
    counters were taken on other kernel sources."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("sources_sha256_16") != kernel_source_hash():
        return None
    e = t.get(workload, {}).get(kernel)
    return None if not e else e.get("hbm_bytes")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


CLOCK_SETTLE_S = 0.25


def settle_clocks(api, plan, tensors, seconds=CLOCK_SETTLE_S):
    """Untimed plain runs, in batches of 64 between synchronisations, until `seconds` of
    wall time have passed; returns their count.  An idle GPU starts a burst of work at a
    low clock and raises it over the first tens of milliseconds, so a few warm-up runs
    (under a millisecond of work) leave the timed runs partly at the idle clock; a
    serving loop runs at the sustained one."""
    import torch
    q, k, v, bt, out, ws = tensors[:6]
    scales = dict(zip(("k_scale", "v_scale"), tensors[6:]))
    run = api.RunCall(plan, q, k, v, bt, out, ws, **scales)
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(64):
            run()
        torch.cuda.synchronize()
        n += 64
    return n


def time_runs(api, plan, tensors, steps, warmup, flush=None):
    """Run warmup + steps iterations; returns (wall ms/step, per-stage mean ms, per-step
    total ms list).  The wall clock times `steps` plain runs.  The stage times come from
    the library's HIP events in a second pass of `steps` runs enqueued behind a few plain
    runs (the host enqueues a run in under 10 µs, so the queue never drains and no
    host-side gap between an event and its kernel is counted as kernel time; real work,
    unlike a spin kernel, also keeps the clocks where the timed runs put them)."""
    import torch
    q, k, v, bt, out, ws = tensors[:6]
    scales = dict(zip(("k_scale", "v_scale"), tensors[6:]))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    run = api.RunCall(plan, q, k, v, bt, out, ws, **scales)
    calls = [run.with_events(e) for e in evs]
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if flush is not None:
            flush()
        run()
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    for _ in range(5):
        run()
    # the cost of one event record on the GPU's queue: pairs of events with nothing between
    empty = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(8)]
    for a, b in empty:
        a.record()
        b.record()
    for i in range(steps):
        if flush is not None:
            flush()
        calls[i]()
    torch.cuda.synchronize()
    stage = {s: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) for j, s in enumerate(STAGES)}
    stage["event_record"] = float(np.median([a.elapsed_time(b) for a, b in empty]))
    totals = [e[0].elapsed_time(e[3]) for e in evs]
    return wall, stage, totals


LAYERS = 32     # attention layers of the model the headline iteration is shaped on (Llama-2-7B)
# untimed runs before a secondary line's timed ones (a new workload's first runs are slower)
SECONDARY_WARMUP = 10


def time_graph(api, plan, tensors, steps, warmup, layers=LAYERS, settle_s=0.0, launches=1):
    """Steps as a model's forward issues them: run i reads and writes the buffers of layer
    i % layers (each layer its own copy of Q, K, V and the output, so no layer finds the
    previous layer's data in the last-level cache; one plan and workspace for all, as in
    an iteration), all `steps` runs captured in one HIP graph (run is enqueue-only).
    Untimed: `warmup` runs replayed from a graph of their own (the graph replayed again
    until `settle_s` seconds have passed), then one launch of the timed graph (a graph's
    first launch also uploads it).  Timed: one launch of the graph
    of `steps` runs between synchronisations, by the wall clock.  Returns (ms/step, ms/step
    with one graph launch per run, ms/step between HIP events recorded on the launch stream
    around the timed graph launch, the graph replays before it, and the events' ms/step of
    each of `launches` timed launches)."""
    import torch
    q, k, v, bt, out, ws = tensors[:6]
    scales = dict(zip(("k_scale", "v_scale"), tensors[6:]))
    sets = [(q, k, v, out)] + [(q.clone(), k.clone(), v.clone(), torch.empty_like(out)) for _ in range(layers - 1)]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        calls = [api.RunCall(plan, a, b, c, bt, d, ws, stream=s, **scales) for a, b, c, d in sets]
        for c in calls:
            c()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(n):
                calls[i % layers]()
        return g

    g_warm, g_steps = capture(max(1, warmup)), capture(steps)
    # the host work of the captures leaves the GPU idle long enough for its clock to drop:
    # replay the warm-up graph for `settle_s` before the timed launch
    n_warm, t0 = 0, time.perf_counter()
    while True:
        g_warm.replay()
        n_warm += 1
        if n_warm % 16 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= settle_s:
                break
    g_steps.replay()
    torch.cuda.synchronize()
    per_launch = []
    for _ in range(launches):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        e0.record()
        g_steps.replay()
        e1.record()
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        per_launch.append(e0.elapsed_time(e1) / steps)
    ms_events = per_launch[0]
    # the same runs launched one graph each (launch overhead per run included)
    g1 = capture(1)
    g1.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g1.replay()
    torch.cuda.synchronize()
    ms_single = (time.perf_counter() - t0) * 1e3 / steps
    del g_warm, g_steps, g1, calls, sets
    torch.cuda.empty_cache()
    return ms, ms_single, ms_events, n_warm * max(1, warmup), per_launch


def setup(api, w, flags=0):
    import torch
    plan = api.plan_for(w, flags=flags)
    q, k, v, bt = api.to_device(w)
    out = torch.zeros_like(q)
    ws = api.new_workspace(plan)
    scales = api.scales_to_device(w) if w.dtype == "fp8" else ()
    return plan, (q, k, v, bt, out, ws) + tuple(scales)


def dominant(stats, stage_ms):
    """The stage with the largest time, with its algorithmic work and roofline bound.  Its
    time is the span between the library's events around it less the cost of recording
    one event (measured in the same pass), i.e. the kernel's own duration."""
    kernels = {k: v for k, v in stage_ms.items() if k in STAGES}
    name = max(kernels, key=kernels.get)
    ms = kernels[name] - stage_ms.get("event_record", 0.0)
    if name == "prefill":
        # every MFMA tile (prefill rows, decodes run as tiles, key chunks, shared-prefix group
        # tiles and members' own keys): all work not done by split-KV items; MFMA-bound unless
        # the tiles mostly stream KV
        flops = stats["flops"] - stats["split_item_flops"]
        qo = stats["q_bytes"] if stats["split_items"] == 0 else stats["q_bytes"] - stats["split_q_bytes"]
        byts = stats["physical_kv_bytes"] - stats["split_item_kv_bytes"] + 2 * qo
        bound = "mfma" if flops / PEAK_BF16 > byts / PEAK_HBM else "hbm"
        work = flops if bound == "mfma" else byts
    elif name == "split_kv":
        # bandwidth-bound unless it also carries the prefill rows (then it is a contraction)
        flops = stats["split_item_flops"]
        byts = stats["split_item_kv_bytes"] + stats["split_q_bytes"] + stats["table_bytes"]
        bound = "mfma" if flops / PEAK_BF16 > byts / PEAK_HBM else "hbm"
        work = flops if bound == "mfma" else byts
    else:
        work, bound = stats["o_bytes"], "hbm"
    return name, ms, work, bound


def roofline(stats, stage_ms, workload=None, fp8=False, kernel_ms=None):
    """kernel_ms, when given, replaces the event-pass time of the dominant kernel."""
    names = KERNEL_NAMES_FP8 if fp8 else KERNEL_NAMES
    name, ms, work, bound = dominant(stats, stage_ms)
    if kernel_ms is not None:
        ms = kernel_ms
    traffic = measured_traffic(workload, names[name]) if workload else None
    sec = ms * 1e-3
    if bound == "mfma":
        a, p, unit = work / sec / 1e12, PEAK_BF16 / 1e12, "TFLOP/s"
    else:
        a, p, unit = work / sec / 1e9, PEAK_HBM / 1e9, "GB/s"
    return {"bound": bound, "achieved": round(a, 2), "peak": p, "unit": unit, "frac": round(a / p, 4),
            "traffic": traffic, "kernel": names[name], "kernel_ms": round(ms, 5),
            "algorithmic_per_launch": work}


def cpu_baseline(w, budget_s=15.0):
    """The fp64 oracle on a bounded sample of the same iteration: the last n rows of the
    4096-row prefill (as a chunk whose cached prefix is the first 4096-n positions) plus
    both decodes.  n is grown until the run takes about budget_s / 2.."""
    import oracle
    from varlen_paged_attention_amd import workloads as W
    threads = max(1, min(16, os.cpu_count() or 1))

    def sample(n):
        s = W.Workload(**{**w.__dict__})
        a0, a1 = int(w.q_start[0]), int(w.q_end[0])
        rows = np.r_[a1 - n:a1, a1:w.total_q_rows]
        s.q = w.q[rows]
        s.q_start = np.array([0, n, n + 1], np.int32)
        s.q_end = np.array([n, n + 1, n + 2], np.int32)
        return s

    n, spent = 32, 0.0
    while True:
        s = sample(n)
        t0 = time.perf_counter()
        oracle.varlen_paged_attention(s.q, s.k_pool, s.v_pool, s.block_table, s.q_start, s.q_end, s.kv_len,
                                      s.page_size, threads=threads)
        dt = time.perf_counter() - t0
        spent += dt
        if dt > budget_s / 2 or n >= 4096 or spent > budget_s:
            break
        n = min(4096, n * 4 if dt < budget_s / 16 else n * 2)
    reps = 1
    if n >= 4096 and dt < budget_s / 2:
        # the whole iteration takes less than the budget: repeat it to fill about half of it
        reps = max(1, int(budget_s / 2 / dt))
        t0 = time.perf_counter()
        for _ in range(reps):
            oracle.varlen_paged_attention(s.q, s.k_pool, s.v_pool, s.block_table, s.q_start, s.q_end, s.kv_len,
                                          s.page_size, threads=threads)
        dt = (time.perf_counter() - t0) / reps
    flops = oracle.attention_flops(s.q_end - s.q_start, s.kv_len, s.num_q_heads, s.head_dim)
    hc = host_cpu()
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"last {n} rows of the 4096-row prefill (cached prefix {4096 - n}) + both decodes, all 32 heads, "
                      f"fp64 NumPy, {threads} threads, {dt:.2f} s per iteration"
                      + (f" (mean of {reps} runs, {dt * reps:.1f} s)" if reps > 1 else ""),
            "seconds": round(dt, 3), "runs": reps, **hc}


def hbm_read_gbps(api):
    """The library's streaming-read kernel over 8 GiB (the 256 MB last-level cache cannot
    hold it): the achievable HBM read rate, the ceiling bandwidth-bound kernels are also
    compared against."""
    import torch
    n = 8 << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(2):
        api.varlen_attn_debug_stream_read(buf, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        api.varlen_attn_debug_stream_read(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    res = round(n * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del buf
    torch.cuda.empty_cache()
    return res


def hbm_copy_gbps():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    return round(2 * n * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)


def append_line(api, W, cid, label, reps=50, dtype=None):
    """Time varlen_attn_append_kv (fp8: varlen_attn_append_kv_fp8, which also quantises) for
    one iteration's new rows (their slots from the plan); algorithmic bytes = new K/V read +
    what is written (the same bytes; fp8: codes + one float32 scale per vector) + the slot
    indices."""
    import torch
    w = W.config(cid, dtype=dtype)
    plan = api.plan_for(w, flags=api.VA_FLAG_HOST_ONLY)
    loc = torch.from_numpy(api.varlen_attn_plan_slots(plan)).cuda()
    _, k, v, _ = api.to_device(w)
    T = int(loc.numel())
    fp8 = w.dtype == "fp8"
    dt = torch.bfloat16 if fp8 else k.dtype
    k_new = torch.randn(T, w.num_kv_heads, w.head_dim, device="cuda").to(dt)
    v_new = torch.randn_like(k_new)
    args = dict(num_kv_heads=w.num_kv_heads, head_dim=w.head_dim, page_size=w.page_size, num_pages=w.num_pages,
                k_new=k_new, v_new=v_new, out_cache_loc=loc, k_pool=k, v_pool=v)
    if fp8:
        ks, vs = api.scales_to_device(w)
        args.update(k_scale=ks, v_scale=vs)
        call = api.varlen_attn_append_kv_fp8
    else:
        args.update(dtype=w.dtype)
        call = api.varlen_attn_append_kv
    for _ in range(5):
        call(**args)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        call(**args)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    written = 2 * k_new.numel() * (1 if fp8 else k_new.element_size()) + (2 * 4 * T * w.num_kv_heads if fp8 else 0)
    byts = 2 * k_new.numel() * k_new.element_size() + written + 8 * T
    return {"workload": label, "us_per_step": round(us, 2), "hbm_GBps": round(byts / (us * 1e-6) / 1e9, 1),
            "hbm_frac": round(byts / (us * 1e-6) / PEAK_HBM, 4), "algorithmic_bytes": byts, "tokens": T}


def long_context_line(api, W, reps=10):
    """256 decodes at 128K context (524,288 block-table entries, 137 GB of bf16 K/V made on
    the device): planner time, block-table upload, eager per-stage times and the
    graph-captured step."""
    import torch
    w = W.config(8)
    plan = api.plan_for(w)                    # first plan of the process loads the kernels
    t0 = time.perf_counter()
    plan = api.plan_for(w)
    plan_ms = (time.perf_counter() - t0) * 1e3
    t0 = time.perf_counter()
    api.plan_for(w, flags=api.VA_FLAG_HOST_ONLY)
    plan_host_only_ms = (time.perf_counter() - t0) * 1e3
    st = api.varlen_attn_plan_stats(plan)
    q, k, v, bt = api.to_device(w)
    out = torch.zeros_like(q)
    ws = api.new_workspace(plan)
    # block-table upload from pinned host memory (what a serving loop copies every step)
    bt_host = torch.from_numpy(np.ascontiguousarray(w.block_table)).pin_memory()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    bt.copy_(bt_host, non_blocking=True)
    e0.record()
    for _ in range(reps):
        bt.copy_(bt_host, non_blocking=True)
    e1.record()
    torch.cuda.synchronize()
    h2d_us = e0.elapsed_time(e1) * 1e3 / reps
    _, stage, totals = time_runs(api, plan, (q, k, v, bt, out, ws), reps, 2)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call = api.RunCall(plan, q, k, v, bt, out, ws, stream=s)
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call()
    g.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_us = e0.elapsed_time(e1) * 1e3 / reps
    byts = st["physical_kv_bytes"] + st["q_bytes"] + st["o_bytes"] + st["table_bytes"]
    res = {"workload": "long-context decode: 256 x 128K positions (524,288 table entries), Hq=32 Hkv=8 D=128, "
                       "page 64, bf16 (hashed page values made on the device)",
           "us_per_step_graph": round(graph_us, 1), "us_per_step_eager": round(float(np.median(totals)) * 1e3, 1),
           "hbm_GBps": round(byts / (graph_us * 1e-6) / 1e9, 1), "hbm_frac": round(byts / (graph_us * 1e-6) / PEAK_HBM, 4),
           "algorithmic_bytes": byts, "plan_ms": round(plan_ms, 2), "plan_ms_host_only": round(plan_host_only_ms, 2),
           "plan_host_us_lib": round(st["plan_host_us"], 1),
           "split_items": st["split_items"], "block_table_h2d_us": round(h2d_us, 2), "table_bytes": st["table_bytes"],
           "stage_ms": {kk: round(vv, 5) for kk, vv in stage.items()}, "roofline": roofline(st, stage, "long128k")}
    del q, k, v, bt, out, ws, g
    return res


def make_flush():
    """A callable that evicts the 256 MB last-level cache by reading 1 GiB (a read leaves no
    dirty lines whose write-back the timed kernels would pay for)."""
    import torch
    buf = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()

    def flush():
        buf.sum()
    return flush


def graph_layers(w):
    """Layer copies for a graph-timed line: enough that the rotating buffers hold over 1 GiB
    (four times the 256 MB last-level cache), so no run finds its K/V there from the runs
    before it; at least 2, at most LAYERS."""
    per = w.k_pool.nbytes + w.v_pool.nbytes + 2 * w.q.nbytes
    return int(min(LAYERS, max(2, -(-(1 << 30) // max(1, per)) + 1)))


def secondary(api, W, cid, flags, reps, label, flush, key=None, dtype=None, tp=1, dp=1, w=None, graph=True):
    """Time one workload (config `cid`, or the given Workload `w`); returns the full record
    (see compact()).  The step: `reps` runs captured in one HIP graph over graph_layers(w)
    copies of its buffers, so consecutive runs read different K/V as consecutive layers do,
    launched five times (median, min and max of the HIP-event time per run around each
    launch); a run of a single-launch plan is that kernel, whose time this also is.  With
    graph=False (a line defined by evicting the cache before every run) the step is the span
    of eager runs between the library's first and last events less the three event records
    inside it.  Per-kernel times come from eager runs with the library's stage events (after
    `flush`, if given), each stage less the cost of one event record: measured in place as
    the empty split-KV stage when the plan has no split-KV items."""
    if w is None:
        w = W.config(cid, dtype=dtype, tp=tp, dp=dp)
    plan, tensors = setup(api, w, flags)
    st = api.varlen_attn_plan_stats(plan)
    settled = settle_clocks(api, plan, tensors, 0.1)     # the workload's build and planning left the GPU idle
    _, stage, totals = time_runs(api, plan, tensors, reps, SECONDARY_WARMUP, flush)
    if st["split_items"] == 0:
        stage["event_record"] = stage["split_kv"]        # no kernel between those two events
    one_launch = st["split_items"] == 0 and st["combine_rows"] == 0
    kernel_ms = None
    if graph:
        layers = graph_layers(w)
        *_, per_launch = time_graph(api, plan, tensors, reps, SECONDARY_WARMUP, layers=layers, settle_s=0.05,
                                    launches=5)
        steps_us = [x * 1e3 for x in per_launch]
        us = float(np.median(steps_us))
        lo, hi = min(steps_us), max(steps_us)
        kernel_ms = us * 1e-3 if one_launch else None
        how = f"one hip-graph launch of {reps} runs over {layers} layers' buffers, median of 5 launches (min, max)"
    else:
        # the step's time less the cost of the three event records inside it (see dominant())
        steps_us = [(t - 3 * stage.get("event_record", 0.0)) * 1e3 for t in totals]
        us = float(np.median(steps_us))
        lo, hi = float(np.percentile(steps_us, 10)), float(np.percentile(steps_us, 90))
        how = f"{reps} eager runs, the last-level cache evicted before each (median, p10, p90)"
    byts = st["physical_kv_bytes"] + st["q_bytes"] + st["o_bytes"] + st["table_bytes"]
    # time at the roofline if the FLOPs and the bytes could not overlap at all
    t_roof_us = (st["flops"] / PEAK_BF16 + byts / PEAK_HBM) * 1e6
    res = {"workload": label, "us_per_step": round(us, 2),
           "us_p10": round(lo, 2), "us_p90": round(hi, 2), "timing": how,
           "t_roof_us": round(t_roof_us, 2), "t_roof_frac": round(t_roof_us / us, 4),
           "share": {"tp": tp, "dp": dp} if tp > 1 or dp > 1 else None,
           "hbm_GBps": round(byts / (us * 1e-6) / 1e9, 1), "hbm_frac": round(byts / (us * 1e-6) / PEAK_HBM, 4),
           "tflops": round(st["flops"] / (us * 1e-6) / 1e12, 2),
           "algorithmic_bytes": byts, "logical_kv_bytes": st["logical_kv_bytes"],
           "physical_kv_bytes": st["physical_kv_bytes"], "flops": st["flops"],
           "stage_ms": {k: round(v, 5) for k, v in stage.items()},
           "roofline": roofline(st, stage, key, fp8=w.dtype == "fp8", kernel_ms=kernel_ms),
           "l2_flushed": flush is not None, "settle_runs": settled,
           "dtype": w.dtype}
    del tensors
    return res


def compact(res, key):
    """The short form of a secondary record kept in the JSON line: median step (p10/p90),
    algorithmic rates over the step, and the dominant kernel's roofline fraction."""
    rf = res.get("roofline") or {}
    out = {"w": key, "us": res.get("us_per_step", res.get("us_per_step_graph")),
           "p10": res.get("us_p10"), "p90": res.get("us_p90"),
           "GBps": res.get("hbm_GBps"), "hbm_frac": res.get("hbm_frac"), "TFLOPs": res.get("tflops"),
           "t_roof_frac": res.get("t_roof_frac")}
    if rf:
        out["kernel"] = {"name": rf["kernel"].replace("_kernel", ""), "us": round(rf["kernel_ms"] * 1e3, 1),
                         "bound": rf["bound"], "frac": rf["frac"], "traffic": rf.get("traffic")}
    for k in ("plan_ms", "block_table_h2d_us", "tokens"):
        if k in res:
            out[k] = res[k]
    return {k: v for k, v in out.items() if v is not None}


def host_cpu():
    """The host the CPU baseline runs on: lscpu's model line with family/model numbers, the
    logical CPUs and those this process may use."""
    info = {}
    try:
        import subprocess
        for line in subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout.splitlines():
            k, _, v = line.partition(":")
            info[k.strip()] = v.strip()
    except Exception:
        pass
    model = info.get("Model name") or cpu_model()
    fam = info.get("CPU family")
    desc = model + (f" (family {fam}, model {info.get('Model')})" if fam else "")
    if info.get("Hypervisor vendor"):
        desc += f", under {info['Hypervisor vendor']}"
    return {"cpu": desc, "nproc": os.cpu_count(), "usable_cpus": len(os.sched_getaffinity(0)),
            "cores_per_socket": int(info["Core(s) per socket"]) if info.get("Core(s) per socket", "").isdigit() else None,
            "threads_per_core": int(info["Thread(s) per core"]) if info.get("Thread(s) per core", "").isdigit() else None}


def targets(rec, full):
    """Each configuration of the pages' workloads with its time, bound and roofline fraction
    (kernel fractions from the dominant kernel's own time, step fractions from the step)."""
    def kern(res):
        r = res["roofline"]
        return {"kernel": r["kernel"].replace("_kernel", ""), "kernel_us": round(r["kernel_ms"] * 1e3, 1),
                "bound": r["bound"], "kernel_frac": r["frac"]}
    t = {"1_tiny_f32": "parity only (max |gpu - oracle| <= 1e-4 in the GPU tests)",
         "2_orca_mixed": {"us": round(rec["ms_per_step"] * 1e3, 1), "bound": "mfma", "frac": rec["roofline"]["frac"],
                          "TFLOPs": rec["value"], "target": ">= 0.50 of 2.5 PFLOP/s"}}
    d = full["decode"]
    t["3_decode_heavy"] = {"us": d["us_per_step"], "hbm_frac_step": d["hbm_frac"], **kern(d),
                           "target": ">= 0.70 of 8 TB/s"}
    c, ca, cd = full["chunk"], full["chunk_alone"], full["chunk_decodes"]
    t["4_chunk_mix"] = {"us": c["us_per_step"], "t_roof_frac": c["t_roof_frac"], **kern(c),
                        "chunk_alone_us": ca["us_per_step"], "chunk_alone_mfma_frac": ca["roofline"]["frac"],
                        "decodes_alone_us": cd["us_per_step"], "decodes_alone_hbm_frac": cd["hbm_frac"],
                        "decodes_alone_kernel_frac": cd["roofline"]["frac"],
                        "target": "both fractions; decodes >= 0.70 of 8 TB/s"}
    for key, name, goal in (("shared6", "5_shared_prefix_6", None), ("shared64", "5_shared_prefix_64_scaled", ">= 0.70")):
        x = full[key]
        t[name] = {"us": x["us_per_step"], "hbm_frac_physical": x["hbm_frac"], **kern(x),
                   "physical_MiB": round(x["physical_kv_bytes"] / 2**20, 1),
                   "logical_MiB": round(x["logical_kv_bytes"] / 2**20, 1),
                   "no_llc_reuse": "step over rotating layers' buffers; kernel time with the cache evicted"}
        if goal:
            t[name]["target"] = goal + " of 8 TB/s on physical bytes"
    return t


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true")
    ap.add_argument("--only", type=int, default=None,
                    help="profile mode: time only this workload (2-9 or 51) and print its line")
    ap.add_argument("--fp8", action="store_true", help="with --only: the workload in fp8 KV storage")
    ap.add_argument("--shard", default=None,
                    help="with --only: one GPU's share of the workload split over GPUs, tpN (by head) or dpN "
                         "(by request)")
    ap.add_argument("--copy-only", action="store_true",
                    help="profile mode: 10 device copies of 1 GiB (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); this library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from varlen_paged_attention_amd import api, workloads as W
    torch.cuda.set_device(0)
    api.lib()
    if args.copy_only:
        print(json.dumps({"copy_GBps": hbm_copy_gbps(), "bytes_per_copy": 2 * (1 << 30)}), flush=True)
        return
    if args.only == 8:
        print(json.dumps(long_context_line(api, W, max(2, args.steps))), flush=True)
        return
    if args.only is not None:
        flags = api.VA_FLAG_SHARED_PREFIX if args.only in (5, 51) else 0
        key = {2: "orca", 3: "decode", 4: "chunk", 5: "shared6", 51: "shared64", 6: "mtp3", 7: "mtp7",
               9: "longchunk"}.get(args.only)
        if args.fp8:
            key += "_fp8"
        fl = make_flush() if args.only in (5, 51) else None     # as in the secondary lines
        tp = dp = 1
        if args.shard:
            kind, n = args.shard[:2], int(args.shard[2:])
            tp, dp = (n, 1) if kind == "tp" else (1, n)
            key = None                                           # no committed counters for shares
        res = secondary(api, W, args.only, flags, args.steps, W.CONFIG_NAMES[args.only], fl, key,
                        "fp8" if args.fp8 else None, tp=tp, dp=dp)
        print(json.dumps(res), flush=True)
        return

    log("[bench] building the ORCA mixed iteration (4096 prefill + decodes 1500, 1700)")
    w = W.config(2)
    api.plan_for(w)                          # the first plan of the process loads the kernels
    plan, tensors = setup(api, w)
    st = api.varlen_attn_plan_stats(plan)
    log(f"[bench] plan: {st['prefill_tiles']} prefill tiles, {st['split_items']} split items, "
        f"{st['plan_host_us']:.0f} us host (incl. the upload of the work lists)")
    # per-kernel times: eager runs with the library's stage events; the step itself: the
    # same run captured in a HIP graph and replayed (no per-launch host gaps)
    settled = settle_clocks(api, plan, tensors)
    wall_eager, stage, totals = time_runs(api, plan, tensors, args.steps, args.warmup)
    ms, ms_single, ms_graph_events, settled_graph, _ = time_graph(api, plan, tensors, args.steps, args.warmup,
                                                                  settle_s=CLOCK_SETTLE_S)
    value = st["flops"] / (ms * 1e-3) / 1e12
    # a run of this plan is one launch of the prefill kernel (its decodes ride in it as
    # tiles), so the timed graph launch is that kernel back to back: its average launch
    # duration over the timed region is the event span / steps (gaps between launches
    # included); the event pass's own figure is kept beside it
    one_launch = st["split_items"] == 0 and st["combine_rows"] == 0
    roof = roofline(st, stage, "orca", kernel_ms=ms_graph_events if one_launch else None)
    roof["kernel_ms_event_pass"] = roofline(st, stage)["kernel_ms"]
    if one_launch:
        roof["kernel_ms_from"] = f"HIP events around the timed graph launch ({args.steps} launches)"
    log(f"[bench] {ms:.4f} ms/step (one graph of {args.steps} runs; one graph per run {ms_single:.4f}; "
        f"eager {wall_eager:.4f})  {value:.1f} TFLOP/s  stages {stage}")

    rec = {"metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "clock_settle": {"seconds": CLOCK_SETTLE_S, "runs_before_eager_pass": settled,
                                                 "graph_replayed_runs_before_timed_launch": settled_graph},
           "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded N(0,1) Q/K/V cast to bf16)",
           "config": {"workload": "orca-mixed-llama7b: one layer; prefill q_rows=4096 kv=4096 + decodes (1,1500), "
                                  "(1,1700); Hq=Hkv=32, head_dim=128, page_size=16, permuted pages, bf16",
                      "total_q_rows": int(w.total_q_rows), "flops_per_step": st["flops"],
                      "kv_bytes": st["physical_kv_bytes"]},
           "launch": f"one hip-graph launch of {args.steps} varlen_attn_run calls over {LAYERS} layers' buffers",
           "ms_per_step_one_graph_per_run": round(ms_single, 5), "ms_per_step_eager": round(wall_eager, 5),
           "plan_host_us": round(st["plan_host_us"], 1),
           "stage_ms": {k: round(v, 5) for k, v in stage.items()},
           "peak_frac": round(value * 1e12 / PEAK_BF16, 4),
           "roofline": roof}
    del tensors
    torch.cuda.empty_cache()

    if not args.no_secondary:
        flush = make_flush()
        full = {}

        def add(key, res):
            full[key] = res
            log(f"[bench] full {key}: " + json.dumps(res))

        w4 = W.config(4)
        for cid, flags, label, fl, key, dt, wl in (
                (3, 0, "decode-heavy-gqa (256 decodes, kv U[1024,8192], g=4, page 64)", None, "decode", None, None),
                (4, 0, "chunked-prefill-mix (2048@S0=30720 + 64 decodes, g=8)", None, "chunk", None, w4),
                (4, 0, "chunked-prefill-mix: the 2048-row chunk alone", None, "chunk_alone", None, W.subset(w4, [0])),
                (4, 0, "chunked-prefill-mix: the 64 decodes alone", None, "chunk_decodes", None,
                 W.subset(w4, range(1, w4.num_reqs))),
                (9, 0, "long-prefix-chunk (256@S0=65536 + 64 decodes, g=4; key-chunk tiles)", None, "longchunk",
                 None, None),
                (5, api.VA_FLAG_SHARED_PREFIX, "shared-prefix-6 (4096 shared + 1024 each)", flush, "shared6", None,
                 None),
                (51, api.VA_FLAG_SHARED_PREFIX, "shared-prefix-64 (16384 shared + 1024 each)", flush, "shared64",
                 None, None),
                (6, 0, "spec-decode verify, 4 rows/request", None, "mtp3", None, None),
                (7, 0, "spec-decode verify, 8 rows/request", None, "mtp7", None, None),
                (3, 0, "decode-heavy-gqa, fp8 KV + scales", None, "decode_fp8", "fp8", None),
                (51, api.VA_FLAG_SHARED_PREFIX, "shared-prefix-64, fp8 KV + scales", flush, "shared64_fp8", "fp8",
                 None),
                (4, 0, "chunked-prefill-mix, fp8 KV + scales", None, "chunk_fp8", "fp8", None),
                (2, 0, "orca-mixed, fp8 KV + scales", None, "orca_fp8", "fp8", None)):
            log(f"[bench] secondary: {label}")
            add(key, secondary(api, W, cid, flags, 20, label, fl, key if wl is None or key == "chunk" else None, dt,
                               w=wl))
            torch.cuda.empty_cache()
        del w4
        log("[bench] secondary: the ORCA iteration with the last-level cache evicted before each run")
        add("orca_llc_evicted", secondary(api, W, 2, 0, 20, "orca-mixed, last-level cache evicted before each run",
                                          flush, None, graph=False))
        # one GPU's share when the iteration is split over 8 GPUs (the kernels at their real shape)
        for cid, tp, dp, key in ((4, 8, 1, "chunk_tp8"), (2, 8, 1, "orca_tp8"), (3, 1, 8, "decode_dp8")):
            log(f"[bench] secondary: {key}")
            add(key, secondary(api, W, cid, 0, 20, key, None, None, tp=tp, dp=dp))
            torch.cuda.empty_cache()
        log("[bench] secondary: long-context decode 256 x 128K")
        add("long128k", long_context_line(api, W))
        torch.cuda.empty_cache()
        for cid, key, dt in ((2, "append_orca", None), (3, "append_decode", None), (2, "append_orca_fp8", "fp8"),
                             (3, "append_decode_fp8", "fp8")):
            log(f"[bench] secondary: {key}")
            add(key, append_line(api, W, cid, key, dtype=dt))
            torch.cuda.empty_cache()
        copy_gbps = hbm_copy_gbps()
        read_ceiling = hbm_read_gbps(api)
        sec = [compact(res, key) for key, res in full.items()]
        sec.append({"w": "copy_1GiB_torch", "GBps": copy_gbps})
        sec.append({"w": "stream_read_8GiB", "GBps": read_ceiling, "hbm_frac": round(read_ceiling * 1e9 / PEAK_HBM, 4)})
        rec["secondary"] = sec
        rec["targets"] = targets(rec, full)
        del flush

    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle on a bounded sample")
        rec["cpu_baseline"] = cpu_baseline(w)
    else:
        rec["cpu_baseline"] = None
    if "targets" in rec:
        rec["targets"] = rec.pop("targets")       # last, so a reader of the line's tail sees it
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
