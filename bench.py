#!/usr/bin/env python3
"""Benchmark of the fused reduce + residual-add + RMSNorm step on one MI355X.

A step is one pass of the hot path over one batch of the workload: the host
split plan for the batch (integer arithmetic, microseconds) and the fused
kernel launch(es) it calls for.  At the default workload (Llama-3-70B-shaped:
T=1024 tokens, h=8192, N=8 bf16 partials) the planner keeps the batch whole
(its GEMM is one wave on 256 CUs), so a step is one fused launch.

Timing: a settle of as many steps as take about 100 ms (from a pause the GPU
needs about 30 ms of load to reach its steady speed; it always runs and is
reported as `settle`), then W untimed warm-up steps, then K timed steps back
to back on the current torch stream -- the stream the library enqueues on --
between two HIP events, with torch.cuda.synchronize() on both sides.  The
host launches every step; with --graph the same launches are recorded into
HIP graphs and the timed steps are graph replays.
Whole buffer sets (inputs and outputs) rotate so that the inputs, and the
outputs on their own, touched between two uses of one set each exceed twice
the 256 MB last-level (MALL) cache: reads are served by HBM, and no output
buffer stays resident in that cache to absorb its writes.

Printed: one JSON line.  `value` is algorithmic GB/s, (N+1 reads + 2 writes)
x T x h x sizeof(bf16) per step over the measured time per step; `roofline`
prices the same bytes against the 8 TB/s HBM peak; `cpu_baseline` times the
float64 CPU oracle on a bounded sample of the same workload on one host core.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, decimal GB/s
MALL_BYTES = 256 * 1000 * 1000  # MI355X Infinity Cache (last-level, memory side)
MAX_ROTATE = 2048
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fused_reduce_rmsnorm_llama70b_traffic.json")
METRIC = "fused reduce-add-RMSNorm HBM GB/s (% of peak), h=8192 T=1024 N=8 bf16"

# From a pause, the GPU needs about 30 ms of sustained load before launches
# reach their steady time (its power management ramps up the clocks): the first
# ~1000 fused launches of the 1024-row workload take 31-33 us each, the rest
# 30.8 us (bench.py --ramp).  Before the requested warm-up steps the bench
# therefore always settles the GPU with about three times that much work.
SETTLE_SECONDS = 0.1
DEFAULT_WARMUP = 20
RAMP_BLOCKS, RAMP_BLOCK = 60, 100
EMPTY_LAUNCHES = 200

# GEMM tile model for the split planner: 256x256 output tiles, one CTA per CU.
GEMM_TILE = 256


def kernel_source_hash() -> str:
    from reduce_rmsnorm_amd.rocprof_summary import kernel_code_hash
    return kernel_code_hash()


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=DEFAULT_WARMUP,
                    help="untimed warm-up steps, run after a settle of about %.0f ms of the "
                         "same steps (which always runs, so that the GPU has reached its "
                         "steady speed under load before the timed steps)"
                         % (1e3 * SETTLE_SECONDS))
    ap.add_argument("--settle-ms", type=float, default=1e3 * SETTLE_SECONDS,
                    help="GPU work, in ms, of the settle that precedes the warm-up (default "
                         "%(default)s; counter passes under a profiler, which serializes every "
                         "dispatch, set 0)")
    ap.add_argument("--ramp", action="store_true",
                    help="also time the first %d steps after a short pause, in blocks of %d: "
                         "the ramp that the warm-up covers" % (RAMP_BLOCKS * RAMP_BLOCK,
                                                                     RAMP_BLOCK))
    ap.add_argument("--workload", default="llama70b")
    ap.add_argument("--tokens", type=int, default=None,
                    help="override the workload's token count T (same distributions)")
    ap.add_argument("--partials", type=int, default=None,
                    help="override the workload's partial count N (same distributions)")
    ap.add_argument("--hidden", type=int, default=None,
                    help="override the workload's hidden size h (same distributions)")
    ap.add_argument("--no-split", dest="split", action="store_false",
                    help="keep every batch whole (one launch per step) whatever the planner says")
    ap.add_argument("--mode", choices=("full", "shard"), default="full",
                    help="full: every row; shard: shard 0's rows (one rank's share)")
    ap.add_argument("--rotate", type=int, default=0,
                    help="buffer sets to rotate through (0: enough that the inputs, and the "
                         "outputs on their own, each exceed 2x the MALL; at most 2048)")
    ap.add_argument("--graph", action="store_true",
                    help="time the steps as replays of HIP graphs that hold the same launches "
                         "(default: every step launched from the host)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="budget of the CPU oracle sample (0 disables the cpu_baseline leg)")
    ap.add_argument("--no-unfused", dest="unfused", action="store_false",
                    help="skip timing the unfused comparator (standalone reduce, then a "
                         "two-pass residual-add + RMSNorm) in full mode")
    ap.add_argument("--footprint", action="store_true",
                    help="also sweep the fused kernel over a fixed number of workgroups "
                         "(2 .. one per row): GB/s against the CUs the launch may occupy")
    ap.add_argument("--overlap", action="store_true",
                    help="also time one tensor-parallel layer step (row-parallel GEMM + fused "
                         "step) unsplit and split in two on two streams, for every offset, at "
                         "several token counts: the measured offset sweep")
    ap.add_argument("--overlap-tokens", default="1024,2048,4096,8192",
                    help="token counts of the --overlap sweep (comma separated)")
    ap.add_argument("--overlap-lean", action="store_true",
                    help="--overlap: time only the unsplit step and the split offsets (no "
                         "confined-workgroup or per-component runs), for long token lists")
    ap.add_argument("--split-table", action="store_true",
                    help="also time the fused step alone as two launches (prefix, suffix) for "
                         "every offset, next to one launch over all rows")
    ap.add_argument("--gemm-staircase", action="store_true",
                    help="also time the layer's row-parallel GEMM alone for M = 64 .. 8192 "
                         "rows in steps of 64: where its time steps up shows the GEMM's "
                         "row tile and waves, which the split planner models")
    ap.add_argument("--cu-mask", action="store_true",
                    help="also run the fused kernel on CU-masked streams: where mask bits land "
                         "(XCD, CU), GB/s against the number of CUs, and the split layer step "
                         "with the fused kernel and the GEMM on disjoint CU sets")
    ap.add_argument("--host-cost", action="store_true",
                    help="also time the host side of one call through the binding (eager with "
                         "stacked or listed partials, prepared, shard, split plan lookup) on a "
                         "64-row launch the GPU keeps up with")
    ap.add_argument("--launch-floor", action="store_true",
                    help="also time an empty kernel of 1, 256, 1024 and 4096 workgroups, "
                         "replayed from a HIP graph: the fixed cost of a dependent launch")
    ap.add_argument("--ceiling", action="store_true",
                    help="also time the bandwidth probes on the same buffers: N+1 streamed reads "
                         "+ 2 streamed writes, reads only, writes only (the achievable envelope; "
                         "their known byte counts also calibrate the hardware counters)")
    return ap.parse_args()


def run_ramp(torch, step, stream) -> dict:
    """Launch time from a pause: after 0.5 s idle and 20 launches, time
    RAMP_BLOCKS blocks of RAMP_BLOCK steps back to back, one HIP event pair
    per block."""
    for i in range(20):
        step(i)
    torch.cuda.synchronize()
    time.sleep(0.5)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(RAMP_BLOCKS + 1)]
    ev[0].record(stream)
    for b in range(RAMP_BLOCKS):
        for i in range(RAMP_BLOCK):
            step(b * RAMP_BLOCK + i)
        ev[b + 1].record(stream)
    torch.cuda.synchronize()
    us = [round(ev[b].elapsed_time(ev[b + 1]) * 1e3 / RAMP_BLOCK, 3) for b in range(RAMP_BLOCKS)]
    steady = statistics.median(us[RAMP_BLOCKS // 2:])
    settled = next((b for b in range(RAMP_BLOCKS) if all(x <= 1.01 * steady for x in us[b:])),
                   RAMP_BLOCKS)
    ms_to_settle = sum(us[:settled]) * RAMP_BLOCK / 1e3
    print(f"[bench] ramp: first block {us[0]:.2f} us/step, steady {steady:.2f}; within 1% of "
          f"steady after {settled * RAMP_BLOCK} steps ({ms_to_settle:.1f} ms)",
          file=sys.stderr, flush=True)
    return {"block_steps": RAMP_BLOCK, "us_per_step": us, "steady_us": round(steady, 3),
            "steps_to_settle": settled * RAMP_BLOCK, "ms_to_settle": round(ms_to_settle, 2)}


def run_ceiling(tw, sets, R, rows, h, itemsize, stream, steps, timer):
    """Time the measurement-only probes of libtw_bwprobe.so over the bench's
    own rotated buffers: sources are the partial rows and the residual rows,
    destinations are out and residual_out.  Flat streams of the same bytes
    (reads and writes, reads only, writes only), and, where the row class has
    one, the schedule twins of the fused launch: its geometry, load order,
    pause, stores and row barrier without its arithmetic."""
    import ctypes
    import torch
    lib = _probe_lib()
    tensor_bytes = rows * h * itemsize
    nvec = tensor_bytes // 16
    ptrs = []
    for parts, res, out, rout in sets:
        src = [parts[i, :rows].data_ptr() for i in range(parts.shape[0])] + [res[:rows].data_ptr()]
        dst = [out.data_ptr(), rout.data_ptr()]
        ptrs.append(((ctypes.c_void_p * len(src))(*src), len(src), (ctypes.c_void_p * 2)(*dst)))
    nsrc = ptrs[0][1]
    res = {"tensor_bytes": tensor_bytes, "grid": 2048}
    for kind, key, nbytes in ((0, "read_write", (nsrc + 2) * tensor_bytes),
                              (1, "read_only", nsrc * tensor_bytes),
                              (2, "write_only", 2 * tensor_bytes)):
        def go(i, kind=kind):
            src, n, dst = ptrs[i % R]
            rc = lib.tw_probe_launch(kind, src, n, dst, 2, nvec, 2048, stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"probe launch failed: {rc}")
        us = timer(go, steps)
        res[key + "_us"] = round(us, 3)
        res[key + "_bytes"] = nbytes
        res[key + "_gbs"] = round(nbytes / (us * 1e-6) / 1e9, 1)
        print(f"[bench] probe {key}: {nbytes} B in {us:.2f} us = {res[key + '_gbs']} GB/s",
              file=sys.stderr, flush=True)
    row_vecs = h * itemsize // 16
    info = tw.tw_fused_launch_info(nsrc - 1, rows, h,
                                   torch.bfloat16 if itemsize == 2 else torch.float32, stream)
    if row_vecs in (512, 1024, 2048) and info["vectors_per_thread"] * \
            info["threads_per_workgroup"] == row_vecs:
        seq = 1 if info["kernel_name"] in ("seq", "strided") else 0
        res["twin_load_order"] = "sequenced" if seq else "all at once"
        for kind, key, nbytes in ((5, "twin_read_write", (nsrc + 2) * tensor_bytes),
                                  (6, "twin_read_only", nsrc * tensor_bytes)):
            def go(i, kind=kind):
                src, n, dst = ptrs[i % R]
                rc = lib.tw_probe_twin_launch(kind, seq, src, n, dst, nvec, rows,
                                              stream.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"twin probe launch failed: {rc}")
            us = timer(go, steps)
            res[key + "_us"] = round(us, 3)
            res[key + "_bytes"] = nbytes
            res[key + "_gbs"] = round(nbytes / (us * 1e-6) / 1e9, 1)
            print(f"[bench] schedule twin {key} ({res['twin_load_order']}): {nbytes} B in "
                  f"{us:.2f} us = {res[key + '_gbs']} GB/s", file=sys.stderr, flush=True)
    return res


HOST_COST_CALLS = 3000


def run_host_cost(tw, torch, wl, sets, w, stream, plan_kw) -> dict:
    """Host time per call of the binding, on 64-row launches (a few µs of GPU
    work each, so the GPU keeps up and the host never waits on a full queue):
    the mean wall time of HOST_COST_CALLS back-to-back calls, no
    synchronization inside the loop."""
    parts, res, out, rout = sets[0]
    p64, r64, o64, ro64 = parts[:, :64], res[:64], out[:64], rout[:64]
    listed = [parts[i, :64] for i in range(parts.shape[0])]
    prepared = tw.PreparedFused(p64, r64, w, wl.eps, o64, ro64, stream)
    # The C side of a prepared call without the launch: zero rows return right
    # after the argument checks; the launch description adds the stream's CU
    # count and the launch plan.
    prepared_empty = tw.PreparedFused(parts[:, :0], res[:0], w, wl.eps, out[:0], rout[:0], stream)
    info = tw.load_library().tw_fused_launch_info
    info_args = (parts.shape[0], 64, wl.hidden, 1 if wl.dtype == "bf16" else 0, stream.cuda_stream,
                 tw._lib.LaunchInfo())
    cache = tw.SplitPlanCache(**plan_kw)
    calls = {
        "eager_stacked": lambda: tw.tw_fused_reduce_rmsnorm(p64, r64, w, wl.eps, out=o64,
                                                            residual_out=ro64),
        "eager_listed": lambda: tw.tw_fused_reduce_rmsnorm(listed, r64, w, wl.eps, out=o64,
                                                           residual_out=ro64),
        "eager_shard": lambda: tw.tw_shard_rmsnorm(p64, r64, w, wl.eps, 0, out=o64,
                                                   residual_out=ro64),
        "prepared": prepared,
        "prepared_zero_rows": prepared_empty,
        "launch_info_c": lambda: info(*info_args),
        "split_plan_cached": lambda: cache(wl.num_tokens),
        "split_plan_c": lambda: tw.tw_split_plan(wl.num_tokens, **plan_kw),
    }
    res_us = {}
    for name, fn in calls.items():
        for _ in range(200):
            fn()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(HOST_COST_CALLS):
            fn()
        us = (time.perf_counter() - t0) * 1e6 / HOST_COST_CALLS
        torch.cuda.synchronize()
        res_us[name] = round(us, 2)
        print(f"[bench] host cost {name}: {us:.2f} us per call", file=sys.stderr, flush=True)
    return {"calls": HOST_COST_CALLS, "rows": 64, "us_per_call": res_us}


def run_launch_floor(torch, timer) -> dict:
    """The fixed cost of one dependent launch: an empty kernel of G
    workgroups of 1024 threads, EMPTY_LAUNCHES of them recorded in a HIP graph
    and replayed (eager launches this short would time the host instead).
    Kept apart from the stream probes: the counter passes run those, and HIP
    graph capture under rocprofv3 --pmc ends the profiler."""
    import ctypes
    lib = _probe_lib()
    cap = torch.cuda.Stream()
    none = (ctypes.c_void_p * 1)()
    res = {}
    for grid in (1, 256, 1024, 4096):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            for _ in range(EMPTY_LAUNCHES):
                rc = lib.tw_probe_launch(4, none, 0, none, 0, 1, grid, cap.cuda_stream)
                if rc != 0:
                    raise RuntimeError(f"empty probe launch failed: {rc}")
        for _ in range(100):            # capture idled the GPU: settle it again first
            g.replay()
        us = timer(lambda i, g=g: g.replay(), 20) / EMPTY_LAUNCHES
        res[str(grid)] = round(us, 3)
        print(f"[bench] empty kernel, {grid} workgroups of 1024 threads: {us:.2f} us per launch "
              f"(graph replay)", file=sys.stderr, flush=True)
        del g
    # Host time of one launch through each launch API (a C++ loop in the probe
    # library, so that Python does not bound it).
    host = {}
    out = ctypes.c_double()
    for api, name in ((0, "hipLaunchKernel"), (1, "hipModuleLaunchKernel"),
                      (2, "hipExtLaunchKernel")):
        for grid in (64, 1024):
            rc = lib.tw_probe_launch_cost(api, grid, 2000, cap.cuda_stream, ctypes.byref(out))
            if rc != 0:
                raise RuntimeError(f"launch cost probe failed: {rc}")
            host[f"{name}_{grid}"] = round(out.value, 3)
            print(f"[bench] host time per {name} of {grid} empty workgroups: {out.value:.2f} us",
                  file=sys.stderr, flush=True)
    res["host_us_per_launch"] = host
    return res


# Down-projection of a Llama-3-70B-shaped layer under 8-way tensor
# parallelism: intermediate 28672 / 8 = 3584 columns per rank.
OVERLAP_K = 3584


def run_gemm_staircase(tw, torch, wl, plan_kw) -> dict:
    """Time X[M, K] @ W[K, h] (bf16, ``torch.mm`` into a preallocated output,
    the layer GEMM of the overlap step) for M = 64 .. 8192 in steps of 64,
    each as the mean of graph replays of 20 back-to-back GEMMs (no host launch
    cost).  Jumps in time against M show the row tile the library picked and
    where a new wave of tiles starts; the split planner's CTA model
    (tokens_per_cta x ctas_per_token_tile on 256 CUs) is checked against
    them."""
    K, h = OVERLAP_K, wl.hidden
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    x = (torch.randn(8192, K, device="cuda", generator=g) * 0.5).to(torch.bfloat16)
    w = (torch.randn(K, h, device="cuda", generator=g) / K ** 0.5).to(torch.bfloat16)
    y = torch.empty(8192, h, device="cuda", dtype=torch.bfloat16)
    side = torch.cuda.Stream()
    points = []
    for M in range(64, 8193, 64):
        with torch.cuda.stream(side):
            torch.mm(x[:M], w, out=y[:M])       # eager first: the library's per-shape set-up
        side.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            for _ in range(20):
                torch.mm(x[:M], w, out=y[:M])
        with torch.cuda.stream(side):
            graph.replay()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(side)
            for _ in range(5):
                graph.replay()
            e1.record(side)
        side.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / 100
        points.append({"m": M, "us": round(us, 2),
                       "tflops": round(2 * M * K * h / (us * 1e-6) / 1e12, 1)})
        del graph
    # A "step" is a rise of more than 8% of the previous time between two
    # neighbouring M values.
    steps = [p["m"] for q, p in zip(points, points[1:]) if p["us"] > 1.08 * q["us"]]
    print("[bench] gemm staircase (M: us): " + ", ".join(f"{p['m']}: {p['us']}" for p in points),
          file=sys.stderr, flush=True)
    print(f"[bench] gemm staircase: time rises by >8% at M = {steps}", file=sys.stderr, flush=True)
    # The pages' offline table from these GEMM times: for each token count,
    # the offset whose two GEMMs cost least relative to one GEMM over all
    # rows, next to the analytic planner's choice.
    t = {p["m"]: p["us"] for p in points}
    table = []
    for T in range(1024, 8193, 128):
        half = T // 2
        cost = {off: (t[half + off] + t[T - half - off]) / t[T] - 1
                for off in (0, 64, 128, 192, 256, 512) if off < half}
        best = min(cost, key=cost.get)
        plan = tw.tw_split_plan(T, **plan_kw)
        table.append({"tokens": T, "gemm_us": t[T], "best_offset": best,
                      "best_penalty": round(cost[best], 4), "planner_reason": plan["reason"],
                      "planner_offset": plan["offset"],
                      "planner_penalty": round(cost[plan["offset"]], 4)
                      if plan["reason"] == 0 else None})
    split = [e for e in table if e["planner_reason"] == 0]
    summary = {"planner_splits": len(split),
               "planner_picks_best": sum(e["planner_offset"] == e["best_offset"] for e in split),
               "planner_penalty_median": round(statistics.median(e["planner_penalty"] for e in split), 4),
               "planner_penalty_max": round(max(e["planner_penalty"] for e in split), 4),
               "best_penalty_median": round(statistics.median(e["best_penalty"] for e in split), 4),
               "best_penalty_max": round(max(e["best_penalty"] for e in split), 4)}
    print(f"[bench] gemm split table vs planner: {summary}", file=sys.stderr, flush=True)
    return {"k": K, "n": h, "points": points, "rises_at": steps, "split_table": table,
            "summary": summary}


def rotation_sets(rows, hidden, num_partials, itemsize) -> int:
    """Buffer sets to rotate so that the inputs, and the outputs on their own,
    of the sets touched between two uses of one set each exceed twice the
    MALL (at most MAX_ROTATE)."""
    in_bytes = (num_partials + 1) * rows * hidden * itemsize
    out_bytes = 2 * rows * hidden * itemsize
    return min(MAX_ROTATE, max(math.ceil(2 * MALL_BYTES / (in_bytes + out_bytes)) + 1,
                               math.ceil(2 * MALL_BYTES / out_bytes) + 1))


def _on(stream, fn, i):
    import torch
    with torch.cuda.stream(stream):
        fn(i)


def run_overlap(tw, torch, wl, plan_kw, token_counts, lean=False) -> dict:
    """For each token count: the unsplit step and every feasible split offset,
    each captured as a HIP graph per rotated buffer set and replayed (no host
    launch cost), plus the eager (Python-launched) times for reference.  Also
    the pages' offline table: per token count, the fastest of unsplit and the
    split offsets, next to what the analytic planner chose."""
    from reduce_rmsnorm_amd.overlap import LayerStep, capture, time_graphs, time_steps
    # Two side streams, default priority (graphs are captured off the null stream).
    stream_a = torch.cuda.Stream()
    stream_b = torch.cuda.Stream()
    rows = []
    for T in token_counts:
        nsets = rotation_sets(T, wl.hidden, wl.num_partials, 2)
        step = LayerStep(T, wl.hidden, OVERLAP_K, wl.num_partials, eps=wl.eps, sets=nsets)
        iters = max(20, int(4e-3 / (T * 4e-9 + 1e-6)))

        def measure(fn):
            # Eager first: it also lets the GEMM library finish its lazy per-shape
            # set-up, which it may not do while a stream is being captured.
            e_us = time_steps(fn, stream_a, stream_b, max(10, iters // 4))
            graphs = [capture(fn, stream_a, stream_b, i) for i in range(nsets)]
            g_us = time_graphs(graphs, stream_a, iters)
            del graphs
            return g_us, e_us

        base, base_e = measure(lambda i: step.run_unsplit(i, stream_a))
        plan = tw.tw_split_plan(T, **plan_kw)
        entry = {"tokens": T, "unsplit_us": round(base, 2), "unsplit_eager_us": round(base_e, 2),
                 "planner": plan, "splits": []}
        half = T // 2
        for off in (0, 64, 128, 192, 256, 512):
            if off >= half:
                continue
            us, us_e = measure(lambda i, p=half + off: step.run_split(i, p, stream_a, stream_b))
            entry["splits"].append({"offset": off, "prefix": half + off, "us": round(us, 2),
                                    "eager_us": round(us_e, 2), "speedup": round(base / us, 4)})
        best = min(entry["splits"], key=lambda e: e["us"])
        entry["best_offset"] = best["offset"]
        entry["best_speedup"] = best["speedup"]
        if lean:
            rows.append(entry)
            print(f"[bench] overlap T={T} (graph replay): unsplit {base:.1f} us; " + ", ".join(
                f"off {e['offset']}: {e['us']:.1f}" for e in entry["splits"]) +
                f"; planner reason {plan['reason']} off {plan['offset']}", file=sys.stderr, flush=True)
            del step
            torch.cuda.empty_cache()
            continue
        # The fused kernel confined to G workgroups during the overlap (the
        # pages run theirs on a few SMs so the GEMM keeps the rest).
        entry["splits_workgroups"] = []
        for G in (64, 128, 256):
            us, _ = measure(lambda i, p=half + best["offset"], G=G:
                            step.run_split(i, p, stream_a, stream_b, workgroups=G))
            entry["splits_workgroups"].append({"workgroups": G, "offset": best["offset"],
                                               "us": round(us, 2)})
        # Components alone (graph replays, one stream).
        comp = {}
        for name, lo, hi, kind in (("gemm_all", 0, T, "g"), ("gemm_half", 0, half, "g"),
                                   ("fused_all", 0, T, "f"), ("fused_half", 0, half, "f")):
            if kind == "g":
                fn = (lambda i, lo=lo, hi=hi: step._gemm(i, lo, hi))
            else:
                fn = (lambda i, lo=lo, hi=hi: step._fused(i, lo, hi, torch.cuda.current_stream(),
                                                          None))
            comp[name], _ = measure(lambda i, fn=fn: _on(stream_a, fn, i))
            comp[name] = round(comp[name], 2)
        entry["components_us"] = comp
        rows.append(entry)
        print(f"[bench] overlap T={T} (graph replay): unsplit {base:.1f} us; " + ", ".join(
            f"off {e['offset']}: {e['us']:.1f}" for e in entry["splits"]) +
            f"; best off {best['offset']} ({best['speedup']:.3f}x); planner reason "
            f"{plan['reason']} off {plan['offset']}; eager unsplit {base_e:.1f} us, eager "
            f"splits " + ", ".join(f"{e['eager_us']:.1f}" for e in entry["splits"]) +
            "; confined fused: " + ", ".join(f"G={e['workgroups']}: {e['us']:.1f}"
                                             for e in entry["splits_workgroups"]) +
            f"; components {entry['components_us']}", file=sys.stderr, flush=True)
        del step
        torch.cuda.empty_cache()
    table = []
    for e in rows:
        choices = {-1: e["unsplit_us"]}
        choices.update({s["offset"]: s["us"] for s in e["splits"]})
        fastest = min(choices, key=choices.get)
        pl = e["planner"]["offset"] if e["planner"]["reason"] == 0 else -1
        table.append({"tokens": e["tokens"], "fastest": fastest, "fastest_us": choices[fastest],
                      "best_split_offset": e["best_offset"],
                      "best_split_us": choices[e["best_offset"]],
                      "planner": pl, "planner_us": choices.get(pl),
                      "planner_over_fastest": round(choices[pl] / choices[fastest] - 1, 4)
                      if pl in choices else None})
    return {"steps": rows, "table": table}


def _probe_lib():
    import ctypes
    from reduce_rmsnorm_amd.build import PROBE_LIB_PATH
    lib = ctypes.CDLL(PROBE_LIB_PATH)
    lib.tw_probe_launch.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_void_p), ctypes.c_int,
                                    ctypes.POINTER(ctypes.c_void_p), ctypes.c_int, ctypes.c_int64,
                                    ctypes.c_int, ctypes.c_void_p]
    lib.tw_probe_launch.restype = ctypes.c_int
    lib.tw_probe_twin_launch.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_void_p),
                                         ctypes.c_int, ctypes.POINTER(ctypes.c_void_p),
                                         ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
    lib.tw_probe_twin_launch.restype = ctypes.c_int
    lib.tw_probe_launch_cost.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                         ctypes.POINTER(ctypes.c_double)]
    lib.tw_probe_launch_cost.restype = ctypes.c_int
    return lib


PLACEMENT_GRID = 4096


def placement(lib, torch, stream, records):
    """Run the placement probe on ``stream``: returns {XCC id: number of
    distinct CUs its workgroups ran on}.  A CU is identified by its XCC id and
    bits [15:8] of HW_ID (CU, shader array and shader engine ids)."""
    import ctypes
    import numpy as np
    records.zero_()
    dst = (ctypes.c_void_p * 1)(records.data_ptr())
    src = (ctypes.c_void_p * 1)()
    torch.cuda.current_stream().synchronize()
    rc = lib.tw_probe_launch(3, src, 0, dst, 1, PLACEMENT_GRID, PLACEMENT_GRID, stream.cuda_stream)
    if rc != 0:
        raise RuntimeError(f"placement probe launch failed: {rc}")
    stream.synchronize()
    r = records.cpu().numpy().view(np.uint32).reshape(PLACEMENT_GRID, 4)
    if not (r[:, 3] == 1).all():
        raise RuntimeError("placement probe left records unwritten")
    cus = {}
    for xcc, loc in set(zip((r[:, 1] & 0xF).tolist(), ((r[:, 0] >> 8) & 0xFF).tolist())):
        cus[xcc] = cus.get(xcc, 0) + 1
    return dict(sorted(cus.items()))


def dealt_share(torch, records) -> float:
    """After ``placement``: the share of workgroups b that ran on XCC b mod 8,
    i.e. how far the dispatcher deals a grid's workgroups over the XCDs in
    turn."""
    import numpy as np
    r = records.cpu().numpy().view(np.uint32).reshape(PLACEMENT_GRID, 4)
    return float(((r[:, 1] & 0xF) == (r[:, 2] % 8)).mean())


def run_cu_mask(tw, torch, wl, sets, R, w, step_bytes) -> dict:
    """CU-masked streams (``hipExtStreamCreateWithCUMask``).

    The runtime accepts a mask only if it leaves at least one CU on each of the
    eight XCDs (a dispatch's workgroups are dealt out over all of them), and
    mask bit b belongs to XCD b mod 8; the placement probe confirms both here by
    counting the CUs each XCD used, and records how often workgroup b ran on XCD
    b mod 8 on the unconfined stream.  Then: (1) fused-kernel GB/s on the first k
    mask bits, which spreads k CUs evenly over the XCDs; (2) a skewed mask, one
    XCD whole and one CU on each other XCD, against a balanced mask of about
    the same size; (3) the split layer step with the fused kernel confined to k
    CUs while the GEMM keeps an unmasked stream.

    Only the fused kernel and the placement probe run on masked streams: their
    workgroups never wait on one another, so confining them cannot stall a
    launch.  The library GEMM's kernels are not known to have that property, so
    they are never confined."""
    from reduce_rmsnorm_amd.overlap import LayerStep, MaskedStream, time_steps
    lib = _probe_lib()
    records = torch.zeros(PLACEMENT_GRID * 4, dtype=torch.int32, device="cuda")
    out = {}

    checks = {"all 256 bits": list(range(256)), "bits 0-7": list(range(8)),
              "bits 0-15": list(range(16)), "bits 0-7 + 8, 16, 24": list(range(8)) + [8, 16, 24]}
    out["placement"] = {}
    for name, bits in checks.items():
        with MaskedStream(bits) as ms:
            per_xcc = placement(lib, torch, ms.stream, records)
        out["placement"][name] = per_xcc
        if name == "all 256 bits":
            out["dealt_b_mod_8"] = dealt_share(torch, records)
            print(f"[bench] cu-mask placement: workgroup b ran on XCC b mod 8 for "
                  f"{100 * out['dealt_b_mod_8']:.2f}% of {PLACEMENT_GRID} workgroups",
                  file=sys.stderr, flush=True)
        print(f"[bench] cu-mask placement {name}: CUs used per XCD {per_xcc}",
              file=sys.stderr, flush=True)

    def time_fused(bits):
        with MaskedStream(bits) as ms:
            per_xcc = placement(lib, torch, ms.stream, records)
            launches = [tw.PreparedFused(parts, res, w, wl.eps, o, ro, ms.stream)
                        for parts, res, o, ro in sets]
            for i in range(3):
                launches[i % R]()
            ms.stream.synchronize()
            est_us = step_bytes / (36e9 * len(bits)) * 1e6
            iters = max(5, min(2000, int(40e3 / est_us)))
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(ms.stream)
            for i in range(iters):
                launches[i % R]()
            e1.record(ms.stream)
            ms.stream.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / iters
        return us, per_xcc

    foot = []
    layouts = [(f"balanced {k}", list(range(k))) for k in (8, 16, 32, 40, 64, 128, 192, 256)]
    layouts.insert(4, ("skewed 39: XCD 0 whole + 1 CU on each other XCD",
                       list(range(0, 256, 8)) + list(range(1, 8))))
    for name, bits in layouts:
        us, per_xcc = time_fused(bits)
        gbs = step_bytes / (us * 1e-6) / 1e9
        foot.append({"layout": name, "cus": len(bits), "cus_per_xcd": list(per_xcc.values()),
                     "us": round(us, 2), "gbs": round(gbs, 1)})
        print(f"[bench] cu-mask footprint {name:50s} {us:9.2f} us {gbs:7.1f} GB/s "
              f"(CUs per XCD {list(per_xcc.values())})", file=sys.stderr, flush=True)
    out["footprint"] = foot

    rows = []
    default_a, default_b = torch.cuda.Stream(), torch.cuda.Stream()
    for T in (4096, 8192):
        step = LayerStep(T, wl.hidden, OVERLAP_K, wl.num_partials, eps=wl.eps,
                         sets=rotation_sets(T, wl.hidden, wl.num_partials, 2))
        P = T // 2
        iters = 40
        base = time_steps(lambda i: step.run_unsplit(i, default_a), default_a, default_b, iters)
        shared = time_steps(lambda i: step.run_split(i, P, default_a, default_b), default_a,
                            default_b, iters)
        entry = {"tokens": T, "prefix": P, "unsplit_us": round(base, 2),
                 "split_shared_us": round(shared, 2), "split_fused_on_k_cus": []}
        for k in (32, 64, 128, 192):
            with MaskedStream(range(k)) as fa:
                us = time_steps(lambda i: step.run_split(i, P, default_a, fa.stream),
                                default_a, fa.stream, iters)
            entry["split_fused_on_k_cus"].append({"cus": k, "us": round(us, 2)})
        rows.append(entry)
        print(f"[bench] cu-mask overlap T={T} (eager): unsplit {base:.1f} us, split on shared "
              f"CUs {shared:.1f} us, split with the fused kernel on k CUs: " +
              ", ".join(f"k={e['cus']}: {e['us']:.1f}" for e in entry["split_fused_on_k_cus"]),
              file=sys.stderr, flush=True)
        del step
        torch.cuda.empty_cache()
    out["overlap"] = rows
    return out


def cpu_baseline(wl, d, budget_s: float) -> dict:
    """Time the float64 oracle as it stands, pinned to one host core, on
    whole rows of the same batch: passes over the batch, 8 rows at a time,
    until the time budget is spent (the last chunk is finished)."""
    import oracle
    parts = list(d["partials"])
    T = wl.num_tokens
    try:
        saved = os.sched_getaffinity(0)
        os.sched_setaffinity(0, {min(saved)})
    except (AttributeError, OSError):
        saved = None
    try:
        rows_done = 0
        t0 = time.perf_counter()
        chunk = 8
        while time.perf_counter() - t0 < budget_s:
            lo = rows_done % T
            rows = range(lo, min(T, lo + chunk))
            oracle.fused_reduce_rmsnorm(parts, d["residual"], d["weight"], d["eps"], wl.dtype,
                                        rows=rows)
            rows_done += len(rows)
        elapsed = time.perf_counter() - t0
    finally:
        if saved is not None:
            os.sched_setaffinity(0, saved)
    gbs = wl.algorithmic_bytes(rows_done) / elapsed / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{rows_done} rows ({rows_done / T:.1f} passes over the {T}-row "
                      f"{wl.name} batch), float64 NumPy oracle, {elapsed:.1f} s on 1 pinned "
                      f"core of {len(saved) if saved else os.cpu_count()}",
            "tokens_per_s": round(rows_done / elapsed, 1)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import reduce_rmsnorm_amd as tw
    from synthetic import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    tw.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = WORKLOADS[args.workload]
    overridden = args.tokens is not None or args.partials is not None or args.hidden is not None
    if overridden:
        import dataclasses
        wl = dataclasses.replace(wl, num_tokens=args.tokens or wl.num_tokens,
                                 num_partials=args.partials or wl.num_partials,
                                 hidden=args.hidden or wl.hidden)
    T, h, N = wl.num_tokens, wl.hidden, wl.num_partials
    tdt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32

    d = make_inputs(wl)

    def up(a):
        if wl.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    if args.mode == "shard":
        lo, hi = (0 * T) // N, (1 * T) // N
    else:
        lo, hi = 0, T
    rows = hi - lo
    step_bytes = wl.algorithmic_bytes(rows)
    # Rotate whole buffer sets (inputs and outputs) so that neither the inputs
    # nor the outputs of the sets fit in the memory-side cache: output buffers
    # that stay resident there would absorb their writes, which on the
    # 1024-row headline shape makes a launch look about 1.6% faster.
    R = args.rotate or rotation_sets(rows, h, N, 2 if wl.dtype == "bf16" else 4)

    base_parts, base_res, w = up(d["partials"]), up(d["residual"]), up(d["weight"])
    sets = []
    for r in range(R):
        parts = base_parts if r == 0 else base_parts.clone()
        res = base_res if r == 0 else base_res.clone()
        sets.append((parts, res, torch.empty_like(res), torch.empty_like(res)))
    stream = torch.cuda.current_stream(dev)

    plan_kw = dict(tokens_per_cta=GEMM_TILE, ctas_per_token_tile=max(1, h // GEMM_TILE),
                   num_cus=256, ctas_per_cu=1,
                   min_split_tokens=4096 if wl.name == "mixtral" else 1024)

    # Each step: the split plan for the batch (a table lookup after the first
    # step, as the pages keep one split per shape) and the fused launch(es),
    # prepared once per rotated buffer set so the host costs one C call each.
    planner = tw.SplitPlanCache(**plan_kw)
    plan0 = planner(T)
    if not args.split and plan0["suffix_tokens"] > 0:
        plan0 = dict(plan0, prefix_tokens=T, suffix_tokens=0, offset=-1, reason=-1)
    def prepare(st):
        per_set = []
        for parts, res, out, rout in sets:
            if args.mode == "shard":
                per_set.append([tw.PreparedFused(parts, res, w, wl.eps, out, rout, st,
                                                 mode="shard", shard_index=0)])
            elif plan0["suffix_tokens"] > 0:
                P = plan0["prefix_tokens"]
                per_set.append([
                    tw.PreparedFused([p[lo:hi] for p in parts], res[lo:hi], w, wl.eps,
                                     out[lo:hi], rout[lo:hi], st) for lo, hi in ((0, P), (P, T))])
            else:
                per_set.append([tw.PreparedFused(parts, res, w, wl.eps, out, rout, st)])
        return per_set

    launches_per_set = prepare(stream)

    def step(i):
        plan = planner(T) if args.mode == "full" and args.split else None
        assert plan is None or plan["prefix_tokens"] == plan0["prefix_tokens"]
        for launch in launches_per_set[i % R]:
            launch()
        return len(launches_per_set[i % R])

    graphs = None
    if args.graph:
        # The same launches recorded into HIP graphs: one graph holds a whole
        # rotation cycle (R steps), a second one the steps % R left over, so
        # the replays run exactly the requested number of steps.  The split
        # plan is the one fixed per shape above.  Recorded before the warm-up:
        # capture idles the GPU (torch collects garbage first), and the timed
        # replays must start from a GPU that has settled under load.
        cap = torch.cuda.Stream(dev)
        cap_sets = prepare(cap)

        def record(count):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                for i in range(count):
                    for launch in cap_sets[i % R]:
                        launch()
            return g

        full = record(R)
        rest = record(args.steps % R) if args.steps % R else None
        graphs = [full] * (args.steps // R) + ([rest] if rest is not None else [])
        with torch.cuda.stream(stream):
            full.replay()
        torch.cuda.synchronize()

    ramp = None
    if args.ramp:
        ramp = run_ramp(torch, step, stream)
    # The settle: steps enough for about SETTLE_SECONDS of GPU work (estimated
    # at the bytes at 6 TB/s plus 3 us per launch), then the requested warm-up.
    est = step_bytes / 6.0e12 + 3e-6 * len(launches_per_set[0])
    settle_steps = max(50, math.ceil(args.settle_ms * 1e-3 / est)) if args.settle_ms > 0 else 0
    print(f"[bench] workload={wl.name} mode={args.mode} rows={rows} h={h} N={N} {wl.dtype} "
          f"rotate={R} settle={settle_steps} warmup={args.warmup} steps={args.steps} "
          f"{'graph' if args.graph else 'eager'}", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t_settle = time.perf_counter()
    for i in range(settle_steps):
        step(i)
    torch.cuda.synchronize()
    settle = {"steps": settle_steps, "seconds": round(time.perf_counter() - t_settle, 4),
              "target_ms": args.settle_ms}
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    launches = 0
    start.record(stream)
    if graphs is None:
        for i in range(args.steps):
            launches += step(i)
    else:
        with torch.cuda.stream(stream):
            for g in graphs:
                g.replay()
        launches = args.steps * len(launches_per_set[0])
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end)
    ms_per_step = ms / args.steps
    gbs = step_bytes / (ms_per_step * 1e-3) / 1e9
    print(f"[bench] timed {args.steps} steps: {ms:.3f} ms, {ms_per_step * 1e3:.2f} us/step, "
          f"{gbs:.1f} GB/s", file=sys.stderr, flush=True)

    unfused = None
    if args.mode == "full" and args.unfused:
        # The reduce-then-normalize sequence the fused kernel replaces, on the
        # same rotated buffers (plus one intermediate tensor per set).
        reds = [torch.empty_like(st[1]) for st in sets]

        def ustep(i):
            parts, res, out, rout = sets[i % R]
            tw.tw_unfused_reduce_rmsnorm(parts, res, w, wl.eps, out=out, residual_out=rout,
                                         reduced=reds[i % R], stream=stream)

        for i in range(args.warmup):
            ustep(i)
        torch.cuda.synchronize()
        u0 = torch.cuda.Event(enable_timing=True)
        u1 = torch.cuda.Event(enable_timing=True)
        u0.record(stream)
        for i in range(args.steps):
            ustep(i)
        u1.record(stream)
        torch.cuda.synchronize()
        u_us = u0.elapsed_time(u1) * 1e3 / args.steps
        u_bytes = (N + 6) * rows * h * wl.itemsize
        unfused = {"us_per_step": round(u_us, 3), "launches_per_step": 2,
                   "traffic_bytes_algorithmic": u_bytes,
                   "gbs_of_own_traffic": round(u_bytes / (u_us * 1e-6) / 1e9, 1),
                   "fused_speedup": round(u_us / (ms_per_step * 1e3), 4)}
        print(f"[bench] unfused comparator: {u_us:.2f} us/step, fused speedup "
              f"{unfused['fused_speedup']:.3f}x", file=sys.stderr, flush=True)
        del reds

    footprint = None
    if args.footprint and args.mode == "full":
        footprint = []
        for G in (2, 4, 8, 16, 32, 64, 128, 256, 512, 768, T):
            if G > T:
                continue

            def gstep(i, G=G):
                parts, res, out, rout = sets[i % R]
                tw.tw_fused_reduce_rmsnorm_grid(parts, res, w, wl.eps, G, out=out,
                                                residual_out=rout, stream=stream)

            k = max(5, min(args.steps, int(0.05 / max(1e-6, step_bytes / 5e12 * 256 / G))))
            for i in range(3):
                gstep(i)
            torch.cuda.synchronize()
            g0 = torch.cuda.Event(enable_timing=True)
            g1 = torch.cuda.Event(enable_timing=True)
            g0.record(stream)
            for i in range(k):
                gstep(i)
            g1.record(stream)
            torch.cuda.synchronize()
            g_us = g0.elapsed_time(g1) * 1e3 / k
            gbs_g = step_bytes / (g_us * 1e-6) / 1e9
            footprint.append({"workgroups": G, "us": round(g_us, 2), "gbs": round(gbs_g, 1)})
            print(f"[bench] footprint {G:5d} workgroups: {g_us:9.2f} us  {gbs_g:7.1f} GB/s",
                  file=sys.stderr, flush=True)

    staircase = None
    if args.gemm_staircase:
        staircase = run_gemm_staircase(tw, torch, wl, plan_kw)

    cu_mask = None
    if args.cu_mask and args.mode == "full":
        cu_mask = run_cu_mask(tw, torch, wl, sets, R, w, step_bytes)

    split_table = None
    if args.split_table and args.mode == "full":
        split_table = []
        half = T // 2
        for off in (None, 0, 64, 128, 192, 256, 512):
            if off is not None and off >= half:
                continue
            P = T if off is None else half + off
            piece_sets = []
            for parts, res, out, rout in sets:
                pieces = [(0, T)] if off is None else [(0, P), (P, T)]
                piece_sets.append([tw.PreparedFused([p[lo:hi] for p in parts], res[lo:hi], w,
                                                    wl.eps, out[lo:hi], rout[lo:hi], stream)
                                   for lo, hi in pieces])
            # Each offset is warmed for about 50 ms of work: its prepared
            # launches are built on the host first, and a GPU that has just
            # waited needs tens of milliseconds of load to return to its
            # steady clocks.
            est = step_bytes / 6.0e12 + 3e-6 * len(piece_sets[0])
            for i in range(max(20, math.ceil(0.05 / est))):
                for launch in piece_sets[i % R]:
                    launch()
            torch.cuda.synchronize()
            s0 = torch.cuda.Event(enable_timing=True)
            s1 = torch.cuda.Event(enable_timing=True)
            s0.record(stream)
            for i in range(args.steps):
                for launch in piece_sets[i % R]:
                    launch()
            s1.record(stream)
            torch.cuda.synchronize()
            us = s0.elapsed_time(s1) * 1e3 / args.steps
            split_table.append({"offset": off, "prefix": P, "suffix": T - P, "us": round(us, 2),
                                "gbs": round(step_bytes / (us * 1e-6) / 1e9, 1)})
            print(f"[bench] split table offset {off}: prefix {P} suffix {T - P}: {us:.2f} us "
                  f"({split_table[-1]['gbs']} GB/s)", file=sys.stderr, flush=True)

    overlap = None
    if args.overlap:
        overlap = run_overlap(tw, torch, wl, plan_kw,
                              [int(t) for t in args.overlap_tokens.split(",")], args.overlap_lean)

    def timer(go, k):
        for i in range(min(20, k)):
            go(i)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(k):
            go(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / k

    ceiling = None
    if args.ceiling:
        ceiling = run_ceiling(tw, sets, R, rows, h, wl.itemsize, stream, min(args.steps, 500),
                              timer)
    host_cost = None
    if args.host_cost:
        host_cost = run_host_cost(tw, torch, wl, sets, w, stream, plan_kw)
    launch_floor = None
    if args.launch_floor:
        launch_floor = run_launch_floor(torch, timer)

    traffic = None
    if os.path.exists(TRAFFIC_FILE) and args.mode == "full" and wl.name == "llama70b" \
            and not overridden:
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_code_sha256") == kernel_source_hash():
            traffic = tr.get("bytes_per_launch")

    result = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle": settle,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{wl.name}: T={T} h={h} N={N} {wl.dtype} storage, "
                               f"{args.mode} mode ({rows} rows), eps={wl.eps}",
                   "num_tokens": T, "hidden": h, "num_partials": N, "storage_dtype": wl.dtype,
                   "mode": args.mode, "rows": rows, "rotated_input_sets": R,
                   "launches_per_step": launches / args.steps,
                   "launch": ("hip graph replays, one graph per %d-step rotation cycle" % R
                              if args.graph else "eager stream launches")},
        "pct_of_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(rows / (ms_per_step * 1e-3), 1),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": step_bytes * args.steps // max(1, launches),
                     "avg_launch_us": round(ms * 1e3 / max(1, launches), 3)},
        "cpu_baseline": None,
    }
    if unfused is not None:
        result["unfused_comparator"] = unfused
    if footprint is not None:
        result["footprint"] = footprint
    if overlap is not None:
        result["overlap"] = overlap
    if split_table is not None:
        result["split_table"] = split_table
    if cu_mask is not None:
        result["cu_mask"] = cu_mask
    if ramp is not None:
        result["ramp"] = ramp
    if launch_floor is not None:
        result["empty_launch_us"] = launch_floor
    if host_cost is not None:
        result["host_cost"] = host_cost
    if staircase is not None:
        result["gemm_staircase"] = staircase
    if ceiling is not None:
        # Secondary context: the fused step against a plain stream that moves
        # exactly its bytes on the same buffers in the same run.
        ceiling["fused_over_read_write_probe"] = round(result["value"] / ceiling["read_write_gbs"], 4)
        if "twin_read_write_gbs" in ceiling:
            ceiling["fused_over_twin"] = round(result["value"] / ceiling["twin_read_write_gbs"], 4)
        result["ceiling"] = ceiling
    if args.cpu_seconds > 0:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(wl, d, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
