#!/usr/bin/env python3
"""Benchmark: ring AllReduce of 8 virtual ranks x 2^26 float32 (sum) on one MI355X.

One step is one AllReduce through the library's default algorithm, which
for this shape is the staged form (per segment, a reducing launch into rank
0, then a broadcasting launch), on synthetic N(0,1) inputs already resident
in HBM.  Prints one JSON line with algbw (S/t, the value), busbw
(algbw * 2(N-1)/N), the HBM roofline of the call's kernels, the fused
one-pass kernel's time beside it, and the CPU oracle timed on this host.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Only one GPU is used: the N ranks are buffers in that GPU's memory.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "AllReduce algbw/busbw GB/s + % HBM peak, N=8 ranks x 64M fp32, 1 MI355X"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, 8 TB/s
# rocprofv3 counter summaries of the headline call, by the form it runs
COUNTERS_FILES = {"staged": os.path.join(ROOT, "profiles", "staged_allreduce_headline_counters.md"),
                  "fused": os.path.join(ROOT, "profiles", "fused_allreduce_headline_counters.md"),
                  "phases": os.path.join(ROOT, "profiles", "phases_allreduce_headline_counters.md"),
                  "double_binary_tree": os.path.join(ROOT, "profiles", "dbt_allreduce_headline_counters.md"),
                  "double_binary_tree_steps": os.path.join(ROOT, "profiles",
                                                           "dbt_steps_allreduce_headline_counters.md")}
# the sources the AllReduce kernels are built from (their counters are only
# used while these are unchanged)
KERNEL_SOURCES = [os.path.join(ROOT, "ring_allreduce_reduction_virtual_amd", "csrc", f)
                  for f in ("ar_kernels.hip", "ar_device.h", "ar_internal.h")]


# the AllReduce algorithms bench.py can time as its step, and the kernels each
# one launches (float32, sum, 16-byte vectors at the headline shape)
STEP_ALGOS = ("auto", "fused", "phases", "staged", "ring", "ring_pipelined", "ring_persistent", "tree",
              "tree_steps", "recursive_doubling", "halving_doubling", "halving_doubling_steps", "double_binary_tree",
              "double_binary_tree_steps")
STEP_KERNELS = {
    "fused": "k_fused_allreduce<f32,sum,vec16>",
    "phases": "k_fused_reduce_scatter<f32,sum,vec16> + k_gather_shards_xcd<f32,vec16> (in place)",
    "ring": "k_ring_reduce_step<f32,sum,vec16> + k_ring_copy_step<f32,vec16>, {launches} launches",
    "ring_pipelined": "k_ring_pipelined<f32,sum,vec16>",
    "ring_persistent": "k_ring_persistent<f32,sum,vec16>",
    "tree": "k_fused_tree<f32,sum,vec16>",
    "halving_doubling": "k_fused_tree<f32,sum,vec16> (bit-reversed ranks)",
    "tree_steps": "k_tree_reduce_step<f32,sum,vec16> + k_tree_copy_step<f32,vec16>, {launches} launches",
    "halving_doubling_steps": "k_tree_reduce_step<f32,sum,vec16> + k_tree_copy_step<f32,vec16>, {launches} launches",
    "recursive_doubling": "k_tree_reduce_step<f32,sum,vec16>, {launches} launches",
    "double_binary_tree": "k_fused_dbt<f32,sum,vec16>",
    "double_binary_tree_steps": "k_dbt_reduce_step<f32,sum,vec16> + k_dbt_copy_step<f32,vec16>, {launches} launches",
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def busbw_factor(coll: str, n: int) -> float:
    """Bus bandwidth factor: 2(N-1)/N for AllReduce, (N-1)/N for one phase alone."""
    return (2.0 if coll == "allreduce" else 1.0) * (n - 1) / n


def algorithmic_bytes(coll: str, n: int, s_bytes: int) -> int:
    """Minimum HBM traffic of one call: AllReduce reads N*S and writes N*S;
    reduce-scatter reads N*S and writes S; all-gather reads S and writes N*S."""
    return 2 * n * s_bytes if coll == "allreduce" else (n + 1) * s_bytes


# kernels of other forms live in files of their own, hashed with the shared ones
FORM_SOURCES = {form: [os.path.join(ROOT, "ring_allreduce_reduction_virtual_amd", "csrc", "ar_dbt_kernels.hip")]
                for form in ("double_binary_tree", "double_binary_tree_steps")}


def kernel_source_hash(form: str = None) -> str:
    h = hashlib.sha256()
    for path in KERNEL_SOURCES + FORM_SOURCES.get(form, []):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(form: str):
    """HBM bytes per call (all the call's launches) of the given form from the
    committed rocprofv3 counter summary, if it was taken on the current kernel
    source; else None."""
    path = COUNTERS_FILES.get(form)
    if path is None or not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"^traffic_json: (\{.*\})\s*$", text, flags=re.M)
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("kernel_source_sha256_16") != kernel_source_hash(form):
        return None
    return d.get("bytes_per_call")


def ensure_library():
    from ring_allreduce_reduction_virtual_amd import _lib

    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__

        __graft_entry__.build()


def time_calls(fn, steps: int, warmup: int, stream):
    """Average milliseconds per call over `steps` calls, timed with HIP events on `stream`."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(steps):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / steps


def median_call_ms(fn, steps: int, warmup: int, stream):
    """Median and minimum milliseconds of single calls, each bracketed by HIP events."""
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    times = sorted(a.elapsed_time(b) for a, b in evs)
    return times[len(times) // 2], times[0]


def flushed_median_ms(fn, steps: int, stream, flush, mode: str = "write"):
    """Median and minimum milliseconds of single calls, each preceded (outside its
    events) by a pass over the whole `flush` tensor, 1 GiB against the 256 MB
    last-level cache, so that every call finds its inputs in HBM.  "write"
    fills it (the cache is then full of dirty lines, which the call's own
    traffic pushes out to HBM, as after a kernel that wrote a lot); "read"
    reduces over it (the cache is left holding clean lines)."""
    import torch

    fn()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (a, b) in enumerate(evs):
        if mode == "write":
            flush.fill_(i & 0xFF)
        else:
            flush.view(torch.int32).max()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    times = sorted(a.elapsed_time(b) for a, b in evs)
    return times[len(times) // 2], times[0]


def graph_ms_per_call(fn, calls: int, stream, replays: int = 5):
    """Milliseconds per call when `calls` calls are captured in one HIP graph and replayed."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        fn()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(calls):
            fn()
    g.replay()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(replays):
        g.replay()
    b.record(stream)
    b.synchronize()
    return a.elapsed_time(b) / (replays * calls)


def _to_device(x, dtype, dev):
    import numpy as np
    import torch

    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(x).to(dev)


def cpu_baseline_headline(xs, s_bytes):
    """The headline line's cpu_baseline: the oracle's executed ring schedule on the
    whole workload, single-threaded, repeated until about 10 s of CPU work
    (at least one run, at most 40), and beside it the oracle's one-thread-per-
    rank ring when the host has a core per rank."""
    import oracle
    from oracle.threaded import ring_allreduce_threaded

    n = len(xs)
    reps, spent = 0, 0.0
    while reps < 40 and spent < 10.0:
        t = time.perf_counter()
        oracle.ring_allreduce(xs, check=False)
        spent += time.perf_counter() - t
        reps += 1
    per = spent / reps
    cpu = {"value": round(s_bytes / per / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
           "sample": f"the whole workload ({n} ranks x {len(xs[0])} f32) through the oracle's executed ring schedule, "
                     f"{reps} run(s), {per:.2f} s each, single-threaded numpy; host {cpu_model()}, "
                     f"{len(os.sched_getaffinity(0))} cores available"}
    log(f"[bench] CPU oracle: {per:.2f} s per AllReduce -> algbw {cpu['value']} GB/s (1 core)")
    # numpy releases the GIL in its array work, so the threads overlap
    if min(n, len(os.sched_getaffinity(0))) == n:
        t = time.perf_counter()
        ring_allreduce_threaded(xs, timeout=600.0)
        tt = time.perf_counter() - t
        cpu["threaded"] = {"value": round(s_bytes / tt / 1e9, 4), "unit": "GB/s", "threads": n,
                           "sample": f"the same workload, one thread per rank, 1 run of {tt:.2f} s"}
        log(f"[bench] CPU oracle, one thread per rank: {tt:.2f} s -> algbw {cpu['threaded']['value']} GB/s")
    return cpu


def cpu_baseline_on_prefix(xs, op, dtype, sample):
    """Seconds the oracle's executed ring schedule takes on the first `sample`
    elements of every rank, single-threaded: the CPU baseline beside each
    workload.  With cpu_baseline_headline, the only use bench.py makes of the
    oracle: parity is the GPU tests' job."""
    import oracle

    t0 = time.perf_counter()
    oracle.ring_allreduce([x[:sample] for x in xs], op=op, dtype=dtype, check=False)
    return time.perf_counter() - t0


def run_configs(args):
    """Every workload with every ring-order algorithm, timed per call (median of K), with
    the CPU oracle timed on a bounded prefix beside it.  Parity at these sizes is
    checked by the GPU tests (tests/test_gpu_parity.py), not here."""
    import torch

    import ring_allreduce_reduction_virtual_amd as ar
    from inputs import WORKLOADS, make_inputs

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "i32": torch.int32}
    esz = {"f32": 4, "bf16": 2, "i32": 4}
    # the headline first, in the state the default line measures it in, and again after the
    # heaviest workload (c5 moves 32 GiB per call) to show what that leaves behind
    names = ("headline", "c1", "c2", "c3", "c4", "c5", "headline")
    if args.workloads:
        names = tuple(args.workloads.split(","))
    flush = None
    for name in names:
        w = WORKLOADS[name]
        n, count, dt = w.nranks, w.count, w.dtype
        s_bytes = count * esz[dt]
        xs = make_inputs(w)
        sends = [_to_device(x, dt, dev) for x in xs]
        recvs = [torch.empty(count, dtype=tdt[dt], device=dev) for _ in range(n)]
        sample = min(count, 1 << 20)
        oracle_s = cpu_baseline_on_prefix(xs, w.ops[0], dt, sample)
        steps = 200 if s_bytes < (1 << 24) else 20
        for op in w.ops:
            for algo in ("fused", "staged", "phases", "auto", "ring", "ring_pipelined"):
                fn = (lambda: ar.ar_allreduce_ex(sends, recvs, op=op, algo=algo))
                med, mn = median_call_ms(fn, steps, 3, stream)
                algo_bytes = algorithmic_bytes("allreduce", n, s_bytes)
                latency = {}
                if s_bytes * n <= (64 << 20):
                    # buffers that fit in the last-level cache: also timed with it flushed before each call
                    if flush is None:
                        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
                    for mode, key in (("write", "flushed"), ("read", "evicted")):
                        fmed, fmn = flushed_median_ms(fn, steps, stream, flush, mode)
                        latency[f"{key}_median_us"] = round(fmed * 1e3, 2)
                        latency[f"{key}_min_us"] = round(fmn * 1e3, 2)
                        latency[f"{key}_hbm_frac"] = round(algorithmic_bytes("allreduce", n, s_bytes) / (fmed / 1e3)
                                                           / 1e9 / HBM_PEAK_GBPS, 4)
                    # small messages: the same call as a persistent plan, and replayed from a HIP graph
                    plan = ar.ar_allreduce_init(sends, recvs, op=op, algo=algo)
                    pmed, _ = median_call_ms(plan.start, steps, 3, stream)
                    latency["plan_median_us"] = round(pmed * 1e3, 2)
                    latency["graph_us_per_call"] = round(graph_ms_per_call(plan.start, 50, stream) * 1e3, 2)
                    plan.close()
                print(json.dumps({**latency, 
                    "config": name, "collective": "allreduce", "algo": algo, "op": op, "dtype": dt, "nranks": n,
                    "count": count, "median_us": round(med * 1e3, 2), "min_us": round(mn * 1e3, 2),
                    "algbw_gbps": round(s_bytes / (med / 1e3) / 1e9, 2),
                    "busbw_gbps": round(s_bytes / (med / 1e3) / 1e9 * busbw_factor("allreduce", n), 2),
                    "hbm_gbps_of_minimum": round(algo_bytes / (med / 1e3) / 1e9, 1),
                    "hbm_frac": round(algo_bytes / (med / 1e3) / 1e9 / HBM_PEAK_GBPS, 4),
                    "oracle_s_on_prefix": round(oracle_s, 3), "oracle_prefix_elems": sample, "oracle_cores": 1,
                }), flush=True)
        if "reduce_scatter" in w.phases:
            shards = [torch.empty(ar.ar_chunk_range(r, count, n)[1] - ar.ar_chunk_range(r, count, n)[0],
                                  dtype=tdt[dt], device=dev) for r in range(n)]
            rs_bytes = algorithmic_bytes("reduce_scatter", n, s_bytes)
            for algo in ("fused", "ring", "ring_pipelined"):
                med, mn = median_call_ms(lambda: ar.ar_reduce_scatter_ex(sends, shards, algo=algo), steps, 3, stream)
                print(json.dumps({"config": name, "collective": "reduce_scatter", "algo": algo, "op": "sum",
                                  "dtype": dt, "nranks": n, "count": count, "median_us": round(med * 1e3, 2),
                                  "min_us": round(mn * 1e3, 2),
                                  "algbw_gbps": round(s_bytes / (med / 1e3) / 1e9, 2),
                                  "busbw_gbps": round(s_bytes / (med / 1e3) / 1e9 * busbw_factor("reduce_scatter", n), 2),
                                  "hbm_gbps_of_minimum": round(rs_bytes / (med / 1e3) / 1e9, 1),
                                  "hbm_frac": round(rs_bytes / (med / 1e3) / 1e9 / HBM_PEAK_GBPS, 4)}), flush=True)
            for algo in ("fused", "ring", "ring_pipelined"):
                med, mn = median_call_ms(lambda: ar.ar_all_gather_ex(shards, recvs, algo=algo), steps, 3, stream)
                print(json.dumps({"config": name, "collective": "all_gather", "algo": algo, "dtype": dt,
                                  "nranks": n, "count": count, "median_us": round(med * 1e3, 2),
                                  "min_us": round(mn * 1e3, 2),
                                  "algbw_gbps": round(s_bytes / (med / 1e3) / 1e9, 2),
                                  "busbw_gbps": round(s_bytes / (med / 1e3) / 1e9 * busbw_factor("all_gather", n), 2),
                                  "hbm_gbps_of_minimum": round(rs_bytes / (med / 1e3) / 1e9, 1),
                                  "hbm_frac": round(rs_bytes / (med / 1e3) / 1e9 / HBM_PEAK_GBPS, 4)}), flush=True)
            del shards
        del sends, recvs, xs
        torch.cuda.empty_cache()


def run_variants(args):
    """The precision and operator variants at full size: the bf16 workload (8 x 2^26)
    with float32 partials and with avg, the headline workload with avg, and
    an 8 x 2^26 binary16 AllReduce of N(0,1) values.  Parity at these sizes is
    checked by the GPU tests (tests/test_gpu_variants.py), not here."""
    import numpy as np
    import torch

    import ring_allreduce_reduction_virtual_amd as ar
    from inputs import WORKLOADS, make_inputs

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    c3 = make_inputs(WORKLOADS["c3"])
    head = make_inputs(WORKLOADS["headline"])
    f16 = [x.astype(np.float16).view(np.uint16) for x in head]   # the headline draws, rounded to binary16
    cases = [("c3 8 x 2^26 bf16", c3, "bf16acc32", "sum", torch.bfloat16),
             ("c3 8 x 2^26 bf16", c3, "bf16acc32", "avg", torch.bfloat16),
             ("c3 8 x 2^26 bf16", c3, "bf16", "avg", torch.bfloat16),
             ("headline 8 x 2^26 f32", head, "f32", "avg", torch.float32),
             ("8 x 2^26 f16, N(0,1)", f16, "f16", "sum", torch.float16)]
    for label, xs, dt, op, tdt in cases:
        n, count = len(xs), len(xs[0])
        if tdt == torch.float32:
            sends = [torch.from_numpy(x).to(dev) for x in xs]
        else:
            sends = [torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(dev).view(tdt) for x in xs]
        recvs = [torch.empty(count, dtype=tdt, device=dev) for _ in range(n)]
        s_bytes = count * sends[0].element_size()
        for algo in ("fused", "staged", "phases", "ring", "ring_pipelined"):
            med, mn = median_call_ms(lambda: ar.ar_allreduce_ex(sends, recvs, op=op, algo=algo, dtype=dt), 20, 3, stream)
            algo_bytes = algorithmic_bytes("allreduce", n, s_bytes)
            print(json.dumps({"workload": label, "dtype": dt, "op": op, "algo": algo, "nranks": n, "count": count,
                              "median_us": round(med * 1e3, 2), "min_us": round(mn * 1e3, 2),
                              "algbw_gbps": round(s_bytes / (med / 1e3) / 1e9, 2),
                              "busbw_gbps": round(s_bytes / (med / 1e3) / 1e9 * busbw_factor("allreduce", n), 2),
                              "hbm_gbps_of_minimum": round(algo_bytes / (med / 1e3) / 1e9, 1),
                              "hbm_frac": round(algo_bytes / (med / 1e3) / 1e9 / HBM_PEAK_GBPS, 4)}), flush=True)
        del sends, recvs
        torch.cuda.empty_cache()


def run_orders(args):
    """The tree-shaped orders beside the ring: full workloads timed, and small
    messages timed as one-shot calls, persistent plans and HIP graph replays
    (the latency regime, where the pages expect 2 log2 N stages to beat the
    ring's 2(N-1)).  Parity of every order at these sizes is checked by the
    GPU tests (tests/test_gpu_orders.py, tests/test_gpu_persistent.py)."""
    import torch

    import ring_allreduce_reduction_virtual_amd as ar
    from inputs import WORKLOADS, make_inputs

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "i32": torch.int32}
    for name in ("headline", "c3", "c4", "c5"):
        w = WORKLOADS[name]
        n, count, dt = w.nranks, w.count, w.dtype
        xs = make_inputs(w)
        sends = [_to_device(x, dt, dev) for x in xs]
        recvs = [torch.empty(count, dtype=tdt[dt], device=dev) for _ in range(n)]
        s_bytes = count * sends[0].element_size()
        for algo in ("fused", "ring", "ring_persistent", "ring_pipelined", "tree", "halving_doubling", "tree_steps",
                     "recursive_doubling", "halving_doubling_steps", "double_binary_tree", "double_binary_tree_steps"):
            if algo in ("recursive_doubling", "halving_doubling", "halving_doubling_steps") and n & (n - 1):
                continue
            med, mn = median_call_ms(lambda: ar.ar_allreduce_ex(sends, recvs, algo=algo), 10, 2, stream)
            algo_bytes = algorithmic_bytes("allreduce", n, s_bytes)
            print(json.dumps({"orders": name, "algo": algo, "dtype": dt, "nranks": n, "count": count,
                              "median_us": round(med * 1e3, 2), "min_us": round(mn * 1e3, 2),
                              "algbw_gbps": round(s_bytes / (med / 1e3) / 1e9, 2),
                              "hbm_gbps_of_minimum": round(algo_bytes / (med / 1e3) / 1e9, 1),
                              "hbm_frac": round(algo_bytes / (med / 1e3) / 1e9 / HBM_PEAK_GBPS, 4)}), flush=True)
        del sends, recvs, xs
        torch.cuda.empty_cache()

    # latency regime: 4 KiB per rank at 4, 8, 64 and 128 ranks
    for n in (4, 8, 64, 128):
        count = 1024
        sends = [torch.randn(count, device=dev) for _ in range(n)]
        recvs = [torch.empty(count, device=dev) for _ in range(n)]
        for algo in ("fused", "ring", "ring_persistent", "ring_pipelined", "tree", "tree_steps", "recursive_doubling",
                     "halving_doubling_steps", "double_binary_tree", "double_binary_tree_steps"):
            med, _ = median_call_ms(lambda: ar.ar_allreduce_ex(sends, recvs, algo=algo), 200, 5, stream)
            plan = ar.ar_allreduce_init(sends, recvs, algo=algo)
            pmed, _ = median_call_ms(plan.start, 200, 5, stream)
            # the persistent ring refuses graph capture (its barrier needs a cooperative launch)
            gus = None if algo == "ring_persistent" else round(graph_ms_per_call(plan.start, 50, stream) * 1e3, 2)
            print(json.dumps({"latency": f"{n} x 1024 f32", "algo": algo, "launches": plan.num_launches,
                              "one_shot_median_us": round(med * 1e3, 2), "plan_median_us": round(pmed * 1e3, 2),
                              "graph_us_per_call": gus}), flush=True)
            plan.close()
        del sends, recvs


def run_interference(args):
    """The fused AllReduce overlapping a bf16 GEMM on another stream.

    arjunsriva.com "AllReduce, All the Way Down" (section on communication
    sharing the machine with the model): an overlapped collective still takes
    compute units and HBM bandwidth from the computation beside it, so the
    fastest collective alone is not necessarily the fastest step.  Here the
    AllReduce's footprint is bounded by capping its workgroups
    (ar_plan_limit_blocks); for each cap: the AllReduce alone, the GEMM alone,
    both launched together (each one's own duration and the makespan), against
    running them one after the other.
    """
    import numpy as np
    import torch

    import ring_allreduce_reduction_virtual_amd as ar
    from inputs import WORKLOADS, make_inputs

    dev = torch.device("cuda:0")
    w = WORKLOADS["headline"]
    n, count = w.nranks, w.count
    s_bytes = count * 4
    xs = make_inputs(w)
    sends = [torch.from_numpy(x).to(dev) for x in xs]
    recvs = [torch.empty(count, device=dev) for _ in range(n)]
    plan = ar.ar_allreduce_init(sends, recvs, algo="fused")
    dim = 8192
    g = torch.Generator(device=dev).manual_seed(5)
    a = torch.randn(dim, dim, device=dev, dtype=torch.bfloat16, generator=g)
    b = torch.randn(dim, dim, device=dev, dtype=torch.bfloat16, generator=g)
    c = torch.empty(dim, dim, device=dev, dtype=torch.bfloat16)
    flops = 2.0 * dim ** 3
    s_ar, s_mm = torch.cuda.Stream(), torch.cuda.Stream()
    gemm_calls = 1

    def gemm():
        for _ in range(gemm_calls):
            torch.matmul(a, b, out=c)

    def alone(fn, stream, reps=15):
        ts = []
        with torch.cuda.stream(stream):
            for i in range(reps + 3):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                e1.synchronize()
                if i >= 3:
                    ts.append(e0.elapsed_time(e1) * 1e3)
        return float(np.median(ts))

    def together(ar_first, reps=15):
        rows = []
        for i in range(reps + 3):
            go = torch.cuda.Event()
            go.record(torch.cuda.current_stream())
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
            s_ar.wait_event(go)
            s_mm.wait_event(go)

            def launch_gemm():
                ev[0].record(s_mm)
                with torch.cuda.stream(s_mm):
                    gemm()
                ev[1].record(s_mm)

            def launch_ar():
                ev[2].record(s_ar)
                plan.start(s_ar)
                ev[3].record(s_ar)

            if ar_first:
                launch_ar()
                launch_gemm()
            else:
                launch_gemm()
                launch_ar()
            torch.cuda.synchronize()
            if i >= 3:
                t_mm = ev[0].elapsed_time(ev[1]) * 1e3
                t_ar = ev[2].elapsed_time(ev[3]) * 1e3
                first = ev[0] if ev[0].elapsed_time(ev[2]) >= 0 else ev[2]
                last_mm = first.elapsed_time(ev[1]) * 1e3
                last_ar = first.elapsed_time(ev[3]) * 1e3
                rows.append((t_ar, t_mm, max(last_mm, last_ar)))
        return [float(np.median([r[k] for r in rows])) for k in range(3)]

    # size the GEMM side to about the AllReduce's length
    t_one = alone(gemm, s_mm)
    t_ar0 = alone(lambda: plan.start(s_ar), s_ar)
    gemm_calls = max(1, int(round(t_ar0 / t_one)))
    t_mm = alone(gemm, s_mm)
    log(f"[interference] GEMM {dim}^3 bf16 x{gemm_calls}: {t_mm:.1f} us alone; AllReduce {t_ar0:.1f} us alone")
    for cap in (0, 2048, 1024, 512, 256, 128, 64):
        plan.limit_blocks(cap)
        t_ar = alone(lambda: plan.start(s_ar), s_ar)
        for ar_first in (False, True):
            o_ar, o_mm, span = together(ar_first)
            print(json.dumps({
                "interference": "fused AllReduce 8 x 2^26 f32 beside bf16 GEMM",
                "gemm": f"{dim}x{dim}x{dim} x{gemm_calls}", "launched_first": "allreduce" if ar_first else "gemm",
                "ar_blocks": cap if cap else "one per tile",
                "ar_alone_us": round(t_ar, 1), "ar_alone_hbm_gbps": round(2 * n * s_bytes / t_ar / 1e3, 1),
                "gemm_alone_us": round(t_mm, 1), "gemm_alone_tflops": round(gemm_calls * flops / t_mm / 1e6, 1),
                "ar_overlap_us": round(o_ar, 1), "gemm_overlap_us": round(o_mm, 1), "makespan_us": round(span, 1),
                "sequential_us": round(t_ar + t_mm, 1),
                "gemm_slowdown_us": round(o_mm - t_mm, 1), "ar_slowdown_us": round(o_ar - t_ar, 1)}), flush=True)
    plan.limit_blocks(0)
    plan.close()


def load_probe_library():
    """libarprobe.so (the HBM ceiling probes), or None when it is not built."""
    import ctypes

    from ring_allreduce_reduction_virtual_amd import build as arbuild

    if not os.path.exists(arbuild.PROBE_PATH):
        return None
    lib = ctypes.CDLL(arbuild.PROBE_PATH)
    lib.arprobe_stream.restype = ctypes.c_int
    lib.arprobe_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64,
                                   ctypes.c_void_p, ctypes.c_void_p]
    lib.arprobe_pattern.restype = ctypes.c_int
    lib.arprobe_pattern.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint64, ctypes.c_void_p,
                                    ctypes.c_int, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
    lib.arprobe_copy_order.restype = ctypes.c_int
    lib.arprobe_copy_order.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_uint64, ctypes.c_void_p]
    lib.arprobe_xcd.restype = ctypes.c_int
    lib.arprobe_xcd.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64,
                                ctypes.c_void_p]
    lib.arprobe_wmap.restype = ctypes.c_int
    lib.arprobe_wmap.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64,
                                 ctypes.c_void_p]
    return lib


WMAPS = {0: "grouped per XCD (a tile's workgroups on one XCD, as the staged broadcast)",
         1: "tile-major (workgroup b: buffer b mod n)",
         2: "buffer-major",
         3: "one contiguous buffer-major range per XCD",
         4: "one contiguous tile-major range per XCD",
         5: "one contiguous eighth of the tiles per XCD, in runs of 16 tiles buffer by buffer",
         6: "one contiguous eighth of the tiles per XCD, in runs of 64 tiles buffer by buffer",
         7: "one contiguous eighth of the tiles per XCD, in runs of 256 tiles buffer by buffer"}


def run_write_maps(lib, steps=20, rounds=3):
    """Writes of 7 and 8 buffers of 128 MiB (the staged broadcast's segment at
    8 ranks: 7 destinations), one 8 KiB tile per workgroup, nontemporal
    stores, in each of the workgroup -> (buffer, tile) maps of k_wmap; alone,
    and with each workgroup loading its tile from one 128 MiB source first, as
    the broadcast does (the source rewritten by torch just before each call).
    The maps are interleaved over `rounds` passes on the same buffers and the
    best median kept.  One JSON line per map and form."""
    import ctypes

    import torch

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    mib = 1 << 20
    size = 128 * mib
    nvec = size // 16
    src = torch.ones(size // 4, device=dev)
    dst = [torch.empty(size // 4, device=dev) for _ in range(8)]
    best = {}
    for _ in range(rounds):
        for n in (7, 8):
            tbl = (ctypes.c_void_p * n)(*[t.data_ptr() for t in dst[:n]])
            for with_src in (False, True):
                for m in WMAPS:
                    ts = []
                    for i in range(steps + 3):
                        if with_src:
                            src.fill_(float(i))
                        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                        e0.record(stream)
                        rc = lib.arprobe_wmap(m, src.data_ptr() if with_src else None, tbl, n, nvec,
                                              ctypes.c_void_p(stream.cuda_stream))
                        e1.record(stream)
                        e1.synchronize()
                        if rc != 0:
                            raise RuntimeError(f"arprobe_wmap map {m}: error {rc}")
                        if i >= 3:
                            ts.append(e0.elapsed_time(e1) * 1e3)
                    ts.sort()
                    key = (n, with_src, m)
                    best[key] = min(best.get(key, 1e18), ts[len(ts) // 2])
    for (n, with_src, m), us in sorted(best.items()):
        nbytes = n * size
        print(json.dumps({"write_map": WMAPS[m], "map": m, "buffers": f"{n} x 128 MiB",
                          "source": "each tile loaded from a 128 MiB source first" if with_src else "none",
                          "bytes_written": nbytes, "us": round(us, 1), "write_tbps": round(nbytes / us / 1e6, 3),
                          "frac_of_8tbps": round(nbytes / us / 1e6 / (HBM_PEAK_GBPS / 1e3), 4)}), flush=True)


def run_xcd_patterns(lib, steps=20):
    """Whether the fast write pattern is about XCDs: writes in which XCD x
    writes buffer x only (8 buffers, and 7 with one XCD idle), against the
    tile-major order over 7 and 16 buffers, where XCDs and buffers do not
    line up; then the staged broadcast's shape (a just-written source copied
    to 7 destinations) with one workgroup per tile storing to all 7, against
    XCD x copying to destination x only, for 128 MiB and 32 MiB sources.
    One JSON line each; median of `steps` event-timed calls."""
    import ctypes

    import torch

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    def timed(fn, before=None):
        ts = []
        for i in range(steps + 3):
            if before is not None:
                before()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            if i >= 3:
                ts.append(e0.elapsed_time(e1) * 1e3)
        ts.sort()
        return ts[len(ts) // 2]

    def check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what}: error {rc}")

    def emit(direction, pattern, nbytes, us, buffers):
        row = {"ceiling_pattern": pattern, "direction": direction, "buffers": buffers, "bytes": nbytes,
               "us": round(us, 1), "tbps": round(nbytes / us / 1e6, 3),
               "frac_of_8tbps": round(nbytes / us / 1e6 / (HBM_PEAK_GBPS / 1e3), 4)}
        print(json.dumps(row), flush=True)

    mib = 1 << 20
    # reads and writes together: copies of 8 x 256 MiB in the kernels' order and the write-friendly orders,
    # each timed twice, interleaved, on the same buffers
    n, size = 8, 256 * mib
    src = [torch.ones(size // 4, device=dev) for _ in range(n)]
    dst = [torch.empty(size // 4, device=dev) for _ in range(n)]
    sp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in src])
    dp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in dst])
    nvec = size // 16
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    for rep in range(2):
        emit("copy", "kernels' pattern: 8 KiB of every buffer per workgroup, nontemporal", 2 * n * size,
             timed(lambda: check(lib.arprobe_stream(2, sp, dp, n, nvec, sink.data_ptr(), stream.cuda_stream),
                                 "copy")), f"{n} x {size >> 20} MiB")
        for order, oname in ((1, "tile-major"), (0, "buffer-major")):
            for nt in (0, 1):
                emit("copy", f"one buffer per workgroup, 8 KiB, {oname}, "
                             f"{'nontemporal' if nt else 'plain'} stores", 2 * n * size,
                     timed(lambda: check(lib.arprobe_copy_order(order, nt, sp, dp, n, nvec, stream.cuda_stream),
                                         "copy order")), f"{n} x {size >> 20} MiB")
    del src, dst
    for n, size in ((8, 256 * mib), (7, 256 * mib)):
        bufs = [torch.empty(size // 4, device=dev) for _ in range(n)]
        bp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in bufs])
        nvec = size // 16
        emit("write", f"XCD x writes buffer x only ({n} buffers; {8 - n} XCDs idle), 8 KiB per workgroup, plain",
             n * size, timed(lambda: check(lib.arprobe_xcd(0, None, bp, n, nvec, stream.cuda_stream), "xcd")),
             f"{n} x {size >> 20} MiB")
        if n == 7:
            emit("write", "one buffer per workgroup, 8 KiB runs, tile-major over 7 buffers, plain", n * size,
                 timed(lambda: check(lib.arprobe_pattern(1, 0, 1, 512, bp, n, nvec, None, stream.cuda_stream),
                                     "pattern")), f"{n} x {size >> 20} MiB")
        del bufs
    n, size = 16, 128 * mib
    bufs = [torch.empty(size // 4, device=dev) for _ in range(n)]
    bp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in bufs])
    emit("write", "one buffer per workgroup, 8 KiB runs, tile-major over 16 buffers, plain", n * size,
         timed(lambda: check(lib.arprobe_pattern(1, 0, 1, 512, bp, n, size // 16, None, stream.cuda_stream),
                             "pattern")), f"{n} x {size >> 20} MiB")
    del bufs
    for g in (128 * mib, 32 * mib):
        src = torch.empty(g // 4, device=dev)
        sp = (ctypes.c_void_p * 1)(src.data_ptr())
        dst = [torch.empty(g // 4, device=dev) for _ in range(7)]
        dp = (ctypes.c_void_p * 7)(*[t.data_ptr() for t in dst])
        nvec = g // 16

        def produce():
            check(lib.arprobe_pattern(1, 0, 1, 512, sp, 1, nvec, None, stream.cuda_stream), "produce")

        for kind, name in ((1, "one workgroup per tile storing to all 7"), (2, "XCD x copies to destination x")):
            us = timed(lambda: check(lib.arprobe_xcd(kind, src.data_ptr(), dp, 7, nvec, stream.cuda_stream), "bcast"),
                       before=produce)
            emit("write", f"broadcast of a just-written {g >> 20} MiB source to 7 destinations: {name}", 7 * g, us,
                 f"1 + 7 x {g >> 20} MiB")
        del src, dst
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def run_ceiling_patterns(lib, n=8, count=1 << 26, steps=20):
    """Read and write rates of HBM for access patterns other than the kernels'
    own, over n buffers of `count` float32 (the headline's 8 x 256 MiB by
    default), one JSON line per pattern: the kernels' pattern (each workgroup
    one 8 KiB tile of every buffer) with nontemporal and plain stores; one
    buffer per workgroup with contiguous runs of 8, 64 and 256 KiB, in
    buffer-major and tile-major block order, nontemporal and plain; reads the
    same ways; and torch's fill_ and hipMemsetD32Async on one 2 GiB tensor.
    Median of `steps` single calls, event-timed."""
    import ctypes

    import torch

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    bufs = [torch.empty(count, device=dev) for _ in range(n)]
    for t in bufs:
        t.fill_(0.5)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    bp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in bufs])
    nvec = count * 4 // 16
    nbytes = n * count * 4
    rows = []

    def emit(direction, pattern, us):
        row = {"ceiling_pattern": pattern, "direction": direction, "buffers": f"{n} x {count * 4 >> 20} MiB",
               "bytes": nbytes, "us": round(us, 1), "tbps": round(nbytes / us / 1e6, 3),
               "frac_of_8tbps": round(nbytes / us / 1e6 / (HBM_PEAK_GBPS / 1e3), 4)}
        rows.append(row)
        print(json.dumps(row), flush=True)

    def timed(fn):
        return median_call_ms(fn, steps, 3, stream)[0] * 1e3

    def stream_probe(kind):
        rc = lib.arprobe_stream(kind, bp, bp, n, nvec, sink.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"arprobe_stream {kind}: {rc}")

    def pattern_probe(write, nt, order, run):
        rc = lib.arprobe_pattern(write, nt, order, run, bp, n, nvec, sink.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"arprobe_pattern {write} {nt} {order} {run}: {rc}")

    emit("write", "kernels' pattern: 8 KiB of every buffer per workgroup, nontemporal", timed(lambda: stream_probe(1)))
    emit("write", "kernels' pattern: 8 KiB of every buffer per workgroup, plain stores",
         timed(lambda: pattern_probe(1, 0, 0, 0)))
    for run_kib in (8, 64, 256):
        run = run_kib * 1024 // 16
        for order, oname in ((0, "buffer-major"), (1, "tile-major")):
            for nt in (1, 0):
                emit("write", f"one buffer per workgroup, {run_kib} KiB runs, {oname}, "
                              f"{'nontemporal' if nt else 'plain stores'}",
                     timed(lambda: pattern_probe(1, nt, order, run)))
    emit("read", "kernels' pattern: 8 KiB of every buffer per workgroup, nontemporal", timed(lambda: stream_probe(0)))
    for run_kib in (64, 256):
        run = run_kib * 1024 // 16
        for order, oname in ((0, "buffer-major"), (1, "tile-major")):
            emit("read", f"one buffer per workgroup, {run_kib} KiB runs, {oname}, nontemporal",
                 timed(lambda: pattern_probe(0, 1, order, run)))
    del bufs
    torch.cuda.empty_cache()
    big = torch.empty(n * count, device=dev)
    emit("write", "torch fill_ of one 2 GiB tensor", timed(lambda: big.fill_(1.0)))
    hip = ctypes.CDLL("libamdhip64.so.7")
    hip.hipMemsetD32Async.restype = ctypes.c_int
    hip.hipMemsetD32Async.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_void_p]

    def memset():
        rc = hip.hipMemsetD32Async(big.data_ptr(), 7, big.numel(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"hipMemsetD32Async: {rc}")

    emit("write", "hipMemsetD32Async of one 2 GiB tensor", timed(memset))
    del big
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rows


def probe_times_us(lib, src, dst, stream, kinds=(("read", 0), ("write", 1), ("copy", 2), ("mix", 3)), steps=20):
    """Median µs of each probe over the tensors src -> dst (n buffers of equal size)."""
    import ctypes

    import torch

    n = len(src)
    sink = torch.zeros(4, dtype=torch.int32, device=src[0].device)
    sp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in src])
    dp = (ctypes.c_void_p * n)(*[t.data_ptr() for t in dst])
    nvec = src[0].numel() * src[0].element_size() // 16

    def probe(kind):
        rc = lib.arprobe_stream(kind, sp, dp, n, nvec, sink.data_ptr(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"arprobe_stream kind {kind}: error {rc}")

    return {name: median_call_ms(lambda: probe(kind), steps, 3, stream)[0] * 1e3 for name, kind in kinds}


def run_ceiling(args):
    """What HBM allows for the AllReduce's traffic, measured beside it.

    The probes of libarprobe.so stream the same buffers with the fused
    kernel's access pattern (one block per 8 KiB tile of every buffer,
    nontemporal hints): reads alone, writes alone, a copy, and an
    AllReduce-shaped mix (read n buffers, store the integer sum to n buffers)
    with none of the chunk logic or float work.  Reading N*S and writing N*S
    over one memory bus cannot take less than the two streams take alone,
    t_read + t_write; the fused AllReduce is reported against that bound and
    against the mix probe.
    """
    import torch

    import ring_allreduce_reduction_virtual_amd as ar

    lib = load_probe_library()
    if lib is None:
        raise SystemExit("libarprobe.so is not built (python -m ring_allreduce_reduction_virtual_amd.build)")
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    run_ceiling_patterns(lib)
    run_xcd_patterns(lib)
    run_write_maps(lib)
    if args.patterns_only:
        return
    for n, count in ((8, 1 << 26), (16, 1 << 24), (64, 1 << 26)):
        s_bytes = count * 4
        src = [torch.randn(count, device=dev) for _ in range(n)]
        dst = [torch.empty(count, device=dev) for _ in range(n)]
        t = probe_times_us(lib, src, dst, stream)
        t["fused"] = median_call_ms(lambda: ar.ar_allreduce_ex(src, dst, algo="fused"), 20, 3, stream)[0] * 1e3
        t["phases"] = median_call_ms(lambda: ar.ar_allreduce_ex(src, dst, algo="phases"), 20, 3, stream)[0] * 1e3
        t["staged"] = median_call_ms(lambda: ar.ar_allreduce_ex(src, dst, algo="staged"), 20, 3, stream)[0] * 1e3
        nbytes = n * s_bytes
        bound = t["read"] + t["write"]
        print(json.dumps({
            "ceiling": f"{n} buffers x {s_bytes >> 20} MiB",
            "read_us": round(t["read"], 1), "read_gbps": round(nbytes / t["read"] / 1e3, 1),
            "write_us": round(t["write"], 1), "write_gbps": round(nbytes / t["write"] / 1e3, 1),
            "copy_us": round(t["copy"], 1), "copy_gbps": round(2 * nbytes / t["copy"] / 1e3, 1),
            "mix_us": round(t["mix"], 1), "mix_gbps": round(2 * nbytes / t["mix"] / 1e3, 1),
            "fused_allreduce_us": round(t["fused"], 1), "fused_allreduce_gbps": round(2 * nbytes / t["fused"] / 1e3, 1),
            "phases_allreduce_us": round(t["phases"], 1),
            "staged_allreduce_us": round(t["staged"], 1),
            "staged_frac_of_bound": round(bound / t["staged"], 4),
            "bound_read_plus_write_us": round(bound, 1),
            "bound_frac_of_8tbps": round(2 * nbytes / bound / 1e3 / HBM_PEAK_GBPS, 4),
            "fused_frac_of_bound": round(bound / t["fused"], 4),
            "fused_frac_of_mix_probe": round(t["mix"] / t["fused"], 4)}), flush=True)
        del src, dst
        torch.cuda.empty_cache()


SWEEP_ALGOS = ("fused", "ring", "ring_persistent", "ring_pipelined", "tree", "tree_steps", "recursive_doubling",
               "halving_doubling_steps", "double_binary_tree", "double_binary_tree_steps")


def dbt_steps_bytes_factor(n: int) -> int:
    """HBM bytes of the double binary tree's level-by-level schedule in units of S.

    Per tree (half the buffer): each of the floor(N/2) inner nodes reads its
    own half and one partial per child (N - 1 children in all) and writes its
    partial; going down, each inner node reads its half once and writes it to
    every child.  Reads 2 floor(N/2) + N - 1 halves and writes
    floor(N/2) + N - 1; the two trees together 3 floor(N/2) + 2 (N - 1) times S.
    """
    return 3 * (n // 2) + 2 * (n - 1)


def run_size_sweep(args):
    """AllReduce time against message size, 8 ranks of float32, every schedule.

    Fits the cost model of tirogla.com "Ring all-reduce" on one GPU,
    t = launches * a + HBM bytes / B: one launch and 2*N*S bytes for the fused
    kernels, 2(N-1) launches and 5(N-1)*S bytes for the ring's steps,
    2 log2 N launches and 5(N-1)*S bytes for the staged tree and
    halving/doubling, log2 N launches and 2*N*S*log2 N bytes for recursive
    doubling.  The persistent ring is fitted like the ring's steps, its
    2(N-1) steps separated by grid barriers instead of launches; the
    pipelined ring with one launch and the ring's 5(N-1)*S bytes, of which
    the re-read partials mostly come from the caches (its fitted B is then
    above what HBM alone would give those bytes).
    """
    import numpy as np
    import torch

    import ring_allreduce_reduction_virtual_amd as ar

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    n = 8
    rows = []
    for k in range(0, 29, 2):               # 1 element to 2^28 (1 GiB) per rank
        count = 1 << k
        sends = [torch.randn(count, device=dev) for _ in range(n)]
        recvs = [torch.empty(count, device=dev) for _ in range(n)]
        for algo in SWEEP_ALGOS:
            med, mn = median_call_ms(lambda: ar.ar_allreduce_ex(sends, recvs, algo=algo), 50, 5, stream)
            rows.append((algo, count, med))
            s_bytes = count * 4
            print(json.dumps({"sweep": "allreduce", "algo": algo, "nranks": n, "count": count, "bytes_per_rank": s_bytes,
                              "median_us": round(med * 1e3, 2), "min_us": round(mn * 1e3, 2),
                              "algbw_gbps": round(s_bytes / (med / 1e3) / 1e9, 3),
                              "busbw_gbps": round(s_bytes / (med / 1e3) / 1e9 * busbw_factor("allreduce", n), 3)}),
                  flush=True)
        del sends, recvs
    fits = {}
    L = (n - 1).bit_length()
    for algo, bytes_factor, launches in (("fused", 2 * n, 1), ("ring", 5 * (n - 1), 2 * (n - 1)),
                                         ("ring_persistent", 5 * (n - 1), 2 * (n - 1)),
                                         ("ring_pipelined", 5 * (n - 1), 1),
                                         ("tree", 2 * n, 1), ("tree_steps", 5 * (n - 1), 2 * L),
                                         ("recursive_doubling", 2 * n * L, L),
                                         ("halving_doubling_steps", 5 * (n - 1), 2 * L),
                                         ("double_binary_tree", 2 * n, 1),
                                         ("double_binary_tree_steps", dbt_steps_bytes_factor(n),
                                          2 * (n.bit_length() - 1))):
        pts = [(c * 4 * bytes_factor, t / 1e3) for a, c, t in rows if a == algo]
        A = np.array([[launches, b] for b, _ in pts], dtype=np.float64)
        y = np.array([t for _, t in pts])
        (alpha, inv_b), *_ = np.linalg.lstsq(A, y, rcond=None)
        fits[algo] = {"alpha_us_per_launch": round(alpha * 1e6, 3), "hbm_gbps": round(1 / inv_b / 1e9, 1)}
    print(json.dumps({"sweep_fit": fits, "model": "t = launches*alpha + hbm_bytes/B"}), flush=True)


FORM_SWEEP = ((8, 256, "float32"), (8, 128, "float32"), (8, 64, "float32"), (8, 32, "float32"),
              (8, 16, "float32"), (8, 4, "float32"), (16, 256, "float32"), (16, 64, "float32"),
              (16, 16, "float32"), (32, 128, "float32"), (32, 32, "float32"), (64, 256, "float32"),
              (64, 64, "float32"), (64, 16, "float32"), (128, 64, "float32"), (4, 256, "float32"),
              (6, 256, "float32"), (2, 512, "float32"), (8, 128, "bfloat16"), (8, 64, "bfloat16"),
              (16, 64, "bfloat16"), (16, 64, "int32"))


def run_form_sweep(args):
    """The three ring-order forms of a large AllReduce side by side (fused,
    phases, staged) over rank counts and sizes: the measurements behind
    AR_ALGO_AUTO's bounds.  Median of 10 single calls each, the three forms
    interleaved, one JSON line per shape (MiB per rank, element type)."""
    import torch

    import ring_allreduce_reduction_virtual_amd as ar

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    for n, mib, dt in FORM_SWEEP:
        tdt = getattr(torch, dt)
        count = (mib << 20) // torch.empty(0, dtype=tdt).element_size()
        if dt == "int32":
            sends = [torch.randint(-2**31, 2**31 - 1, (count,), dtype=tdt, device=dev) for _ in range(n)]
        else:
            sends = [torch.randn(count, device=dev).to(tdt) for _ in range(n)]
        recvs = [torch.empty(count, dtype=tdt, device=dev) for _ in range(n)]
        us = {}
        for rep in range(2):
            for algo in ("fused", "phases", "staged"):
                med, _ = median_call_ms(lambda: ar.ar_allreduce_ex(sends, recvs, algo=algo), 10, 2, stream)
                us.setdefault(algo, []).append(med * 1e3)
        plan = ar.ar_allreduce_init(sends, recvs, algo="auto")
        auto_launches = plan.num_launches
        plan.close()
        row = {"form_sweep": f"{n} x {mib} MiB {dt}", "nranks": n, "mib_per_rank": mib, "dtype": dt,
               "us": {k: round(min(v), 1) for k, v in us.items()}, "auto_launches": auto_launches}
        print(json.dumps(row), flush=True)
        del sends, recvs
        torch.cuda.empty_cache()


RANK_SCALING = ((8, 1 << 26), (16, 1 << 26), (32, 1 << 26), (64, 1 << 26), (64, (1 << 26) + 7))


def run_rank_scaling(args):
    """The fused AllReduce at 8 to 64 ranks of 256 MiB of float32 each (and
    the 64-rank workload's own length, 2^26 + 7), beside the staged form: the
    same bytes per rank, more interleaved streams.  Median of --steps single
    calls after --warmup, one JSON line per shape.  Run under rocprofv3 with
    address-translation and memory-side counters, it is the command of the
    fused kernel's rank-count counter summary.  --shapes replaces the shapes
    (N x count pairs, e.g. 8x67108864,8x268435456: the same 8 ranks with more
    bytes each).  --alloc-factors F1,F2,... runs every shape on views of the
    first `count` elements of allocations F times larger, the factors
    alternating in three rounds in one process (same bytes touched, different
    allocations)."""
    import torch

    import ring_allreduce_reduction_virtual_amd as ar

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    shapes = RANK_SCALING
    if args.shapes:
        shapes = tuple(tuple(int(v) for v in s.split("x")) for s in args.shapes.split(","))
    if args.alloc_factors:
        factors = [int(v) for v in args.alloc_factors.split(",")]
        for n, count in shapes:
            cases = {}
            for f in factors:
                base_s = [torch.randn(count * f, device=dev) for _ in range(n)]
                base_r = [torch.empty(count * f, device=dev) for _ in range(n)]
                cases[f] = ([t[:count] for t in base_s], [t[:count] for t in base_r])
            times = {(f, algo): [] for f in factors for algo in ("fused", "staged")}
            for _ in range(3):
                for f in factors:
                    sends, recvs = cases[f]
                    for algo in ("fused", "staged"):
                        med, _ = median_call_ms(lambda: ar.ar_allreduce_ex(sends, recvs, algo=algo),
                                                max(args.steps, 1), args.warmup, stream)
                        times[(f, algo)].append(round(med * 1e3, 1))
            for f in factors:
                print(json.dumps({"rank_scaling": f"{n} x {count} f32 sum", "nranks": n, "count": count,
                                  "alloc_factor": f, "fused_us": times[(f, "fused")],
                                  "staged_us": times[(f, "staged")]}), flush=True)
            del cases
            torch.cuda.empty_cache()
        return
    for n, count in shapes:
        sends = [torch.randn(count, device=dev) for _ in range(n)]
        recvs = [torch.empty(count, device=dev) for _ in range(n)]
        row = {"rank_scaling": f"{n} x {count} f32 sum", "nranks": n, "count": count}
        for algo in ("fused", "staged"):
            med, best = median_call_ms(lambda: ar.ar_allreduce_ex(sends, recvs, algo=algo),
                                       max(args.steps, 1), args.warmup, stream)
            row[f"{algo}_us"] = round(med * 1e3, 1)
            row[f"{algo}_hbm_frac"] = round(2 * n * count * 4 / (med * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
        print(json.dumps(row), flush=True)
        del sends, recvs
        torch.cuda.empty_cache()


def run_cache_sweep(args):
    """The fused AllReduce around the bound of its cache-allocating loads.

    Inputs of N*S = 32 to 512 MiB of float32 at 8, 16 and 64 ranks, per call
    in a replayed HIP graph of 20 plan starts (the same buffers every call, as
    a benchmark loop or a training step's repeated bucket sees them).  The
    library reads inputs of at most 256 MiB with cache-allocating loads and
    larger ones with nontemporal loads; run under AR_CACHED_LOADS_MAX=0 (never
    cached) or a huge value (always cached) for the other forms.
    """
    import torch

    import ring_allreduce_reduction_virtual_amd as ar

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    form = os.environ.get("AR_CACHED_LOADS_MAX", "default (256 MiB)")
    for n in (8, 16, 64):
        for mib in (32, 128, 192, 256, 320, 384, 512):
            count = (mib << 20) // (4 * n)
            sends = [torch.randn(count, device=dev) for _ in range(n)]
            recvs = [torch.empty(count, device=dev) for _ in range(n)]
            plan = ar.ar_allreduce_init(sends, recvs, algo="fused")
            per_call = [graph_ms_per_call(plan.start, 20, stream, replays=3) * 1e3 for _ in range(3)]
            us = sorted(per_call)[1]
            print(json.dumps({"cache_sweep": "allreduce fused f32 sum", "AR_CACHED_LOADS_MAX": form, "nranks": n,
                              "inputs_mib": mib, "count": count, "graph_us_per_call": round(us, 2),
                              "hbm_frac": round(2 * n * count * 4 / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)}),
                  flush=True)
            plan.close()
            del sends, recvs
            torch.cuda.empty_cache()


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def release():
    """Close what a run leaves alive and wait for the GPU before the interpreter
    exits: plans and captured graphs dropped, the caching allocator emptied,
    the device synchronized.  The HIP runtime and a profiler attached to the
    process then tear down with nothing of the run still pending."""
    import gc

    gc.collect()
    if "torch" in sys.modules:
        import torch

        if torch.cuda.is_initialized():
            torch.cuda.synchronize()
            torch.cuda.empty_cache()


def main():
    try:
        _main()
    finally:
        release()


def _main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the CPU oracle")
    ap.add_argument("--algo", default="auto", choices=STEP_ALGOS,
                    help="the AllReduce algorithm the step runs (default: the library's default); every one "
                         "but auto, fused, phases and staged runs another schedule or order, timed against "
                         "the same 2*N*S minimum")
    ap.add_argument("--no-extra", action="store_true", help="skip the ring / phase / copy side measurements")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (calibrates HBM byte counters)")
    ap.add_argument("--configs", action="store_true",
                    help="instead of the headline line: time every workload (c1..c5) with both algorithms, "
                         "one JSON line each")
    ap.add_argument("--workloads", default="",
                    help="with --configs: comma-separated workload names (default: all, the headline twice)")
    ap.add_argument("--shapes", default="",
                    help="with --rank-scaling: comma-separated NxCOUNT shapes instead of the default ones")
    ap.add_argument("--alloc-factors", default="",
                    help="with --rank-scaling: run each shape on views into allocations this many times larger "
                         "(comma-separated factors, alternating in one process)")
    ap.add_argument("--variants", action="store_true",
                    help="instead of the headline line: time the precision and operator variants "
                         "(float32 partials for bf16, avg, binary16) at full size, one JSON line each")
    ap.add_argument("--orders", action="store_true",
                    help="instead of the headline line: the tree-shaped orders beside the ring at full size "
                         "and in the latency regime (one-shot, plan, graph)")
    ap.add_argument("--interference", action="store_true",
                    help="instead of the headline line: the fused AllReduce overlapping a bf16 GEMM, "
                         "with the AllReduce's workgroups capped at several sizes")
    ap.add_argument("--ceiling", action="store_true",
                    help="instead of the headline line: HBM read-only, write-only, copy and AllReduce-shaped "
                         "probes beside the fused AllReduce (the bound its traffic allows)")
    ap.add_argument("--patterns-only", action="store_true",
                    help="with --ceiling: only the table of read and write patterns (8 x 256 MiB)")
    ap.add_argument("--size-sweep", action="store_true",
                    help="instead of the headline line: AllReduce time against message size (8 ranks, f32, 1 element "
                         "to 1 GiB per rank), every schedule, with an alpha-beta fit")
    ap.add_argument("--form-sweep", action="store_true",
                    help="instead of the headline line: fused, phases and staged AllReduce side by side over rank "
                         "counts and sizes (the measurements behind the default's choice)")
    ap.add_argument("--cache-sweep", action="store_true",
                    help="instead of the headline line: the fused AllReduce at 32-512 MiB of inputs and 8, 16, "
                         "64 ranks, per call in a replayed graph (around the bound of its cache-allocating loads)")
    ap.add_argument("--rank-scaling", action="store_true",
                    help="instead of the headline line: the fused and staged AllReduce at 8, 16, 32 and 64 ranks "
                         "of 256 MiB float32 each (the 64-rank workload's length too)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the ring's N ranks are virtual, held as N buffers in "
              "one GPU's HBM; there is no multi-GPU run", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    ensure_library()
    import ring_allreduce_reduction_virtual_amd as ar
    from inputs import WORKLOADS, make_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.configs:
        run_configs(args)
        return
    if args.size_sweep:
        run_size_sweep(args)
        return
    if args.variants:
        run_variants(args)
        return
    if args.orders:
        run_orders(args)
        return
    if args.interference:
        run_interference(args)
        return
    if args.ceiling:
        run_ceiling(args)
        return
    if args.cache_sweep:
        run_cache_sweep(args)
        return
    if args.form_sweep:
        run_form_sweep(args)
        return
    if args.rank_scaling:
        run_rank_scaling(args)
        return
    w = WORKLOADS["headline"]
    n, count = w.nranks, w.count
    s_bytes = count * 4
    log(f"[bench] device {torch.cuda.get_device_name(dev)}; workload N={n} x {count} f32 sum; drawing inputs")
    t0 = time.perf_counter()
    xs = make_inputs(w)
    sends = [torch.from_numpy(x).to(dev) for x in xs]
    recvs = [torch.empty(count, dtype=torch.float32, device=dev) for _ in range(n)]
    torch.cuda.synchronize()
    log(f"[bench] inputs resident in HBM ({time.perf_counter() - t0:.1f} s)")
    stream = torch.cuda.current_stream()

    def step():
        if args.algo == "auto":
            ar.ar_allreduce(sends, recvs)
        else:
            ar.ar_allreduce_ex(sends, recvs, algo=args.algo)

    # which form the timed call takes here (the library's default, AR_ALGO_AUTO,
    # unless --algo names one), as the plan of the same call reports it
    plan = ar.ar_allreduce_init(sends, recvs, algo=args.algo)
    default_algo, timed_launches = plan.algo, plan.num_launches
    plan.close()
    launches = {"timed": timed_launches}
    if default_algo == "staged":
        segments = timed_launches // 2
        kernel_name = (f"k_staged_reduce<f32,sum,vec16> + k_staged_broadcast_xcd<f32,vec16>, "
                       f"{segments} segments of {s_bytes // segments >> 20} MiB of results")
    else:
        kernel_name = STEP_KERNELS[default_algo].format(launches=timed_launches)

    # timed region: K AllReduce calls, synchronized on both sides
    ms = time_calls(step, args.steps, args.warmup, stream)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - wall0) * 1e3 / args.steps
    t_s = ms / 1e3
    algbw = s_bytes / t_s / 1e9
    busbw = algbw * busbw_factor("allreduce", n)
    algo_bytes = algorithmic_bytes("allreduce", n, s_bytes)
    hbm_gbps = algo_bytes / t_s / 1e9
    log(f"[bench] AllReduce ({default_algo}, {launches['timed']} launches): {ms * 1e3:.1f} us/call "
        f"(wall {wall_ms * 1e3:.1f} us), algbw {algbw:.1f} GB/s, "
        f"busbw {busbw:.1f} GB/s, HBM {hbm_gbps:.0f} GB/s = {hbm_gbps / HBM_PEAK_GBPS:.1%} of 8 TB/s")

    extra = {"wall_ms_per_step": round(wall_ms, 4)}
    if not args.no_extra:
        # the one-pass fused kernel on the same buffers
        fused_ms = time_calls(lambda: ar.ar_allreduce_ex(sends, recvs, algo="fused"), max(10, args.steps // 2), 2,
                              stream)
        extra["fused_ms"] = round(fused_ms, 4)
        extra["fused_hbm_frac_of_peak"] = round(algo_bytes / (fused_ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4)
        # the other large-buffer forms on the same buffers (the same bits)
        for form in ("phases", "staged"):
            f_ms = time_calls(lambda: ar.ar_allreduce_ex(sends, recvs, algo=form), max(10, args.steps // 2), 2, stream)
            extra[f"{form}_ms"] = round(f_ms, 4)
            extra[f"{form}_hbm_frac_of_peak"] = round(algo_bytes / (f_ms / 1e3) / 1e9 / HBM_PEAK_GBPS, 4)
        # the step-faithful ring mode and the phases alone, on the same buffers
        ring_ms = time_calls(lambda: ar.ar_allreduce_ex(sends, recvs, algo="ring"), max(3, args.steps // 10), 1, stream)
        extra["ring_mode_ms"] = round(ring_ms, 4)
        extra["ring_mode_hbm_gbps_of_minimum"] = round(algo_bytes / (ring_ms / 1e3) / 1e9, 1)
        # the same steps pipelined slice by slice in one launch
        pipe_ms = time_calls(lambda: ar.ar_allreduce_ex(sends, recvs, algo="ring_pipelined"),
                             max(3, args.steps // 10), 1, stream)
        extra["ring_pipelined_ms"] = round(pipe_ms, 4)
        extra["ring_pipelined_hbm_gbps_of_minimum"] = round(algo_bytes / (pipe_ms / 1e3) / 1e9, 1)
        shards = [recvs[r][slice(*ar.ar_chunk_range(r, count, n))] for r in range(n)]
        rs_ms = time_calls(lambda: ar.ar_reduce_scatter(sends, shards), 20, 2, stream)
        ag_ms = time_calls(lambda: ar.ar_all_gather(shards, sends), 20, 2, stream)
        rs_bytes = algorithmic_bytes("reduce_scatter", n, s_bytes)
        extra["reduce_scatter_ms"] = round(rs_ms, 4)
        extra["reduce_scatter_hbm_gbps"] = round(rs_bytes / (rs_ms / 1e3) / 1e9, 1)
        extra["all_gather_ms"] = round(ag_ms, 4)
        extra["all_gather_hbm_gbps"] = round(rs_bytes / (ag_ms / 1e3) / 1e9, 1)
        # a plain device-to-device copy of the same byte volume: the streaming ceiling for reference
        src = torch.empty(n * count, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        copy_ms = time_calls(lambda: dst.copy_(src), 20, 2, stream)
        extra["torch_copy_2x2GiB_hbm_gbps"] = round(2 * src.numel() * 4 / (copy_ms / 1e3) / 1e9, 1)
        del src, dst
        # what HBM gives this traffic: the probes of libarprobe.so on the same buffers (bench.py --ceiling)
        plib = load_probe_library()
        if plib is not None:
            pt = probe_times_us(plib, sends, recvs, stream, kinds=(("read", 0), ("write", 1), ("mix", 3)))
            extra["hbm_ceiling"] = {
                "read_alone_us": round(pt["read"], 1), "write_alone_us": round(pt["write"], 1),
                "read_plus_write_us": round(pt["read"] + pt["write"], 1),
                "read_plus_write_frac_of_8tbps": round(algo_bytes / (pt["read"] + pt["write"]) / 1e3 / HBM_PEAK_GBPS, 4),
                "mix_probe_us": round(pt["mix"], 1),
                "allreduce_frac_of_read_plus_write": round((pt["read"] + pt["write"]) / (ms * 1e3), 4),
                "allreduce_speed_vs_mix_probe": round(pt["mix"] / (ms * 1e3), 4)}
        log(f"[bench] fused {fused_ms:.3f} ms; phases {extra['phases_ms']:.3f} ms; staged {extra['staged_ms']:.3f} ms; "
            f"ring mode {ring_ms:.3f} ms; pipelined ring {pipe_ms:.3f} ms; "
            f"reduce-scatter {rs_ms:.3f} ms; "
            f"all-gather {ag_ms:.3f} ms; "
            f"torch copy {extra['torch_copy_2x2GiB_hbm_gbps']} GB/s")
        # restore the inputs overwritten by the all-gather above
        for r in range(n):
            sends[r].copy_(torch.from_numpy(xs[r]).to(dev))
    if args.copy_probe:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)      # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None if args.no_cpu_baseline else cpu_baseline_headline(xs, s_bytes)

    traffic = measured_traffic(default_algo)
    out = {
        "metric": METRIC,
        "value": round(algbw, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "ring AllReduce, 8 virtual ranks x 2^26 float32 (256 MiB each), sum, "
                               + ("the library's default algorithm" if args.algo == "auto"
                                  else f"algorithm {args.algo}"),
                   "nranks": n, "count": count, "op": "sum",
                   "algo": f"auto ({default_algo})" if args.algo == "auto" else args.algo,
                   "inputs": "N(0,1), seed 1"},
        "algbw_gbps": round(algbw, 2),
        "busbw_gbps": round(busbw, 2),
        "hbm_gbps": round(hbm_gbps, 1),
        "hbm_frac_of_peak": round(hbm_gbps / HBM_PEAK_GBPS, 4),
        "roofline": {"bound": "hbm", "achieved": round(hbm_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(hbm_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                     "kernel": kernel_name, "launches_per_call": launches["timed"],
                     "algorithmic_bytes_per_call": algo_bytes},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
