#!/usr/bin/env python3
"""Benchmark of the fused decode-time hidden-state projection on one MI355X.

Workload (the pages' headline op): DeepSeek-V4.1 wq_a (5120 -> 1280) fused
with wkv (5120 -> 512), bf16 in/out with fp32 accumulation, one fused call
per token count M = 1..8 ("tinygemm2 for the DeepSeek-V4.1 hidden-state
projections", TensorRT-LLM PR #20636, Description: op-level timing under
CUDA-graph replay with the weights rotated past the cache).

Protocol.  A pool of independent concatenated-weight copies of at least
1 GiB (four times the 256 MiB Infinity Cache) is built, one plan each;
consecutive calls use consecutive copies, so every call streams its weights
from HBM.  One hipGraph per M holds one fused call per copy; a step replays
the eight graphs (M = 1..8).  W warm-up steps, then K timed steps between
HIP events on the launch stream, bracketed by device synchronizations.

Reported: ``value`` = algorithmic bytes (W_cat + x + y per call, summed over
the step) / step time, in GB/s; ``roofline`` for the dominant kernel (the
kernel instantiation with the most time in the step): its algorithmic bytes
per launch over its average launch duration -- the back-to-back average of
the committed rocprofv3 kernel trace when that record matches the current
kernel sources, with the HIP-event average over the timed region (on the
launch stream) beside it -- against the 8 TB/s HBM peak, with the HBM
traffic per launch from the rocprofv3 counters of the same record;
per-M microseconds per call for the fused and the one-launch-per-projection
path; ``cpu_baseline`` = the CPU oracle (one thread and OpenMP over the host
cores, median of 5 runs) on a bounded sample of the same M sweep over one
copy.

Table modes (each writes PREFIX.json and PREFIX.md and exits):
``--crossover`` times every kernel path that serves each M on a rotated
pool (``--crossover-workload``: the headline weights, the three-way fused-A
shape, the pages' 2624-row fused-A shape or the dense-MLP down projection
[6144, 768]); ``--ceiling`` the streaming
ceiling against the launch shape and the per-launch floor;
``--indexer-splits`` the fp32 indexer fusion with its K split across
workgroups; ``--pool-sweep`` the per-call time against the pool size.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("µs/call and HBM GB/s (% of peak), fused skinny GEMM M=1..8, "
          "weights past MALL")
HBM_PEAK_GBS = 8000.0
MALL_BYTES = 256 << 20
K = 5120
N = (1280, 512)
MS = (1, 2, 3, 4, 5, 6, 7, 8)


def _kernel_sources():
    """The library's HIP sources and headers, in a fixed order (the digest
    that gates recorded counter values)."""
    import glob
    d = os.path.join(ROOT, "projection_gemm_sparse_amd", "csrc")
    files = sorted(glob.glob(os.path.join(d, "*.hip")) + glob.glob(os.path.join(d, "*.hpp")) +
                   glob.glob(os.path.join(d, "*.h")))
    return tuple(os.path.relpath(f, ROOT) for f in files)


KERNEL_SOURCES = _kernel_sources()
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_sources_digest() -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def recorded_kernel(kernel: str):
    """The committed rocprofv3 record of `kernel` (its kernel-trace average
    duration and HBM bytes per launch), or None when there is none or the
    kernel sources changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sources_sha256_16") != kernel_sources_digest():
        return None
    return rec.get("kernels", {}).get(kernel)


def recorded_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter record,
    or None when there is none or the kernel sources changed since."""
    ent = recorded_kernel(kernel)
    return None if ent is None else ent.get("hbm_bytes_per_launch")


def kernel_name(P, M: int, tiling) -> str:
    """The kernel instantiation a (resolved) tiling runs, as rocprofv3 names it."""
    path, kparts, chunks, splits, rows, groups = tiling
    if path in (P.FP_PATH_SKINNY, P.FP_PATH_SKINNY_SPLITK):
        mt = 1 if M <= 1 else 2 if M <= 2 else 4 if M <= 4 else 8
        return "fp::skinny_kernel<%d, %d, %d, true, 0>" % (mt, rows, chunks)
    if path == P.FP_PATH_MFMA_SMALL:
        # token halves; with two, up to 12 tokens the interleaved load order;
        # row tiles per wave (rows above 8: two tiles of rows / 2)
        return "fp::smfma_kernel<%d, false, %d, %s, %d>" % (
            chunks, 1 if M <= 8 else 2 if M <= 16 else 3, "false" if 8 < M <= 12 else "true",
            2 if rows > 8 else 1)
    mt16 = next(b for b in (1, 2, 4, 8, 16) if 16 * b >= M)
    cs = 4 if chunks in (8, 16) else 5
    return "fp::tile_kernel<%d, %d, %d, %d>" % (mt16, kparts, cs, chunks // cs)


def algorithmic_bytes(M: int, K: int, N, esize: int = 2) -> int:
    n_total = sum(N)
    return esize * (n_total * K + M * K + M * n_total)


def build_pool(P, torch, n_copies, max_M, seed=0, shape=None, workspace_bytes=None):
    """n_copies independent weight sets U(-1/sqrt(K), 1/sqrt(K)) -> bf16,
    drawn on the GPU, each concatenated by its own plan (shape: (K, N),
    default the headline's; workspace_bytes: each plan's split-K workspace,
    default what its default tilings need)."""
    k, ns = shape if shape is not None else (K, N)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    a = 1.0 / math.sqrt(k)
    plans = []
    for _ in range(n_copies):
        ws = [((torch.rand(n, k, generator=g, device="cuda") * 2 - 1) * a)
              .to(torch.bfloat16) for n in ns]
        plans.append(P.FusedProjection(ws, max_M=max_M, workspace_bytes=workspace_bytes))
        del ws
    return plans


def capture(torch, fn):
    fn()  # eager warm-up outside capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_graphs(torch, graphs, steps, warmup):
    """Replays the graphs in order per step; returns (total_ms, per-graph ms
    summed over the timed steps)."""
    for _ in range(warmup):
        for g in graphs:
            g.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(graphs) + 1)]
    per = [0.0] * len(graphs)
    total = 0.0
    for _ in range(steps):
        evs[0].record(stream)
        for i, g in enumerate(graphs):
            g.replay()
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        for i in range(len(graphs)):
            per[i] += evs[i].elapsed_time(evs[i + 1])
        total += evs[0].elapsed_time(evs[-1])
    return total, per


def cpu_baseline(plan0_weights_cpu, xs_cpu, run_s=2.0, runs=5):
    """The oracle (plain C loop, fp64) on the M = 1..8 sweep over one weight
    copy, in two forms: single-threaded, and with the output elements spread
    over all host threads (OpenMP, the same per-element loop).  Each form:
    `runs` runs of repeated sweeps of at least `run_s` seconds each; the
    median run gives the seconds per sweep."""
    import oracle
    import synthetic_inputs as si
    oracle.build(force=False)
    wb = [si.bits(w) for w in plan0_weights_cpu]
    xb = {M: si.bits(xs_cpu[M]) for M in MS}
    sweep_bytes = sum(algorithmic_bytes(M, K, N) for M in MS)
    variants = {}
    for name, lin, cores in (("single_thread", oracle.linear, 1),
                             ("openmp", oracle.linear_omp, oracle.omp_threads())):
        per = []
        for _ in range(runs):
            n, t0 = 0, time.perf_counter()
            while True:
                for M in MS:
                    for w in wb:
                        lin(xb[M], w)
                n += 1
                el = time.perf_counter() - t0
                if el >= run_s:
                    break
            per.append(el / n)
        per.sort()
        med = per[len(per) // 2]
        variants[name] = {"value": round(sweep_bytes / med / 1e9, 4), "unit": "GB/s",
                          "cores": cores, "sweep_s_median": round(med, 5),
                          "sweep_s_runs": [round(v, 5) for v in per],
                          "us_per_call": round(med / len(MS) * 1e6, 1)}
    omp = variants["openmp"]
    return {"value": omp["value"], "unit": "GB/s", "cores": omp["cores"], "kind": "oracle",
            "host": host_info(),
            "sample": "the M=1..8 sweep (16 projection calls) over one [1792, 5120] bf16 weight "
                      "copy; median of %d runs of >= %.0f s each; C fp64 loop (gcc -O2, no "
                      "fast-math), output elements over %d OpenMP threads; the single-threaded "
                      "form in single_thread" % (runs, run_s, omp["cores"]),
            "us_per_call": omp["us_per_call"], "single_thread": variants["single_thread"]}


def stream_ceiling(P, torch, dev, plans, n_copies, steps):
    """The read-only streaming ceiling on the same pool: fp_stream_read
    over every copy's W_cat (the weight bytes, the fused call's launch
    shape, nothing else), one call per copy, hipGraph replay."""
    sink = torch.zeros(256, dtype=torch.int32, device=dev)
    wb = plans[0].n_total * K * 2
    ptrs = [p.views[0].data_ptr() for p in plans]

    def calls():
        h = torch.cuda.current_stream().cuda_stream
        for ptr in ptrs:
            st = P.fp_stream_read(ptr, wb, sink.data_ptr(), h)
            if st != P.FP_OK:
                raise RuntimeError("fp_stream_read: %d" % st)
    g = capture(torch, calls)
    t, _ = time_graphs(torch, [g], steps, 2)
    us = t * 1e3 / (steps * n_copies)
    return {"us_per_call": round(us, 4), "GBps": round(wb / us / 1e3, 1),
            "frac_of_peak": round(wb / us / 1e3 / HBM_PEAK_GBS, 4), "bytes": wb,
            "note": "fp_stream_read of each copy's W_cat (18,350,080 B) with the fused "
                    "call's launch shape and no other work; same pool and protocol"}


def command_line() -> str:
    """The command that produced a table, for its summary."""
    return "python -u bench.py " + " ".join(sys.argv[1:])


def write_table_md(path, title, header, rows, notes=()):
    """A markdown summary: title, the producing command, notes, one table."""
    lines = ["# " + title, "", "Command (run from the repository root):", "", "```",
             command_line(), "```", ""]
    for n in notes:
        lines += [n, ""]
    lines.append("| " + " | ".join(header) + " |")
    lines.append("|" + "---|" * len(header))
    for r in rows:
        lines.append("| " + " | ".join("" if c is None else str(c) for c in r) + " |")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")


def write_outputs(prefix, title, payload, header, rows, notes=()):
    with open(prefix + ".json", "w") as fh:
        json.dump(payload, fh, indent=1)
    write_table_md(prefix + ".md", title, header, rows, notes)
    print("bench: wrote %s.json and %s.md" % (prefix, prefix), file=sys.stderr, flush=True)


# Launch shapes of the streaming-ceiling sweep: (workgroups, threads,
# loads in flight per lane); the first is the fused call's shape.
STREAM_SHAPES = ((256, 640, 8), (256, 256, 32), (256, 512, 16), (256, 1024, 8), (512, 512, 8),
                 (1024, 256, 8), (2048, 128, 8), (4096, 64, 8), (224, 640, 8), (128, 640, 16),
                 (256, 256, 8))


def ceiling_sweep(P, torch, dev, plans, n_copies, steps, prefix):
    """The read-only streaming ceiling against the launch shape, and where a
    fused call's time goes: the per-launch floor (a graph of tiny kernels,
    and a launch of the fused call's shape that reads one vector), the
    stream of the weights, and the fused calls (M = 1, 8) on the same pool
    and protocol."""
    import synthetic_inputs as si
    sink = torch.zeros(65536, dtype=torch.int32, device=dev)
    wb = plans[0].n_total * K * 2
    ptrs = [p.views[0].data_ptr() for p in plans]

    def per_call(fn):
        g = capture(torch, fn)
        t, _ = time_graphs(torch, [g], steps, 2)
        del g
        return t * 1e3 / (steps * n_copies)

    def shaped(groups, threads, batch, nbytes):
        def calls():
            h = torch.cuda.current_stream().cuda_stream
            for ptr in ptrs:
                st = P.fp_stream_read_shaped(ptr, nbytes, groups, threads, batch,
                                             sink.data_ptr(), h)
                if st != P.FP_OK:
                    raise RuntimeError("fp_stream_read_shaped: %d" % st)
        return per_call(calls)

    tiny = torch.zeros(64, device=dev)
    floor_tiny = per_call(lambda: [tiny.add_(1.0) for _ in range(n_copies)])
    floor_shape = shaped(256, 640, 8, 16)
    rows, shapes = [], []
    for groups, threads, batch in STREAM_SHAPES:
        us = shaped(groups, threads, batch, wb)
        shapes.append({"groups": groups, "threads": threads, "batch": batch,
                       "us": round(us, 4), "GBps": round(wb / us / 1e3, 1)})
        rows.append(("%d x %d" % (groups, threads), batch,
                     -(-wb // 16 // groups // threads), "%.3f" % us, "%.0f" % (wb / us / 1e3),
                     "%.1f" % (100 * wb / us / 1e3 / HBM_PEAK_GBS)))
        print("bench: stream shape %s" % json.dumps(shapes[-1]), file=sys.stderr, flush=True)
    fused = {}
    for M in (1, 8):
        x = si.make_case(K, N, "bf16", M, seed=100 + M)[0].to(dev)
        out = [torch.empty(M, n, dtype=torch.bfloat16, device=dev) for n in N]
        fused[M] = per_call(lambda: [p.forward(x, out=out) for p in plans])
    ceil_us = shapes[0]["us"]
    decomp = [("graph of tiny kernels (per launch)", "%.3f" % floor_tiny, "", ""),
              ("fused-call launch shape reading one vector", "%.3f" % floor_shape, "", ""),
              ("stream of the weights, fused-call shape", "%.3f" % ceil_us,
               "%.3f" % (ceil_us - floor_shape), ""),
              ("fused call, M = 1", "%.3f" % fused[1], "%.3f" % (fused[1] - floor_shape),
               "%.3f" % (fused[1] - ceil_us)),
              ("fused call, M = 8", "%.3f" % fused[8], "%.3f" % (fused[8] - floor_shape),
               "%.3f" % (fused[8] - ceil_us))]
    payload = {"workload": "wq_a+wkv [1280,512]x5120 bf16, %d copies rotated" % n_copies,
               "weight_bytes": wb, "floor_tiny_us": round(floor_tiny, 4),
               "floor_fused_shape_us": round(floor_shape, 4), "shapes": shapes,
               "fused_us": {str(k): round(v, 4) for k, v in fused.items()}}
    notes = ["Every row: one call per weight copy (%d copies of %d bytes, %.0f MiB, past the "
             "256 MiB MALL), captured in a hipGraph, %d timed replays; microseconds per call."
             % (n_copies, wb, n_copies * wb / 2 ** 20, steps),
             "Where a call's time goes (us per call; 'above launch' subtracts the fused-call "
             "launch shape reading one vector, 'above ceiling' the stream of the same bytes):",
             "\n".join(["| part | us | above launch | above ceiling |", "|---|---|---|---|"] +
                       ["| %s |" % " | ".join(r) for r in decomp]),
             "Streaming ceiling against the launch shape (fp_stream_read_shaped: workgroup b "
             "reads the b-th contiguous 1/groups of the copy, 16-byte non-temporal loads):"]
    write_outputs(prefix, "Streaming ceiling and per-launch floor, wq_a+wkv [1792, 5120] bf16 "
                  "weights rotated past the MALL", payload,
                  ["workgroups x threads", "loads in flight / lane", "loads / lane", "us / call",
                   "GB/s", "% of 8 TB/s"], rows, notes)
    return payload


# Forced K splits of the fp32 indexer fusion: (name, tiling) with tiling
# (path, waves per slice P, chunks per lane CJ, slices S, rows, groups).
INDEXER_SPLITS = (("S=1 (P=14, CJ=2)", None), ("S=2 (P=14, CJ=1)", (2, 14, 1, 2, 0, 0)),
                  ("S=2 (P=7, CJ=2)", (2, 7, 2, 2, 0, 0)), ("S=4 (P=7, CJ=1)", (2, 7, 1, 4, 0, 0)),
                  ("S=7 (P=2, CJ=2)", (2, 2, 2, 7, 0, 0)), ("S=7 (P=4, CJ=1)", (2, 4, 1, 7, 0, 0)),
                  ("S=14 (P=2, CJ=1)", (2, 2, 1, 14, 0, 0)))


def indexer_split_sweep(P, torch, dev, steps, prefix, Ms=(1, 4, 8)):
    """The fp32 indexer fusion (K = 7168, [128, 64], fp32) with its K split
    across 1..14 workgroups per row block, on a pool past the MALL: the
    measurement its default split is chosen from."""
    import synthetic_inputs as si
    wl = si.WORKLOADS["indexer_f32"]
    wb = sum(wl.N) * wl.K * 4
    n = max(2, math.ceil((1 << 30) / wb))
    g = torch.Generator(device="cuda")
    g.manual_seed(17)
    plans = []
    for _ in range(n):
        ws = [(torch.randn(nr, wl.K, generator=g, device="cuda") * 0.02) for nr in wl.N]
        plans.append(P.FusedProjection(ws, max_M=max(Ms), workspace_bytes=1 << 20))
        del ws
    res, rows = [], []
    for M in Ms:
        x = si.make_case(wl.K, wl.N, wl.dtype, M, seed=700 + M)[0].to(dev)
        out = [torch.empty(M, nr, dtype=torch.float32, device=dev) for nr in wl.N]
        for name, t in INDEXER_SPLITS:
            for p in plans:
                p.set_tiling(M, None)
            if t is not None:
                st = plans[0].set_tiling(M, t)
                if st != P.FP_OK:
                    res.append({"M": M, "split": name, "status": st})
                    continue
                for p in plans[1:]:
                    p.set_tiling(M, t)
            gr = capture(torch, lambda: [p.forward(x, out=out) for p in plans])
            tt, _ = time_graphs(torch, [gr], steps, 2)
            del gr
            us = tt * 1e3 / (steps * n)
            tl = list(plans[0].get_tiling(M))
            wgs = -(-sum(wl.N) // (tl[4] * tl[5])) * tl[3]
            b = 4 * (sum(wl.N) * wl.K + M * wl.K + M * sum(wl.N))
            res.append({"M": M, "split": name, "tiling": tl, "workgroups": wgs,
                        "us": round(us, 4), "GBps": round(b / us / 1e3, 1)})
            rows.append((M, name, tl, wgs, "%.3f" % us, "%.0f" % (b / us / 1e3)))
            print("bench: indexer split %s" % json.dumps(res[-1]), file=sys.stderr, flush=True)
    for p in plans:
        p.close()
    write_outputs(prefix, "fp32 indexer fusion [192, 7168] (wk 128 + weights_proj 64): K split "
                  "across workgroups", {"workload": "indexer_f32 K=7168 N=[128, 64] fp32, %d "
                                        "copies rotated" % n, "rows": res},
                  ["M", "split", "tiling (path, P, CJ, S, RW, G)", "workgroups", "us / call",
                   "GB/s"], rows,
                  ["One fused call per weight copy (%d copies of %d bytes, past the MALL), "
                   "hipGraph replay, %d timed replays; the split is forced with "
                   "fp_plan_set_tiling (S=1 is the default)." % (n, wb, steps)])
    return res


def trial_stats(torch, graphs, n_calls, trials=15, min_calls=2000):
    """Per graph: median, p10 and p90 of the per-call time over `trials`
    trials of R replays each (R * n_calls >= min_calls)."""
    reps = max(1, -(-min_calls // n_calls))
    out = []
    for g in graphs:
        vals = []
        for _ in range(trials):
            _, per = time_graphs(torch, [g], reps, 0)
            vals.append(per[0] * 1e3 / (reps * n_calls))
        vals.sort()
        q = lambda f: vals[min(len(vals) - 1, max(0, round(f * (len(vals) - 1))))]
        out.append({"median": round(q(0.5), 4), "p10": round(q(0.1), 4),
                    "p90": round(q(0.9), 4)})
    return out, reps


def eager_us(torch, fn, n_calls, reps=3):
    """Per-call time of eager (not captured) calls from Python: `fn` makes
    n_calls calls; best of `reps` runs, bracketed by synchronisations."""
    best = float("inf")
    fn()
    torch.cuda.synchronize()
    for _ in range(reps):
        t0 = time.perf_counter()
        fn()
        torch.cuda.synchronize()
        best = min(best, time.perf_counter() - t0)
    return round(best * 1e6 / n_calls, 4)


def workload_cells(P, torch, dev, steps, name):
    """The other workloads of the projection on their own pools past the
    MALL, fused and one launch per projection: the fp32 indexer fusion
    (K = 7168, [128, 64], fp32 in and out, M = 1, 4, 8) and the three-way
    fused-A shape (K = 6144, [2048, 576, 128], bf16, M = 1..8)."""
    import synthetic_inputs as si
    wl = si.WORKLOADS[name]
    esize = 4 if wl.dtype == "f32" else 2
    dt = torch.float32 if esize == 4 else torch.bfloat16
    wb = sum(wl.N) * wl.K * esize
    n = max(2, math.ceil((1 << 30) / wb))
    Ms = (1, 4, 8) if esize == 4 else tuple(range(1, 9))
    g = torch.Generator(device="cuda")
    g.manual_seed(17)
    plans = []
    for _ in range(n):
        if esize == 4:
            ws = [(torch.randn(nr, wl.K, generator=g, device="cuda") * 0.02) for nr in wl.N]
        else:
            a = 1.0 / math.sqrt(wl.K)
            ws = [((torch.rand(nr, wl.K, generator=g, device="cuda") * 2 - 1) * a).to(dt)
                  for nr in wl.N]
        plans.append(P.FusedProjection(ws, max_M=max(Ms)))
        del ws
    res = {}
    for M in Ms:
        x = si.make_case(wl.K, wl.N, wl.dtype, M, seed=700 + M)[0].to(dev)
        out = [torch.empty(M, nr, dtype=dt, device=dev) for nr in wl.N]
        gf = capture(torch, lambda: [p.forward(x, out=out) for p in plans])
        gs = capture(torch, lambda: [p.forward_separate(x, out=out) for p in plans])
        _, per = time_graphs(torch, [gf, gs], steps, 2)
        uf = per[0] * 1e3 / (steps * n)
        us_ = per[1] * 1e3 / (steps * n)
        b = esize * (sum(wl.N) * wl.K + M * wl.K + M * sum(wl.N))
        res[str(M)] = {"fused_us": round(uf, 4), "separate_us": round(us_, 4),
                       "GBps": round(b / uf / 1e3, 1),
                       "frac_of_peak": round(b / uf / 1e3 / HBM_PEAK_GBS, 4), "bytes": b,
                       "path": P._lib.PATH_NAMES[plans[0].query(M)[0]],
                       "tiling": list(plans[0].get_tiling(M))}
        del gf, gs
    for p in plans:
        p.close()
    res["note"] = ("%s: K=%d N=%s %s, %d copies rotated (>= 1 GiB), one call per copy, "
                   "hipGraph replay" % (name, wl.K, list(wl.N), wl.dtype, n))
    return res


def pool_sweep(P, torch, dev, steps, Ms=(1, 8)):
    """Per-call time of the fused call against the size of the rotated pool
    (one copy, then 64 MiB .. 2 GiB): the time must level off once the pool
    is well past the 256 MiB MALL."""
    import synthetic_inputs as si
    w_bytes = sum(N) * K * 2
    rows = []
    for mib in (0, 64, 128, 256, 512, 1024, 2048):
        n = max(1, math.ceil((mib << 20) / w_bytes)) if mib else 1
        plans = build_pool(P, torch, n, max(Ms))
        for M in Ms:
            x = si.make_case(K, N, "bf16", M, seed=100 + M)[0].to(dev)
            out = [torch.empty(M, nn, dtype=torch.bfloat16, device=dev) for nn in N]
            reps = max(1, 400 // n)
            gr = capture(torch, lambda: [p.forward(x, out=out) for p in plans * reps])
            t, _ = time_graphs(torch, [gr], steps, 2)
            us = t * 1e3 / (steps * n * reps)
            rows.append({"pool_MiB": round(n * w_bytes / 2**20, 1), "copies": n, "M": M,
                         "us": round(us, 4),
                         "GBps": round(algorithmic_bytes(M, K, N) / us / 1e3, 1)})
            print("bench: pool sweep %s" % json.dumps(rows[-1]), file=sys.stderr, flush=True)
            del gr
        for p in plans:
            p.close()
        del plans
        torch.cuda.empty_cache()
    return rows


def host_info():
    """CPU model name and logical CPU count of the host."""
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count()}


# Workloads of the crossover tables: (title, K, N, token counts, small-M
# row layouts forced besides the library's: (label, rows, groups) -- rows
# above 8 are two row tiles of rows / 2 per wave --, K slice counts of the
# ring tile kernel).
_SMALL_ROWS = (("one tile of 6 rows", 6, 1), ("one tile of 8 rows", 8, 1),
               ("two tiles of 6 rows", 12, 1), ("two tiles of 8 rows", 16, 1))
CROSSOVER_SHAPES = {
    "wq_a+wkv": ("wq_a+wkv [1792, 5120] bf16", 5120, (1280, 512),
                 (1, 2, 3, 4, 5, 8, 9, 12, 16, 17, 24, 32, 48, 64, 96, 128), (), (9,)),
    "fused_a_3way": ("three-way fused-A [2752, 6144] bf16", 6144, (2048, 576, 128),
                     tuple(range(1, 17)) + (17, 32, 48, 64, 96, 128), _SMALL_ROWS,
                     (5, 7, 9, 11)),
    "glm_fused_a": ("fused-A of the pages [2624, 6144] bf16 (2048 + 512 + 64)", 6144,
                    (2048, 512, 64), tuple(range(1, 17)) + (17, 32, 48, 64), _SMALL_ROWS,
                    (9, 12)),
    # the dense-MLP down projection of the pages' small-M MLP (one projection,
    # K = 768): row layouts of three K parts
    "mlp_down": ("dense-MLP down projection [6144, 768] bf16", 768, (6144,),
                 (1, 2, 3, 4, 5, 8, 9, 12, 16), _SMALL_ROWS + (
                     ("three groups of one 8-row tile", 8, 3),
                     ("two groups of two tiles of 6 rows", 12, 2)), (9,)),
}


def crossover(prefix, P, torch, dev, workload="wq_a+wkv", pool_mib=1024):
    """Per token count, every kernel path that serves it, on a rotated pool
    of the workload's weights past the MALL: the measured crossovers that
    place each kernel."""
    import synthetic_inputs as si
    title, k, ns, Ms, small_rows, ring_slices = CROSSOVER_SHAPES[workload]
    n_copies = max(2, math.ceil((pool_mib << 20) / (sum(ns) * k * 2)))
    # room for the partials of every forced slice count
    ws_bytes = (64 << 10) + max(ring_slices + (9,)) * sum(ns) * 16 * (-(-max(Ms) // 16)) * 4
    big = build_pool(P, torch, n_copies, max(Ms), shape=(k, ns), workspace_bytes=ws_bytes)
    kc = k * 2 // 16
    steps = -(-kc // 8)
    kt = 4 if steps <= 64 else 8 if steps <= 128 else 16
    pk = -(-steps // kt)
    res, rows = [], []
    for M in Ms:
        xc, _ = si.make_case(k, ns, "bf16", M, seed=200 + M)
        x = xc.to(dev)
        out = [torch.empty(M, n, dtype=torch.bfloat16, device=dev) for n in ns]
        cands = [("default", None)]
        if M <= 8:
            cands.append(("vector ALU", (P.FP_PATH_SKINNY, min(16, -(-kc // 64)), 1, 1, 0, 0)))
        if M <= 24:
            cands.append(("small-M MFMA", (P.FP_PATH_MFMA_SMALL, pk, kt, 1, 0, 0)))
            for label, r, g in small_rows:
                cands.append(("small-M MFMA, " + label, (P.FP_PATH_MFMA_SMALL, pk, kt, 1, r, g)))
        if M > 8:
            cands.append(("tile (S=8)", (P.FP_PATH_MFMA, 0, 0, 8, 0, 0)))
            for rs in ring_slices:
                cands.append(("ring tile (S=%d)" % rs,
                              (P.FP_PATH_MFMA, 4, 3 if M > 128 else 4, rs, 0, 0)))
            cands.append(("weight-resident (S=8)", (P.FP_PATH_MFMA, 4, 2, 8, 0, 0)))
            cands.append(("weight-resident (S=9)", (P.FP_PATH_MFMA, 4, 2, 9, 0, 0)))
        default_t = list(big[0].get_tiling(M))
        for name, t in cands:
            if t is not None:
                if any(p.set_tiling(M, t) for p in big):
                    for p in big:
                        p.set_tiling(M, None)
                    continue
                if name != "default" and list(big[0].get_tiling(M)) == default_t:
                    name += " = default"
            g = capture(torch, lambda: [p.forward(x, out=out) for p in big])
            ms, _ = time_graphs(torch, [g], 10, 2)
            us = ms * 1e3 / (10 * n_copies)
            b = algorithmic_bytes(M, k, ns)
            tl = list(big[0].get_tiling(M))
            res.append({"M": M, "variant": name, "path": P._lib.PATH_NAMES[big[0].query(M)[0]],
                        "tiling": tl, "us": round(us, 3), "GBps": round(b / us / 1e3, 1)})
            rows.append((M, name, tl, "%.3f" % us, "%.0f" % (b / us / 1e3),
                         "%.1f" % (100 * b / us / 1e3 / HBM_PEAK_GBS)))
            print("bench: crossover %s" % json.dumps(res[-1]), file=sys.stderr, flush=True)
            for p in big:
                p.set_tiling(M, None)
            del g
    for p in big:
        p.close()
    write_outputs(prefix, "Kernel crossover, %s, weights rotated past the MALL" % title,
                  {"workload": "%s, %d rotated copies" % (title, n_copies), "rows": res},
                  ["M", "kernel", "tiling (path, kparts, chunks, S, rows, groups)", "us / call",
                   "GB/s", "% of 8 TB/s"], rows,
                  ["Every kernel that serves M, forced with fp_plan_set_tiling, on one pool "
                   "of %d copies (one fused call per copy, hipGraph replay, 10 timed replays); "
                   "'default' is the library's choice.  Small-M rows: rows per row group "
                   "(above 8: two row tiles of rows / 2 per wave sharing the activation "
                   "operand); 0 = chosen per launch." % n_copies])


def epilogue_cells(P, torch, dev, plans, n_copies, steps, Ms=(1, 2, 4, 8)):
    """The fused epilogues on rotated pools, next to their unfused chains.

    RMSNorm (q_norm / kv_norm over the wq_a / wkv outputs) on the main pool:
    fused (the fused projection, then one normalisation launch for both
    projections) vs the unfused chain (one projection launch per projection,
    then one RMSNorm launch per projection).  SwiGLU on a pool of gate/up
    weights [2 x 768, 6144] (past the MALL as well): fused (one launch over
    gate/up row pairs) vs gate and up launches followed by the SwiGLU
    launch."""
    L = P._lib
    eps = 1e-6
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    gammas = [(1.0 + 0.1 * torch.randn(n, generator=g, device="cuda")).to(torch.bfloat16)
              for n in N]
    res = {"rmsnorm": {}, "swiglu": {}}
    for M in Ms:
        xc, _ = __import__("synthetic_inputs").make_case(K, N, "bf16", M, seed=300 + M)
        x = xc.to(dev)
        outs = [torch.empty(M, n, dtype=torch.bfloat16, device=dev) for n in N]

        def fused():
            for p in plans:
                p.forward_rmsnorm(x, gammas, eps, out=outs)

        def chain():
            s = torch.cuda.current_stream().cuda_stream
            for p in plans:
                p.forward_separate(x, out=outs)
                for i, n in enumerate(N):
                    L.check(L.fp_rmsnorm(outs[i].data_ptr(), M, n, gammas[i].data_ptr(), eps,
                                         outs[i].data_ptr(), s), "fp_rmsnorm")
        gf, gc = capture(torch, fused), capture(torch, chain)
        (tf, _), (tc, _) = time_graphs(torch, [gf], steps, 2), time_graphs(torch, [gc], steps, 2)
        b = algorithmic_bytes(M, K, N) + 2 * sum(N)
        uf, uc = tf * 1e3 / (steps * n_copies), tc * 1e3 / (steps * n_copies)
        res["rmsnorm"][str(M)] = {"fused_us": round(uf, 4), "unfused_us": round(uc, 4),
                                  "fused_launches": 2, "unfused_launches": 2 * len(N),
                                  "fused_GBps": round(b / uf / 1e3, 1), "bytes": b}
        del gf, gc
    # gate/up pool
    Kg, Ng = 6144, (768, 768)
    wb = sum(Ng) * Kg * 2
    ng = max(2, math.ceil((1 << 30) / wb))
    a = 1.0 / math.sqrt(Kg)
    gplans = []
    for _ in range(ng):
        ws = [((torch.rand(n, Kg, generator=g, device="cuda") * 2 - 1) * a).to(torch.bfloat16)
              for n in Ng]
        gplans.append(P.FusedProjection(ws, max_M=8))
        del ws
    for M in Ms:
        xc, _ = __import__("synthetic_inputs").make_case(Kg, Ng, "bf16", M, seed=400 + M)
        x = xc.to(dev)
        h = torch.empty(M, Ng[0], dtype=torch.bfloat16, device=dev)
        gu = [torch.empty(M, n, dtype=torch.bfloat16, device=dev) for n in Ng]

        def fused():
            for p in gplans:
                p.forward_swiglu(x, out=h)

        def chain():
            s = torch.cuda.current_stream().cuda_stream
            for p in gplans:
                p.forward_separate(x, out=gu)
                L.check(L.fp_swiglu(gu[0].data_ptr(), gu[1].data_ptr(), M, Ng[0], h.data_ptr(),
                                    s), "fp_swiglu")
        gf, gc = capture(torch, fused), capture(torch, chain)
        (tf, _), (tc, _) = time_graphs(torch, [gf], steps, 2), time_graphs(torch, [gc], steps, 2)
        b = 2 * (sum(Ng) * Kg + M * Kg + M * Ng[0])
        uf, uc = tf * 1e3 / (steps * ng), tc * 1e3 / (steps * ng)
        res["swiglu"][str(M)] = {"fused_us": round(uf, 4), "unfused_us": round(uc, 4),
                                 "fused_launches": 1, "unfused_launches": 3,
                                 "fused_GBps": round(b / uf / 1e3, 1), "bytes": b}
        del gf, gc
    for p in gplans:
        p.close()
    res["note"] = ("us per call on pools rotated past the MALL (rmsnorm: %d wq_a+wkv copies; "
                   "swiglu: %d gate/up [2x768, 6144] copies); unfused = one projection launch "
                   "per projection, then the standalone epilogue launch(es)" % (n_copies, ng))
    return res


def router_cells(P, torch, dev, steps, Ms=(1, 4, 8, 16)):
    """The fp32-output router GEMV (256 expert logits at hidden 6144, bf16
    operands) on a pool of weight copies rotated past the MALL."""
    import synthetic_inputs as si
    Kr, Nr = 6144, (256,)
    wb = Nr[0] * Kr * 2
    n = max(2, math.ceil((1 << 30) / wb))
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    a = 1.0 / math.sqrt(Kr)
    plans = [P.FusedProjection([((torch.rand(Nr[0], Kr, generator=g, device="cuda") * 2 - 1) * a)
                                .to(torch.bfloat16)], max_M=16, out_dtype=torch.float32)
             for _ in range(n)]
    res = {}
    for M in Ms:
        x = si.make_case(Kr, Nr, "bf16", M, seed=500 + M)[0].to(dev)
        out = [torch.empty(M, Nr[0], dtype=torch.float32, device=dev)]
        gr = capture(torch, lambda: [p.forward(x, out=out) for p in plans])
        t, _ = time_graphs(torch, [gr], steps, 2)
        us = t * 1e3 / (steps * n)
        b = wb + M * Kr * 2 + M * Nr[0] * 4
        res[str(M)] = {"us": round(us, 4), "GBps": round(b / us / 1e3, 1), "bytes": b,
                       "tiling": list(plans[0].get_tiling(M))}
        del gr
    for p in plans:
        p.close()
    res["note"] = ("fp32 logits of a [256, 6144] bf16 router weight, %d copies rotated "
                   "(1 GiB), one call per copy, hipGraph replay" % n)
    return res


def mxfp8_cells(P, torch, dev, steps, Ms=(1, 2, 4, 8), fmt="mxfp8", variants=False):
    """The wq_a + wkv projection with MX weights, bf16 x and y, on a pool of
    weight copies rotated past the MALL.  mxfp8: E4M3 codes, one E8M0 scale
    per 32 elements, packed rows of K + K/32 bytes; mxfp4: E2M1 codes two per
    byte, rows of K/2 + K/32 bytes; nvfp4: E2M1 codes two per byte, one E4M3
    scale per 16 elements and an fp32 tensor scale per projection, rows of
    K/2 + K/16 bytes.  variants: also time the vector-ALU and the small-M
    matrix-core kernels at every M (crossover runs)."""
    import synthetic_inputs as si
    row = {"mxfp8": K + K // 32, "mxfp4": K // 2 + K // 32, "nvfp4": K // 2 + K // 16}[fmt]
    wb = sum(N) * row
    n = max(2, math.ceil((1 << 30) / wb))
    g = torch.Generator(device="cuda")
    g.manual_seed(13)
    plans = []
    for _ in range(n):
        ws = []
        for nr in N:
            if fmt == "mxfp8":
                codes = torch.randint(0, 254, (nr, K), generator=g, device="cuda")
                codes = codes + (codes >= 0x7F).to(codes.dtype)
                sc = torch.randint(112, 118, (nr, K // 32), generator=g, device="cuda")
            elif fmt == "mxfp4":
                codes = torch.randint(0, 256, (nr, K // 2), generator=g, device="cuda")
                sc = torch.randint(116, 122, (nr, K // 32), generator=g, device="cuda")
            else:
                codes = torch.randint(0, 256, (nr, K // 2), generator=g, device="cuda")
                sc = torch.randint(0x28, 0x41, (nr, K // 16), generator=g, device="cuda")
            ws.append(torch.cat([codes, sc], 1).to(torch.uint8))
        ts = [0.0087890625, 0.0107421875] if fmt == "nvfp4" else None
        plans.append(P.FusedProjection(ws, max_M=16, weight_format=fmt, tensor_scales=ts))
        del ws
    res = {}
    for M in Ms:
        x = si.make_case(K, N, "bf16", M, seed=600 + M)[0].to(dev)
        out = [torch.empty(M, nr, dtype=torch.bfloat16, device=dev) for nr in N]
        gr = capture(torch, lambda: [p.forward(x, out=out) for p in plans])
        t, _ = time_graphs(torch, [gr], steps, 2)
        us = t * 1e3 / (steps * n)
        b = wb + 2 * M * K + 2 * M * sum(N)
        res[str(M)] = {"us": round(us, 4), "GBps": round(b / us / 1e3, 1), "bytes": b,
                       "frac_of_peak": round(b / us / 1e3 / HBM_PEAK_GBS, 4),
                       "tiling": list(plans[0].get_tiling(M))}
        del gr
        if variants:
            steps64 = K // 64
            kt = 4 if steps64 <= 64 else 8 if steps64 <= 128 else 16
            for name, t in (("skinny", (P.FP_PATH_SKINNY, 10, 1, 1, 0, 0)),
                            ("mfma_small", (P.FP_PATH_MFMA_SMALL, -(-steps64 // kt), kt, 1, 0, 0))):
                if any(p.set_tiling(M, t) for p in plans):
                    for p in plans:
                        p.set_tiling(M, None)
                    continue
                gr = capture(torch, lambda: [p.forward(x, out=out) for p in plans])
                t2, _ = time_graphs(torch, [gr], steps, 2)
                res[str(M)][name + "_us"] = round(t2 * 1e3 / (steps * n), 4)
                del gr
                for p in plans:
                    p.set_tiling(M, None)
    for p in plans:
        p.close()
    res["note"] = ("wq_a+wkv [1280,512]x5120 with %s weights (%d bytes per call), %d "
                   "copies rotated (1 GiB), one call per copy, hipGraph replay"
                   % (fmt.upper(), wb, n))
    if fmt == "nvfp4":
        res["note"] += "; fp32 tensor scales %s" % ts
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--pool-mib", type=int, default=1024,
                    help="total size of the rotated weight pool (>= 1024 for past-MALL)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--details", default="", help="write per-M details JSON here")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this size (counter calibration)")
    ap.add_argument("--fused-only", action="store_true",
                    help="skip the one-launch-per-projection timing (profiler runs: every "
                         "dispatch of a kernel is then a fused call)")
    ap.add_argument("--no-epilogues", action="store_true",
                    help="skip the fused RMSNorm / SwiGLU epilogue cells")
    ap.add_argument("--crossover", default="",
                    help="time every kernel path per M in 1..128, write PREFIX.json and "
                         "PREFIX.md and exit")
    ap.add_argument("--crossover-workload", default="wq_a+wkv",
                    choices=sorted(CROSSOVER_SHAPES),
                    help="the weights of the --crossover table")
    ap.add_argument("--ceiling", default="",
                    help="time the streaming ceiling against the launch shape and the "
                         "per-launch floor, write PREFIX.json and PREFIX.md and exit")
    ap.add_argument("--indexer-splits", default="",
                    help="time the fp32 indexer fusion with its K split across 1..14 "
                         "workgroups, write PREFIX.json and PREFIX.md and exit")
    ap.add_argument("--timed-only", action="store_true",
                    help="only the warm-up and timed steps of the fused graphs (profiler runs: "
                         "every dispatch is a graph replay of the timed step)")
    ap.add_argument("--mfma-only", action="store_true",
                    help="time only the matrix-core cells (M = 8..24 on the small-M kernel, "
                         "32..128 on the tile kernels) and print them (profiler runs of the "
                         "MFMA and HBM counters); not the benchmark line")
    ap.add_argument("--pool-sweep", default="",
                    help="write a pool-size sweep (per-call time vs rotated pool size) to "
                         "PREFIX.json and PREFIX.md and exit")
    ap.add_argument("--mx-variants", action="store_true",
                    help="with --mxfp8-only: M = 1..8 and both MX kernels at every M")
    ap.add_argument("--mxfp8-only", action="store_true",
                    help="time only the MXFP8- and MXFP4-weight cells and print them "
                         "(profiler runs of those kernels); not the benchmark line")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py measures one GPU: this path runs on a single MI355X with no "
              "sharding or collectives (got --gpus %d)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import projection_gemm_sparse_amd as P
    import synthetic_inputs as si

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.mfma_only:
        import synthetic_inputs as si2
        w_bytes = sum(N) * K * 2
        n_copies = max(2, math.ceil((args.pool_mib << 20) / w_bytes))
        plans = build_pool(P, torch, n_copies, 128)
        res = {}
        for M in (8, 9, 16, 17, 24, 32, 48, 64, 96, 128):
            x = si2.make_case(K, N, "bf16", M, seed=800 + M)[0].to(dev)
            out = [torch.empty(M, n, dtype=torch.bfloat16, device=dev) for n in N]
            gr = capture(torch, lambda: [p.forward(x, out=out) for p in plans])
            t, _ = time_graphs(torch, [gr], args.steps, 1)
            res[str(M)] = {"us": round(t * 1e3 / (args.steps * n_copies), 4),
                           "tiling": list(plans[0].get_tiling(M)),
                           "flops": 2 * M * sum(N) * K}
            del gr
        if args.calib_copy_mib:
            src = torch.ones((args.calib_copy_mib << 20) // 2, dtype=torch.bfloat16, device=dev)
            dst = torch.empty_like(src)
            for _ in range(3):
                torch.neg(src, out=dst)
            torch.cuda.synchronize()
        print(json.dumps({"mfma": res}), flush=True)
        return
    if args.indexer_splits:
        indexer_split_sweep(P, torch, dev, args.steps, args.indexer_splits)
        return
    if args.pool_sweep:
        rows = pool_sweep(P, torch, dev, max(3, args.steps // 4))
        write_outputs(args.pool_sweep, "Pool-size sweep, wq_a+wkv [1792, 5120] bf16 fused calls",
                      {"workload": "wq_a+wkv [1280,512]x5120 bf16 fused calls", "rows": rows},
                      ["pool MiB", "copies", "M", "us / call", "GB/s"],
                      [(r["pool_MiB"], r["copies"], r["M"], r["us"], r["GBps"]) for r in rows],
                      ["Per-call time of the fused call against the size of the rotated pool "
                       "(one copy, then 64 MiB .. 2 GiB); the time levels off once the pool is "
                       "past the 256 MiB MALL."])
        print(json.dumps({"pool_sweep": rows}), flush=True)
        return
    if args.mxfp8_only:
        Ms = tuple(range(1, 9)) + (12, 16) if args.mx_variants else (1, 2, 4, 8)
        res = {"mxfp8": mxfp8_cells(P, torch, dev, args.steps, Ms=Ms, variants=args.mx_variants),
               "mxfp4": mxfp8_cells(P, torch, dev, args.steps, Ms=Ms, fmt="mxfp4",
                                    variants=args.mx_variants),
               "nvfp4": mxfp8_cells(P, torch, dev, args.steps, Ms=Ms, fmt="nvfp4",
                                    variants=args.mx_variants)}
        if args.calib_copy_mib:
            src = torch.ones((args.calib_copy_mib << 20) // 2, dtype=torch.bfloat16, device=dev)
            dst = torch.empty_like(src)
            for _ in range(3):
                torch.neg(src, out=dst)
            torch.cuda.synchronize()
        print(json.dumps(res), flush=True)
        return
    w_bytes = sum(N) * K * 2
    n_copies = max(2, math.ceil((args.pool_mib << 20) / w_bytes))
    print("bench: pool of %d weight copies (%.0f MiB), M=%s" %
          (n_copies, n_copies * w_bytes / 2**20, list(MS)), file=sys.stderr, flush=True)
    plans = build_pool(P, torch, n_copies, max(MS))
    if args.crossover:
        del plans
        torch.cuda.empty_cache()
        crossover(args.crossover, P, torch, dev, args.crossover_workload, args.pool_mib)
        return
    if args.ceiling:
        ceiling_sweep(P, torch, dev, plans, n_copies, args.steps, args.ceiling)
        return

    xs_cpu, xs, outs = {}, {}, {}
    for M in MS:
        xc, _ = si.make_case(K, N, "bf16", M, seed=100 + M)
        xs_cpu[M] = xc
        xs[M] = xc.to(dev)
        outs[M] = [torch.empty(M, n, dtype=torch.bfloat16, device=dev) for n in N]

    def fused_calls(M):
        def run():
            for p in plans:
                p.forward(xs[M], out=outs[M])
        return run

    def separate_calls(M):
        def run():
            for p in plans:
                p.forward_separate(xs[M], out=outs[M])
        return run

    # per-launch floor of this stack: a graph of tiny one-block kernels
    tiny = torch.zeros(64, device=dev)
    floor_graph = capture(torch, lambda: [tiny.add_(1.0) for _ in range(n_copies)])
    floor_ms, _ = time_graphs(torch, [floor_graph], max(3, args.steps // 4), 1)
    floor_us = floor_ms * 1e3 / (max(3, args.steps // 4) * n_copies)

    fused_graphs = [capture(torch, fused_calls(M)) for M in MS]
    print("bench: graphs captured", file=sys.stderr, flush=True)
    total_ms, per_ms = time_graphs(torch, fused_graphs, args.steps, args.warmup)
    sep_steps = max(3, args.steps // 4)
    if args.fused_only or args.timed_only:
        sep_ms = [float("nan")] * len(MS)
    else:
        sep_graphs = [capture(torch, separate_calls(M)) for M in MS]
        _, sep_ms = time_graphs(torch, sep_graphs, sep_steps, 1)

    if args.timed_only:
        trials, trial_reps = [None] * len(MS), 0
        eager, ceiling = None, None
    else:
        trials, trial_reps = trial_stats(torch, fused_graphs, n_copies)
        eager = {str(M): eager_us(torch, fused_calls(M), n_copies) for M in (1, 8)}
        ceiling = stream_ceiling(P, torch, dev, plans, n_copies, max(3, args.steps // 2))

    calls = args.steps * n_copies
    per_m = {}
    step_bytes = 0
    for i, M in enumerate(MS):
        us = per_ms[i] * 1e3 / calls
        b = algorithmic_bytes(M, K, N)
        step_bytes += b * n_copies
        tl = plans[0].get_tiling(M)
        per_m[str(M)] = {
            "fused_us": round(us, 4),
            "separate_us": (None if args.fused_only or args.timed_only else
                            round(sep_ms[i] * 1e3 / (sep_steps * n_copies), 4)),
            "bytes": b,
            "fused_GBps": round(b / us / 1e3, 1),
            "frac_of_peak": round(b / us / 1e3 / HBM_PEAK_GBS, 4),
            "path": P._lib.PATH_NAMES[plans[0].query(M)[0]],
            "tiling": list(tl),
            "kernel": kernel_name(P, M, tl),
            "trials_us": trials[i],
        }
    ms_per_step = total_ms / args.steps
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    if args.calib_copy_mib:
        # counter calibration: an elementwise kernel that reads and writes
        # exactly calib_copy_mib MiB (bf16 negation)
        src = torch.ones((args.calib_copy_mib << 20) // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()

    # sanity check of one call against a plain PyTorch fp32 product (outside
    # the timed region)
    M = 4
    ref_w = plans[0].views
    ys = plans[0].forward(xs[M])
    torch.cuda.synchronize()
    worst = 0.0
    for y, w in zip(ys, ref_w):
        ref = xs[M].float() @ w.float().t()
        s = xs[M].float().abs() @ w.float().abs().t()
        worst = max(worst, float(((y.float() - ref).abs() / (2 ** -7 * s + 1e-6)).max()))
    if not worst <= 1.0:
        print("bench: SANITY FAILURE, |err|/bound = %.3g" % worst, file=sys.stderr)
        sys.exit(3)

    cpu = None
    if not args.no_cpu_baseline and not args.timed_only:
        w0 = [v.cpu() for v in plans[0].views]
        cpu = cpu_baseline(w0, xs_cpu)

    # dominant kernel: the instantiation with the most time in the step
    by_kernel = {}
    for M in MS:
        e = per_m[str(M)]
        k = e["kernel"]
        t_us, b_sum, n = by_kernel.get(k, (0.0, 0, 0))
        by_kernel[k] = (t_us + e["fused_us"], b_sum + e["bytes"], n + 1)
    dom = max(by_kernel, key=lambda k: by_kernel[k][0])
    t_us, b_sum, n_m = by_kernel[dom]
    bytes_launch = b_sum / n_m
    ev_us = t_us / n_m  # HIP events: timed region / launches, gaps included
    rec = recorded_kernel(dom)
    trace_us = (rec or {}).get("trace_avg_ns")
    trace_us = None if not trace_us else trace_us / 1e3
    launch_us = trace_us if trace_us else ev_us
    achieved = bytes_launch / launch_us / 1e3  # GB/s
    roofline = {
        "kernel": dom,
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": (rec or {}).get("hbm_bytes_per_launch"),
        "launch_us": round(launch_us, 4),
        "launch_us_source": ("rocprofv3 kernel-trace average of the kernel's graph-replayed "
                             "dispatches, profiles/traffic.json" if trace_us else
                             "HIP events (no current profile record)"),
        "bytes_per_launch": round(bytes_launch),
        "launch_us_events": round(ev_us, 4),
        "achieved_events": round(bytes_launch / ev_us / 1e3, 1),
        "frac_events": round(bytes_launch / ev_us / 1e3 / HBM_PEAK_GBS, 4),
        "note": "per launch, over the token counts this kernel serves in the step: "
                "achieved = algorithmic bytes per launch / average launch duration; "
                "launch_us_events = timed region / launches (HIP events on the launch "
                "stream, inter-kernel gaps included); traffic = HBM bytes per launch from "
                "rocprofv3 counters; both recorded values are used only while the kernel "
                "sources match the record",
    }
    us_all = [per_m[str(M)]["fused_us"] for M in MS]
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded U(-1/sqrt(K),1/sqrt(K)) weights, N(0,1) x, bf16)",
        "config": {
            "workload": "wq_a+wkv fused [1280,512]x5120 bf16, M=1..8, one fused call "
                        "per M per weight copy, %d copies rotated (%.2f GiB > 256 MiB MALL), "
                        "hipGraph replay" % (n_copies, n_copies * w_bytes / 2**30),
            "K": K, "N": list(N), "M": list(MS), "pool_copies": n_copies,
            "calls_per_step": n_copies * len(MS),
        },
        "us_per_call": {"mean_M1_8": round(sum(us_all) / len(us_all), 4),
                        "M1": per_m["1"]["fused_us"], "M8": per_m["8"]["fused_us"]},
        "launch_floor_us": round(floor_us, 4),
        "kernel_only_estimate": {
            "note": "per-call time minus the per-launch floor of a graph of tiny kernels",
            "us_M1": round(per_m["1"]["fused_us"] - floor_us, 4),
            "GBps_M1_8": round(step_bytes / ((ms_per_step * 1e-3) / 1.0 -
                                             floor_us * 1e-6 * n_copies * len(MS)) / 1e9, 1),
        },
        "roofline": roofline,
        "stream_ceiling": None if ceiling is None else dict(
            ceiling, fused_M1_over_ceiling=round(per_m["1"]["fused_us"] / ceiling["us_per_call"], 4),
            fused_minus_ceiling_us={str(M): round(per_m[str(M)]["fused_us"] -
                                                  ceiling["us_per_call"], 4) for M in MS}),
        "timing_protocol": {
            "trials": "per M: 15 trials of %d graph replays (%d calls each); median, p10, "
                      "p90 per call in per_m[M].trials_us; fused_us is the timed step "
                      "region" % (trial_reps, trial_reps * n_copies),
            "eager_us_per_call": eager,
            "eager_note": "the same fused calls launched one by one from Python (ctypes), "
                          "not captured; includes the Python call overhead"},
        "cpu_baseline": cpu,
        "per_m": per_m,
        "context": {"pages_sm107_fused_m1_us": 4.13,
                    "note": "Vera Rubin figure from the pages, other hardware"},
    }
    if not args.no_epilogues and not args.fused_only and not args.timed_only:
        line["epilogues"] = epilogue_cells(P, torch, dev, plans, n_copies,
                                           max(3, args.steps // 4))
        line["router_f32"] = router_cells(P, torch, dev, max(3, args.steps // 4))
        line["mxfp8"] = mxfp8_cells(P, torch, dev, max(3, args.steps // 4))
        line["mxfp4"] = mxfp8_cells(P, torch, dev, max(3, args.steps // 4), fmt="mxfp4")
        line["nvfp4"] = mxfp8_cells(P, torch, dev, max(3, args.steps // 4), fmt="nvfp4")
        line["indexer_f32"] = workload_cells(P, torch, dev, max(3, args.steps // 4),
                                             "indexer_f32")
        line["fused_a_3way"] = workload_cells(P, torch, dev, max(3, args.steps // 4),
                                              "fused_a_3way")
    print(json.dumps(line), flush=True)
    if args.details:
        with open(args.details, "w") as fh:
            json.dump(line, fh, indent=1)


if __name__ == "__main__":
    main()
