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
per launch over its average launch duration (HIP events over the timed
region, on the launch stream), against the 8 TB/s HBM peak, with the HBM
traffic per launch measured by rocprofv3 counters when the recorded
measurement (profiles/traffic.json) matches the current kernel sources;
per-M microseconds per call for the fused and the one-launch-per-projection
path; ``cpu_baseline`` = the CPU oracle (single thread) on a bounded sample
of the same M sweep over one copy.

``--crossover FILE`` additionally times, per token count M in
{1, 2, 4, 8, 9, 16, 32, 64, 128}, every kernel path that serves M (vector
ALU, small-M matrix core, tile) on the same rotated pool and writes the
table to FILE: the measured crossover that places the MFMA path.
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


def recorded_traffic(kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter record,
    or None when there is none or the kernel sources changed since."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_sources_sha256_16") != kernel_sources_digest():
        return None
    ent = rec.get("kernels", {}).get(kernel)
    return None if ent is None else ent.get("hbm_bytes_per_launch")


def kernel_name(P, M: int, tiling) -> str:
    """The kernel instantiation a (resolved) tiling runs, as rocprofv3 names it."""
    path, kparts, chunks, splits, rows, groups = tiling
    if path in (P.FP_PATH_SKINNY, P.FP_PATH_SKINNY_SPLITK):
        mt = 1 if M <= 1 else 2 if M <= 2 else 4 if M <= 4 else 8
        return "fp::skinny_kernel<%d, %d, %d, true, 0>" % (mt, rows, chunks)
    if path == P.FP_PATH_MFMA_SMALL:
        # token halves; with two, up to 12 tokens the interleaved load order
        return "fp::smfma_kernel<%d, false, %d, %s>" % (
            chunks, 1 if M <= 8 else 2, "false" if 8 < M <= 12 else "true")
    mt16 = next(b for b in (1, 2, 4, 8, 16) if 16 * b >= M)
    cs = 4 if chunks in (8, 16) else 5
    return "fp::tile_kernel<%d, %d, %d, %d>" % (mt16, kparts, cs, chunks // cs)


def algorithmic_bytes(M: int, K: int, N, esize: int = 2) -> int:
    n_total = sum(N)
    return esize * (n_total * K + M * K + M * n_total)


def build_pool(P, torch, n_copies, max_M, seed=0):
    """n_copies independent weight sets U(-1/sqrt(K), 1/sqrt(K)) -> bf16,
    drawn on the GPU, each concatenated by its own plan."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    a = 1.0 / math.sqrt(K)
    plans = []
    for _ in range(n_copies):
        ws = [((torch.rand(n, K, generator=g, device="cuda") * 2 - 1) * a)
              .to(torch.bfloat16) for n in N]
        plans.append(P.FusedProjection(ws, max_M=max_M))
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


def cpu_baseline(plan0_weights_cpu, xs_cpu, budget_s=12.0):
    """The oracle (single-threaded C loop, fp64) on the M = 1..8 sweep over
    one weight copy, repeated until ``budget_s`` of CPU time is spent."""
    import oracle
    import synthetic_inputs as si
    oracle.build(force=False)
    wb = [si.bits(w) for w in plan0_weights_cpu]
    passes, t0 = 0, time.perf_counter()
    while True:
        for M in MS:
            xb = si.bits(xs_cpu[M])
            for w in wb:
                oracle.linear(xb, w)
        passes += 1
        el = time.perf_counter() - t0
        if el >= budget_s or passes >= 50:
            break
    byts = passes * sum(algorithmic_bytes(M, K, N) for M in MS)
    return {"value": byts / el / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "host": host_info(),
            "sample": "%d pass(es) of the M=1..8 sweep over one [1792, 5120] bf16 "
                      "weight copy, %.1f s, single-threaded C fp64 loop" % (passes, el),
            "us_per_call": el / (passes * len(MS)) * 1e6}


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


def crossover(path, P, torch, dev, plans, n_copies):
    """Per token count, every kernel path that serves it, on the rotated
    pool (plans are made for max_M = 8, so a second pool is built)."""
    import synthetic_inputs as si
    del plans
    torch.cuda.empty_cache()
    big = build_pool(P, torch, n_copies, 128)
    n_total = sum(N)
    tile_min = next(m for m in range(2, 257)
                    if P.fp_default_tiling(0, K, n_total, m, n_total)[1][0] == P.FP_PATH_MFMA)
    rows = []
    for M in (1, 2, 3, 4, 5, 8, 9, 16, 32, 64, 128):
        xc, _ = si.make_case(K, N, "bf16", M, seed=200 + M)
        x = xc.to(dev)
        out = [torch.empty(M, n, dtype=torch.bfloat16, device=dev) for n in N]
        cands = [("default", None)]
        kc = K * 2 // 16
        steps = -(-kc // 8)
        kt = 4 if steps <= 64 else 8 if steps <= 128 else 16
        if M <= 8:
            cands.append(("skinny", (P.FP_PATH_SKINNY, 10, 1, 1, 0, 0)))
        if M <= 16:
            cands.append(("mfma_small", (P.FP_PATH_MFMA_SMALL, -(-steps // kt), kt, 1, 0, 0)))
        if 8 < M < tile_min:
            cands.append(("tile", "tile"))
        for name, t in cands:
            if t == "tile":
                for p in big:
                    p.set_mfma_min_m(M)
            elif t is not None and any(p.set_tiling(M, t) for p in big):
                for p in big:
                    p.set_tiling(M, None)
                continue
            g = capture(torch, lambda: [p.forward(x, out=out) for p in big])
            ms, _ = time_graphs(torch, [g], 10, 2)
            us = ms * 1e3 / (10 * n_copies)
            b = algorithmic_bytes(M, K, N)
            rows.append({"M": M, "variant": name,
                         "path": P._lib.PATH_NAMES[big[0].query(M)[0]],
                         "tiling": list(big[0].get_tiling(M)), "us": round(us, 3),
                         "GBps": round(b / us / 1e3, 1)})
            print("bench: crossover %s" % json.dumps(rows[-1]), file=sys.stderr, flush=True)
            for p in big:
                p.set_tiling(M, None)
                p.set_mfma_min_m(tile_min)
            del g
    with open(path, "w") as fh:
        json.dump({"workload": "wq_a+wkv [1280,512]x5120 bf16, %d rotated copies" % n_copies,
                   "rows": rows}, fh, indent=1)


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
                    help="also time every kernel path per M in 1..128 and write the table here")
    ap.add_argument("--mfma-only", action="store_true",
                    help="time only the matrix-core cells (M = 8 on the small-M kernel, "
                         "9..128 on the tile kernel) and print them (profiler runs of the "
                         "MFMA counters); not the benchmark line")
    ap.add_argument("--pool-sweep", default="",
                    help="write a pool-size sweep (per-call time vs rotated pool size) to this "
                         "JSON file and exit")
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
        for M in (8, 9, 16, 32, 64, 128):
            x = si2.make_case(K, N, "bf16", M, seed=800 + M)[0].to(dev)
            out = [torch.empty(M, n, dtype=torch.bfloat16, device=dev) for n in N]
            gr = capture(torch, lambda: [p.forward(x, out=out) for p in plans])
            t, _ = time_graphs(torch, [gr], args.steps, 1)
            res[str(M)] = {"us": round(t * 1e3 / (args.steps * n_copies), 4),
                           "tiling": list(plans[0].get_tiling(M)),
                           "flops": 2 * M * sum(N) * K}
            del gr
        print(json.dumps({"mfma": res}), flush=True)
        return
    if args.pool_sweep:
        rows = pool_sweep(P, torch, dev, max(3, args.steps // 4))
        with open(args.pool_sweep, "w") as fh:
            json.dump({"workload": "wq_a+wkv [1280,512]x5120 bf16 fused calls", "rows": rows},
                      fh, indent=1)
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
    if args.fused_only:
        sep_ms = [float("nan")] * len(MS)
    else:
        sep_graphs = [capture(torch, separate_calls(M)) for M in MS]
        _, sep_ms = time_graphs(torch, sep_graphs, sep_steps, 1)

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
            "separate_us": (None if args.fused_only else
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
    if not args.no_cpu_baseline:
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
    achieved = b_sum / t_us / 1e3  # GB/s: bytes per launch / average launch duration
    traffic = recorded_traffic(dom)
    roofline = {
        "kernel": dom,
        "bound": "hbm",
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic,
        "launch_us": round(t_us / n_m, 4),
        "bytes_per_launch": round(b_sum / n_m),
        "note": "per launch, over the token counts this kernel serves in the step; launch "
                "duration = timed region / launches (HIP events on the launch stream); "
                "traffic = HBM bytes per launch from rocprofv3 counters (null if the "
                "kernel changed since they were taken)",
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
        "stream_ceiling": dict(ceiling, fused_M1_over_ceiling=round(
            per_m["1"]["fused_us"] / ceiling["us_per_call"], 4)),
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
    if not args.no_epilogues and not args.fused_only:
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
    if args.crossover:
        crossover(args.crossover, P, torch, dev, plans, n_copies)
    print(json.dumps(line), flush=True)
    if args.details:
        with open(args.details, "w") as fh:
            json.dump(line, fh, indent=1)


if __name__ == "__main__":
    main()
