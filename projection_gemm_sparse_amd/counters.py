"""Summaries of rocprofv3 runs of bench.py (kernel trace and HBM counters).

    python -m projection_gemm_sparse_amd.counters --trace DIR --pmc DIR [DIR ...] \\
        --calib-bytes B --out-md FILE.md --out-json profiles/traffic.json --command "..."
    python -m projection_gemm_sparse_amd.counters --trace DIR --trace-only \\
        --out-md FILE.md --command "..."
    python -m projection_gemm_sparse_amd.counters --mfma --pmc DIR [--trace DIR] \\
        --out-md FILE.md --command "..."

Reads the CSV files rocprofv3 writes (``*_kernel_stats.csv`` of a
``--kernel-trace --stats`` run; ``*_counter_collection.csv`` of ``--pmc``
runs) and writes a markdown table of the library's kernels plus, for the
skinny and tile kernels, the HBM bytes read and written per launch.

HBM bytes per launch come from the L2-to-fabric request counters
(TCC_EA0_RDREQ_{32B,64B,128B}_sum, TCC_EA0_WRREQ_{64B,}_sum: bytes = size
x requests), each divided by the factor the same counters read for the
elementwise kernel of known size (bf16 negation: reads and writes
--calib-copy-mib MiB) that bench.py runs with --calib-copy-mib.
The derived FETCH_SIZE / WRITE_SIZE are summarised too, but FETCH_SIZE
counts the non-temporal 16-byte loads of these kernels at about half their
size, so the request counters are the ones used.  The record carries a
digest of the kernel sources; bench.py reports the traffic only while the
sources still match it.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import re
import statistics

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _short(name: str) -> str:
    return re.sub(r"\(.*$", "", name).strip()


def _open_csv(path):
    if path.endswith(".gz"):
        import gzip
        return gzip.open(path, "rt")
    return open(path)


def load_pmc(dirs):
    """{(kernel, grid): {counter: [values per dispatch]}} from the
    ``*counter_collection.csv`` (or ``.csv.gz``) files of the runs."""
    out = {}
    for d in dirs:
        for path in (glob.glob(os.path.join(d, "*counter_collection.csv")) +
                     glob.glob(os.path.join(d, "*counter_collection.csv.gz"))):
            with _open_csv(path) as fh:
                for r in csv.DictReader(fh):
                    key = (_short(r["Kernel_Name"]), int(r["Grid_Size"]))
                    out.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(
                        float(r["Counter_Value"]))
    return out


def load_stats(d):
    rows = []
    for path in glob.glob(os.path.join(d, "*kernel_stats.csv")):
        with open(path) as fh:
            for r in csv.DictReader(fh):
                rows.append({"kernel": _short(r["Name"]), "calls": int(r["Calls"]),
                             "avg_ns": float(r["AverageNs"]), "min_ns": float(r["MinNs"]),
                             "max_ns": float(r["MaxNs"])})
    return rows


def load_back_to_back(d, gap_ns=1000):
    """Per kernel, the dispatches of the ``*kernel_trace.csv`` of a run that
    started within ``gap_ns`` of the previous dispatch's end on the same queue
    (graph replays of back-to-back calls, not eager launches from the host):
    {kernel: (count, average duration ns)}."""
    acc = {}
    for path in (glob.glob(os.path.join(d, "*kernel_trace.csv")) +
                 glob.glob(os.path.join(d, "*kernel_trace.csv.gz"))):
        with _open_csv(path) as fh:
            rows = [(int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Queue_Id"],
                     _short(r["Kernel_Name"])) for r in csv.DictReader(fh)]
        rows.sort()
        last_end = {}
        for st, en, q, k in rows:
            prev = last_end.get(q)
            if prev is not None and st - prev <= gap_ns:
                n, tot = acc.get(k, (0, 0))
                acc[k] = (n + 1, tot + (en - st))
            last_end[q] = en
    return {k: (n, tot / n) for k, (n, tot) in acc.items()}


def back_to_back_runs(dirs, gap_ns=1000):
    """load_back_to_back over repeated runs of one command (one directory
    each): {kernel: (median over the runs of the run's average, [each run's
    average])}.  The profiler spaces graph-replayed dispatches unevenly and
    differently from box to box, so one run's average is a noisy figure;
    the median of several independent runs is the one recorded."""
    per = {}
    for d in dirs:
        for k, (n, avg) in load_back_to_back(d, gap_ns).items():
            per.setdefault(k, []).append(avg)
    return {k: (statistics.median(v), v) for k, v in per.items()}


def med(vals):
    return statistics.median(vals) if vals else None


def hbm_bytes(c):
    """Read and write bytes per dispatch from the request counters."""
    rd = None
    if "TCC_EA0_RDREQ_128B_sum" in c:
        rd = (128 * med(c["TCC_EA0_RDREQ_128B_sum"]) + 64 * med(c.get("TCC_EA0_RDREQ_64B_sum", [0]))
              + 32 * med(c.get("TCC_EA0_RDREQ_32B_sum", [0])))
    wr = None
    if "TCC_EA0_WRREQ_sum" in c and "TCC_EA0_WRREQ_64B_sum" in c:
        w64 = med(c["TCC_EA0_WRREQ_64B_sum"])
        wr = 64 * w64 + 32 * (med(c["TCC_EA0_WRREQ_sum"]) - w64)
    return rd, wr


def trace_only(args):
    """Markdown table of the library's kernels in one kernel-trace run."""
    rows = [r for r in load_stats(args.trace[0])
            if r["kernel"].startswith("void fp::") or r["kernel"].startswith("fp::")]
    lines = ["# %s" % (args.title or "Kernel trace"), "",
             "Command (run from /tmp with TMPDIR=/tmp, repository root $R):", "", "```"]
    lines += args.command + ["```", ""]
    b2b = load_back_to_back(args.trace[0])
    lines += ["Back-to-back: the dispatches that started within 1 us of the previous one's "
              "end on the same queue (graph replays of consecutive calls; the trace's "
              "durations then tile the timeline, launch gaps included).", ""]
    lines += ["| kernel | calls | avg ns | min ns | max ns | back-to-back calls | "
              "back-to-back avg ns |", "|---|---|---|---|---|---|---|"]
    for r in sorted(rows, key=lambda r: r["kernel"]):
        n, a = b2b.get(r["kernel"], (0, None))
        lines.append("| `%s` | %d | %.1f | %.0f | %.0f | %d | %s |" % (
            r["kernel"].replace("void ", ""), r["calls"], r["avg_ns"], r["min_ns"], r["max_ns"],
            n, "" if a is None else "%.1f" % a))
    with open(args.out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("wrote", args.out_md)


def mfma_summary(args):
    """Matrix-core use per kernel from one --pmc run of
    SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_BF16 and
    GRBM_GUI_ACTIVE (medians per dispatch) and the kernel trace's average
    duration: busy fraction = busy SIMD-cycles / (SIMDs x duration x clock),
    bf16 rate = MOPS x 512 flops / duration against the dense bf16 peak.
    The profiler's own MfmaUtil divides by GRBM_GUI_ACTIVE instead, which
    under counter collection covers the whole serialized dispatch and is
    summed over the XCDs; it is listed as read."""
    simds, ghz, peak = args.simds, args.clock_ghz, args.peak_tflops
    pmc = load_pmc(args.pmc)
    stats = {r["kernel"]: r for r in load_stats(args.trace[0])} if args.trace else {}
    lines = ["# %s" % (args.title or "Matrix-core utilisation"), "",
             "Commands (run from /tmp with TMPDIR=/tmp, repository root $R):", "", "```"]
    lines += args.command + ["```", ""]
    lines += ["Busy = SQ_VALU_MFMA_BUSY_CYCLES / (%d SIMDs x trace duration x %.1f GHz); "
              "rate = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 flops / trace duration, against "
              "%.0f TFLOP/s dense bf16; cycles/MFMA = busy cycles / (MOPS / 32) "
              "(one 16x16x32 bf16 MFMA = 32 MOPS); medians per dispatch; the profiler's "
              "MfmaUtil (busy / (GRBM_GUI_ACTIVE x SIMDs)) as read."
              % (simds, ghz, peak), ""]
    lines += ["| kernel | grid | dispatches | avg ns (trace) | MFMA flops / dispatch | "
              "bf16 TFLOP/s | % of peak | busy % | cycles / MFMA | MfmaUtil as read % |",
              "|---|---|---|---|---|---|---|---|---|---|"]
    for (k, grid), c in sorted(pmc.items()):
        if not (k.startswith("void fp::") or k.startswith("fp::")):
            continue
        busy = med(c.get("SQ_VALU_MFMA_BUSY_CYCLES", []))
        mops = med(c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", []))
        act = med(c.get("GRBM_GUI_ACTIVE", []))
        if busy is None or act is None or not mops:
            continue
        st = stats.get(k) or {}
        ns = st.get("avg_ns")
        flops = mops * 512
        if ns:
            rate = flops / ns / 1e3
            cells = "%.0f | %.4g | %.1f | %.2f | %.2f | %.2f" % (
                ns, flops, rate, 100.0 * rate / peak, 100.0 * busy / (simds * ns * ghz),
                busy / (mops / 32))
        else:
            cells = " | %.4g | | | | %.2f" % (flops, busy / (mops / 32))
        lines.append("| `%s` | %d | %d | %s | %.2f |" % (
            k.replace("void ", ""), grid, len(c.get("GRBM_GUI_ACTIVE", [])), cells,
            100.0 * busy / (act * simds)))
    with open(args.out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("wrote", args.out_md)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--trace", nargs="+", default=[],
                    help="kernel-trace run directories (repeated runs of one command: the "
                         "median of their back-to-back averages is recorded)")
    ap.add_argument("--trace-only", action="store_true",
                    help="only summarise the kernel trace (no counters)")
    ap.add_argument("--mfma", action="store_true",
                    help="summarise one run of the MFMA counters (see mfma_summary)")
    ap.add_argument("--simds", type=int, default=1024, help="SIMDs of the GPU (MI355X: 1024)")
    ap.add_argument("--clock-ghz", type=float, default=2.4, help="engine clock (MI355X: 2.4)")
    ap.add_argument("--peak-tflops", type=float, default=2500.0,
                    help="dense bf16 matrix peak (MI355X: 2500)")
    ap.add_argument("--pmc", nargs="+", default=[])
    ap.add_argument("--calib-bytes", type=int, default=0,
                    help="bytes read (and written) by the calibration copy kernel")
    ap.add_argument("--calib-name", default="neg_kernel",
                    help="substring of the calibration kernel's name")
    ap.add_argument("--out-md", required=True)
    ap.add_argument("--out-json", default="")
    ap.add_argument("--command", action="append", default=[])
    ap.add_argument("--title", default="")
    args = ap.parse_args()
    if args.trace_only:
        trace_only(args)
        return
    if args.mfma:
        mfma_summary(args)
        return
    if not args.pmc or not args.calib_bytes or not args.out_json:
        raise SystemExit("--pmc, --calib-bytes and --out-json are needed with counters")

    import sys
    sys.path.insert(0, ROOT)
    import bench

    pmc = load_pmc(args.pmc)
    calib = None
    calib_grid = None
    for (k, grid), c in pmc.items():
        if args.calib_name in k and (calib_grid is None or grid > calib_grid):
            calib, calib_grid = c, grid
    if calib is None:
        raise SystemExit("no calibration kernel named *%s* in the counter runs" % args.calib_name)
    crd, cwr = hbm_bytes(calib)
    f_rd = crd / args.calib_bytes if crd else None
    f_wr = cwr / args.calib_bytes if cwr else None
    f_fetch = (med(calib.get("FETCH_SIZE", [])) or 0) * 1024 / args.calib_bytes or None
    f_write = (med(calib.get("WRITE_SIZE", [])) or 0) * 1024 / args.calib_bytes or None

    stats = {r["kernel"]: r for r in load_stats(args.trace[0])}
    b2b = back_to_back_runs(args.trace)
    lines = ["# %s" % (args.title or "Fused projection kernels: duration and HBM traffic"), "",
             "Commands (run from /tmp with TMPDIR=/tmp, repository root $R):", "", "```"]
    lines += args.command + ["```", ""]
    lines += ["Calibration: the bf16 negation kernel over %d bytes (grid %d) reads as %s read bytes "
              "and %s written bytes by the request counters (factors %s / %s), FETCH_SIZE "
              "factor %s, WRITE_SIZE factor %s." % (
                  args.calib_bytes, calib_grid, crd, cwr,
                  None if f_rd is None else round(f_rd, 4),
                  None if f_wr is None else round(f_wr, 4),
                  None if f_fetch is None else round(f_fetch, 4),
                  None if f_write is None else round(f_write, 4)), ""]
    if len(args.trace) > 1:
        lines += ["The kernel-trace command ran %d times, each in a separate GPU session; "
                  "avg ns (back-to-back) is the median over those runs of each run's "
                  "average, every run's average listed beside it." % len(args.trace), ""]
    lines += ["avg ns (back-to-back): the kernel-trace average over the dispatches that "
              "started within 1 us of the previous one's end (graph replays of consecutive "
              "calls); avg ns (all) includes eager launches (first run).", ""]
    lines += ["| kernel | grid | calls | avg ns (all) | avg ns (back-to-back) | per run | "
              "min ns | HBM read B/launch | HBM write B/launch | FETCH_SIZE B (scaled) | "
              "WRITE_SIZE B (scaled) |",
              "|---|---|---|---|---|---|---|---|---|---|---|"]
    rec = {"kernel_sources_sha256_16": bench.kernel_sources_digest(), "kernels": {},
           "calibration": {"bytes": args.calib_bytes, "read_factor": f_rd, "write_factor": f_wr}}
    for (k, grid), c in sorted(pmc.items()):
        if not (k.startswith("void fp::") or k.startswith("fp::")):
            continue
        name = k.replace("void ", "")
        rd, wr = hbm_bytes(c)
        rd = rd / f_rd if (rd is not None and f_rd) else None
        wr = wr / f_wr if (wr is not None and f_wr) else None
        fs = med(c.get("FETCH_SIZE", []))
        ws = med(c.get("WRITE_SIZE", []))
        fs = fs * 1024 / f_fetch if (fs is not None and f_fetch) else None
        ws = ws * 1024 / f_write if (ws is not None and f_write) else None
        st = stats.get(k) or stats.get(name) or {}
        bb, runs = b2b.get(k) or b2b.get(name) or (None, [])
        lines.append("| `%s` | %d | %s | %s | %s | %s | %s | %s | %s | %s | %s |" % (
            name, grid, st.get("calls", ""), st.get("avg_ns", ""),
            "" if bb is None else round(bb, 1), ", ".join("%.1f" % v for v in runs),
            st.get("min_ns", ""),
            None if rd is None else round(rd), None if wr is None else round(wr),
            None if fs is None else round(fs), None if ws is None else round(ws)))
        if rd is not None and wr is not None:
            rec["kernels"][name] = {"grid": grid, "hbm_read_bytes_per_launch": round(rd),
                                    "hbm_write_bytes_per_launch": round(wr),
                                    "hbm_bytes_per_launch": round(rd + wr),
                                    "trace_avg_ns": None if bb is None else round(bb, 1),
                                    "trace_avg_ns_runs": [round(v, 1) for v in runs],
                                    "trace_avg_ns_all": st.get("avg_ns")}
    with open(args.out_md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    with open(args.out_json, "w") as fh:
        json.dump(rec, fh, indent=1)
    print("wrote", args.out_md, args.out_json)


if __name__ == "__main__":
    main()
