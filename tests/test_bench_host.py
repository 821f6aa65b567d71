"""Host logic of bench.py (no GPU): the kernel names it looks up in the
counter record, the gate on the kernel-source digest, the algorithmic
bytes of a call."""
import json
import os
import re

import bench
import projection_gemm_sparse_amd as P


def test_kernel_names_of_the_default_tilings():
    assert (bench.kernel_name(P, 1, (P.FP_PATH_SKINNY, 10, 1, 1, 7, 1))
            == "fp::skinny_kernel<1, 7, 1, true, 0>")
    assert (bench.kernel_name(P, 2, (P.FP_PATH_SKINNY, 10, 1, 1, 7, 1))
            == "fp::skinny_kernel<2, 7, 1, true, 0>")
    small = (P.FP_PATH_MFMA_SMALL, 10, 8, 1, 7, 1)
    for M in range(3, 9):
        assert bench.kernel_name(P, M, small) == "fp::smfma_kernel<8, false, 1, true, 1>"
    for M in range(9, 13):
        assert bench.kernel_name(P, M, small) == "fp::smfma_kernel<8, false, 2, false, 1>"
    for M in range(13, 17):
        assert bench.kernel_name(P, M, small) == "fp::smfma_kernel<8, false, 2, true, 1>"
    for M in range(17, 25):
        assert bench.kernel_name(P, M, small) == "fp::smfma_kernel<8, false, 3, true, 1>"
    # two row tiles of 6 per wave (plans of more rows than 8 per CU)
    two = (P.FP_PATH_MFMA_SMALL, 12, 8, 1, 12, 1)
    assert bench.kernel_name(P, 8, two) == "fp::smfma_kernel<8, false, 1, true, 2>"


def test_two_halves_order_threshold_matches_the_library():
    # the library picks the interleaved two-halves instantiation up to this
    # many tokens; the bench names it the same way
    src = open(os.path.join(bench.ROOT, "projection_gemm_sparse_amd", "csrc", "k_smfma.hip")).read()
    m = re.search(r"constexpr int kSmfmaInterleaveMaxM = (\d+);", src)
    assert m is not None
    lim = int(m.group(1))
    small = (P.FP_PATH_MFMA_SMALL, 10, 8, 1, 7, 1)
    assert bench.kernel_name(P, lim, small).endswith(", false, 1>")
    assert bench.kernel_name(P, lim + 1, small).endswith(", true, 1>")


def test_recorded_traffic_needs_the_current_kernel_sources(tmp_path, monkeypatch):
    name = "fp::smfma_kernel<8, false, 1, true, 1>"
    rec = {"kernel_sources_sha256_16": bench.kernel_sources_digest(),
           "kernels": {name: {"hbm_bytes_per_launch": 12345}}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.recorded_traffic(name) == 12345
    assert bench.recorded_traffic("fp::no_such_kernel") is None
    rec["kernel_sources_sha256_16"] = "0" * 16
    f.write_text(json.dumps(rec))
    assert bench.recorded_traffic(name) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.recorded_traffic(name) is None


def test_algorithmic_bytes_of_the_headline_call():
    # weights + activations + outputs, bf16
    assert bench.algorithmic_bytes(1, 5120, (1280, 512)) == 2 * (1792 * 5120 + 5120 + 1792)
    assert bench.algorithmic_bytes(8, 5120, (1280, 512)) == 18350080 + 2 * 8 * (5120 + 1792)
    assert bench.algorithmic_bytes(1, 7168, (128, 64), esize=4) == 4 * (192 * 7168 + 7168 + 192)


def test_trace_runs_record_the_median_of_each_runs_back_to_back_average(tmp_path):
    from projection_gemm_sparse_amd import counters
    head = "Kind,Queue_Id,Kernel_Name,Start_Timestamp,End_Timestamp\n"

    def run(name, durations, gap=100):
        d = tmp_path / name
        d.mkdir()
        t, lines = 0, []
        for du in durations:
            lines.append("KERNEL_DISPATCH,1,fp::k(int),%d,%d" % (t, t + du))
            t += du + gap
        # an eager launch far from the previous end: not back-to-back
        lines.append("KERNEL_DISPATCH,1,fp::k(int),%d,%d" % (t + 50000, t + 59000))
        (d / "bench_kernel_trace.csv").write_text(head + "\n".join(lines) + "\n")
        return str(d)

    dirs = [run("a", [100, 100, 100]), run("b", [300, 300, 300]), run("c", [200, 220, 180])]
    one = counters.load_back_to_back(dirs[0])
    assert one["fp::k"] == (2, 100.0)  # the first dispatch has no predecessor
    med, per = counters.back_to_back_runs(dirs)["fp::k"]
    assert per == [100.0, 300.0, 200.0] and med == 200.0
