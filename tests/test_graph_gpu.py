"""hipGraph capture of the fused call: replays bitwise equal to eager.

"tinygemm2 for the DeepSeek-V4.1 hidden-state projections" (TensorRT-LLM
PR #20636), Test Coverage: CUDA graph capture/replay of the fused call is
bitwise equal to eager over three new inputs, and a 20,000-replay stress
with no positive control.  Here the 20,000 replays run too (fixed input,
every replay compared with the first), and in the shorter stresses every
replay gets new inputs written into
the captured input buffer, the program's own eager calls and
synchronizations run between replays, every replay is compared with an
eager run, and a positive control (a perturbed input) must be detected.
Split-K launches are included -- the tile and ring tile kernels of the
crossover cases (32, 64 and 128 tokens) and a forced K split of the
vector-ALU kernel (the fp32 indexer fusion, its in-launch finish) -- and
their arrival counters reset themselves, so replays need no host action.
"""
import ctypes

import numpy as np
import pytest
import torch

import synthetic_inputs as si
import projection_gemm_sparse_amd as P
from gpu_util import assert_bitwise_equal, assert_matches_oracle, out_bits, to_gpu

pytestmark = pytest.mark.gpu


def _capture(fp, x_static, outs):
    fp(x_static, out=outs)  # eager warm-up (kernel attributes set outside capture)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp(x_static, out=outs)
    torch.cuda.synchronize()
    return g


CASES = [("wq_a+wkv_m1", 1), ("wq_a+wkv_m2_8", 8), ("indexer_f32", 4),
         ("fused_a_3way", 1), ("fused_a_3way", 5), ("fused_a_3way", 8),
         ("crossover", 12), ("crossover", 32), ("crossover", 64), ("crossover", 128)]


@pytest.mark.parametrize("name,M", CASES)
def test_replay_bitwise_equal_to_eager(name, M):
    x0, ws = si.workload_case(name, M, 0)
    fp = P.FusedProjection([to_gpu(w) for w in ws], max_M=max(8, M))
    x_static = to_gpu(x0)
    outs = [torch.empty(M, n, dtype=x_static.dtype, device="cuda") for n in fp.N]
    g = _capture(fp, x_static, outs)
    # above 16 tokens the oracle checks sampled token rows (every element is
    # still compared with the eager call)
    rows = None if M <= 16 else sorted({0, 1, M // 2, M - 1} | set(range(5, M, 31)))
    for seed in (11, 12, 13):
        xn, _ = si.workload_case(name, M, seed)
        x_static.copy_(to_gpu(xn))
        g.replay()
        torch.cuda.synchronize()
        eager = fp(x_static)  # eager call between replays
        assert_bitwise_equal(outs, eager, "%s M=%d replay seed %d" % (name, M, seed))
        assert_matches_oracle(outs, xn, ws, rows=rows, label="%s replay" % name)


@pytest.mark.parametrize("name,M", [("wq_a+wkv_m1", 1), ("indexer_f32", 8), ("crossover", 16),
                                    ("crossover", 20)])
def test_replay_stress_with_positive_control(name, M):
    x0, ws = si.workload_case(name, M, 0)
    fp = P.FusedProjection([to_gpu(w) for w in ws], max_M=max(8, M))
    x_static = to_gpu(x0)
    outs = [torch.empty(M, n, dtype=x_static.dtype, device="cuda") for n in fp.N]
    g = _capture(fp, x_static, outs)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1234)
    mismatches = 0
    for it in range(300):
        x_static.copy_(torch.randn(x_static.shape, generator=gen, device="cuda")
                       .to(x_static.dtype))
        g.replay()
        eager = fp(x_static)
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            if not torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else
                               a.view(torch.int32),
                               b.view(torch.int16) if b.dtype == torch.bfloat16 else
                               b.view(torch.int32)):
                mismatches += 1
    assert mismatches == 0
    # positive control: the same comparison must see a one-element change
    g.replay()
    x_pert = x_static.clone()
    x_pert[0, 17] += 1.0
    eager = fp(x_pert)
    torch.cuda.synchronize()
    differs = any(not np.array_equal(p, q) for p, q in zip(out_bits(outs), out_bits(eager)))
    assert differs, "comparison cannot see a perturbed input"


@pytest.mark.parametrize("name,M", [("wq_a+wkv_m1", 1), ("wq_a+wkv_m2_8", 8), ("crossover", 32)])
def test_twenty_thousand_replays_stay_bitwise_stable(name, M):
    """The pages' stress length: 20,000 replays of one captured call on a
    fixed input, every replay's outputs compared on the device with the
    first replay's (and those with an eager call); at 32 tokens the split
    finish's arrival counters must reset themselves every time."""
    x0, ws = si.workload_case(name, M, 5)
    fp = P.FusedProjection([to_gpu(w) for w in ws], max_M=max(8, M))
    x_static = to_gpu(x0)
    outs = [torch.empty(M, n, dtype=x_static.dtype, device="cuda") for n in fp.N]
    g = _capture(fp, x_static, outs)
    g.replay()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    assert_bitwise_equal(ref, fp(x_static), "%s M=%d first replay vs eager" % (name, M))
    diff = torch.zeros((), dtype=torch.int64, device="cuda")
    for _ in range(20000):
        g.replay()
        for o, r in zip(outs, ref):
            diff += (o.view(torch.int16) != r.view(torch.int16)).sum()
    torch.cuda.synchronize()
    assert int(diff) == 0, "%d output elements changed over 20,000 replays" % int(diff)
    assert_matches_oracle(outs, x0, ws, rows=None if M <= 16 else [0, M - 1],
                          label="%s M=%d after 20,000 replays" % (name, M))


def _hip():
    return ctypes.CDLL("libamdhip64.so")


def _count_graph_nodes(fn, stream: torch.cuda.Stream) -> int:
    hip = _hip()
    hip.hipStreamBeginCapture.argtypes = [ctypes.c_void_p, ctypes.c_int]
    hip.hipStreamEndCapture.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_void_p)]
    hip.hipGraphGetNodes.argtypes = [ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.POINTER(ctypes.c_size_t)]
    hip.hipGraphDestroy.argtypes = [ctypes.c_void_p]
    h = ctypes.c_void_p(stream.cuda_stream)
    assert hip.hipStreamBeginCapture(h, 2) == 0  # relaxed mode
    try:
        fn()
    finally:
        graph = ctypes.c_void_p()
        assert hip.hipStreamEndCapture(h, ctypes.byref(graph)) == 0
    n = ctypes.c_size_t(0)
    assert hip.hipGraphGetNodes(graph, None, ctypes.byref(n)) == 0
    hip.hipGraphDestroy(graph)
    return int(n.value)


@pytest.mark.parametrize("name,M", [("wq_a+wkv_m1", 1), ("wq_a+wkv_m2_8", 2),
                                     ("wq_a+wkv_m2_8", 8), ("fused_a_3way", 4),
                                     ("indexer_f32", 8), ("crossover", 9),
                                     ("crossover", 32), ("crossover", 64)])
def test_launch_count_fused_one_separate_n(name, M):
    """The pages count tinygemm2 calls per token count; here the fused call
    is one kernel node (two where its split-K slices are added by a second
    launch, as its tiling says) and the separate path as many per
    projection; the graph holds exactly what fp_plan_query reports."""
    x0, ws = si.workload_case(name, M, 0)
    fp = P.FusedProjection([to_gpu(w) for w in ws], max_M=max(8, M))
    x = to_gpu(x0)
    outs = [torch.empty(M, n, dtype=x.dtype, device="cuda") for n in fp.N]
    fp(x, out=outs)
    fp.forward_separate(x, out=outs)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        n_fused = _count_graph_nodes(lambda: fp(x, out=outs, stream=s), s)
        n_sep = _count_graph_nodes(lambda: fp.forward_separate(x, out=outs, stream=s), s)
    torch.cuda.synchronize()
    path, lf, ls = fp.query(M)
    t = fp.get_tiling(M)
    per_call = 2 if (t[0] == P.FP_PATH_MFMA and t[3] > 1 and t[5] == 2) else 1
    assert (n_fused, n_sep) == (lf, ls) == (per_call, per_call * len(fp.N))


def test_replay_of_a_split_vector_alu_launch():
    """The vector-ALU kernel's in-launch split-K finish under replay: the
    fp32 indexer fusion with its K split across 4 workgroups (partials in
    the workspace, the last workgroup adds them), three new inputs and a
    300-replay stress, each replay against an eager call."""
    M = 8
    split = (P.FP_PATH_SKINNY_SPLITK, 7, 1, 4, 0, 0)
    x0, ws = si.workload_case("indexer_f32", M, 0)
    fp = P.FusedProjection([to_gpu(w) for w in ws], max_M=M, workspace_bytes=1 << 20)
    assert fp.set_tiling(M, split) == P.FP_OK
    assert fp.query(M)[0] == P.FP_PATH_SKINNY_SPLITK
    x_static = to_gpu(x0)
    outs = [torch.empty(M, n, dtype=x_static.dtype, device="cuda") for n in fp.N]
    g = _capture(fp, x_static, outs)
    for seed in (21, 22, 23):
        xn, _ = si.workload_case("indexer_f32", M, seed)
        x_static.copy_(to_gpu(xn))
        g.replay()
        torch.cuda.synchronize()
        eager = fp(x_static)
        assert_bitwise_equal(outs, eager, "split replay seed %d" % seed)
        assert_matches_oracle(outs, xn, ws, label="split replay")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(4321)
    mismatches = 0
    for _ in range(300):
        x_static.copy_(torch.randn(x_static.shape, generator=gen, device="cuda"))
        g.replay()
        eager = fp(x_static)
        torch.cuda.synchronize()
        for a, b in zip(outs, eager):
            mismatches += int(not torch.equal(a.view(torch.int32), b.view(torch.int32)))
    assert mismatches == 0
    fp.set_tiling(M, None)
