"""Parity of the fp32-output router GEMV (through the C ABI) with the oracle.

Router commit of "Staircase: GLM-5.2 NVFP4 low-latency decode target for
Rubin (TP16)" (TensorRT-LLM PR #20502): 256 expert logits at hidden 6144
from bf16 operands, kept in fp32, checked against an FP64 reference, with a
fixed summation order.  Here: a bf16 plan set to fp32 outputs, M = 1..16,
every logit compared with the oracle's fp64 sum under the fp32 rule
(|err| <= 1e-5 * S + 1e-7); repeats and graph replays bitwise equal; exact
data bit exact.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
import projection_gemm_sparse_amd as P
from gpu_util import assert_bitwise_equal, out_bits, to_gpu

pytestmark = pytest.mark.gpu


def _router(ws, max_M=16):
    return P.FusedProjection([to_gpu(w) for w in ws], max_M=max_M, out_dtype=torch.float32)


def _check(ys, x_cpu, ws, label):
    torch.cuda.synchronize()
    for i, (y, w) in enumerate(zip(ys, ws)):
        assert y.dtype == torch.float32
        ref, s = oracle.linear(si.bits(x_cpu), si.bits(w))
        got = oracle.f32_bits_to_f64(si.bits(y.cpu()))
        ok, worst, idx = oracle.check_within_bound(got, ref, s, oracle.F32)
        assert ok, "%s proj %d: worst |err|/bound %.3g at %s" % (label, i, worst, idx)


@pytest.mark.parametrize("M", list(range(1, 17)))
@pytest.mark.parametrize("seed", [0, 1])
def test_router_logits(M, seed):
    x, ws = si.workload_case("router_f32out", M, seed)
    fp = _router(ws)
    xg = to_gpu(x)
    ys = fp(xg)
    _check(ys, x, ws, "router M=%d seed=%d" % (M, seed))
    assert_bitwise_equal(ys, fp(xg), "repeat")
    assert_bitwise_equal(ys, fp.forward_separate(xg), "fused vs separate")
    assert fp.query(M)[0] in (P.FP_PATH_SKINNY, P.FP_PATH_SKINNY_SPLITK)


@pytest.mark.parametrize("M", [1, 9, 16])
def test_router_exact_data_bit_exact(M):
    # every fp32 partial sum exact: the logits equal the exact sums bit for bit
    x, ws = si.sparse_int_case(6144, (256,), M, 41, nnz=64)
    fp = _router(ws)
    ys = fp(to_gpu(x))
    torch.cuda.synchronize()
    ref, _ = oracle.linear(si.bits(x), si.bits(ws[0]))
    got = oracle.f32_bits_to_f64(si.bits(ys[0].cpu()))
    assert np.array_equal(got, ref)


def test_router_two_projections_and_strided_x():
    # the same variant fuses more than one fp32-output projection, x strided
    M = 12
    x, ws = si.make_case(6144, (256, 64), "bf16", M, 3, ldx=6144 + 64)
    fp = _router(ws)
    ys = fp(to_gpu(x)[:, :6144])
    _check(ys, x[:, :6144].contiguous(), ws, "two projections")
    assert_bitwise_equal(ys, fp.forward_separate(to_gpu(x)[:, :6144]), "fused vs separate")


def test_router_graph_replay_equals_eager():
    M = 16
    x0, ws = si.workload_case("router_f32out", M, 0)
    fp = _router(ws)
    x_static = to_gpu(x0)
    outs = [torch.empty(M, 256, dtype=torch.float32, device="cuda")]
    fp(x_static, out=outs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp(x_static, out=outs)
    torch.cuda.synchronize()
    for seed in (11, 12, 13):
        xn, _ = si.workload_case("router_f32out", M, seed)
        x_static.copy_(to_gpu(xn))
        g.replay()
        torch.cuda.synchronize()
        assert_bitwise_equal(outs, fp(x_static), "replay seed %d" % seed)
        _check(outs, xn, ws, "replay seed %d" % seed)


def test_router_refusals():
    x, ws = si.workload_case("router_f32out", 1, 0)
    fp = _router(ws, max_M=32)
    x32 = to_gpu(si.workload_case("router_f32out", 17, 0)[0])
    assert fp.supported(x32) is False  # above 16 tokens
    st = P.fp_plan_set_out_dtype(fp.plan, 7)
    assert st == P.FP_ERR_INVALID_ARG
    # no epilogue forms on an fp32-output plan
    g = torch.ones(256, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(1, 256, dtype=torch.float32, device="cuda")
    st = P.fp_forward_rmsnorm(to_gpu(x).data_ptr(), 1, 6144, fp.plan, 0, [g.data_ptr()], 1e-6,
                              [out.data_ptr()])
    assert st == P.FP_ERR_UNSUPPORTED
    # an fp32 plan cannot be switched to bf16 outputs
    xf, wf = si.workload_case("indexer_f32", 1, 0)
    f32 = P.FusedProjection([to_gpu(w) for w in wf], max_M=8)
    assert P.fp_plan_set_out_dtype(f32.plan, P.FP_BF16) == P.FP_ERR_UNSUPPORTED
    assert P.fp_plan_set_out_dtype(f32.plan, P.FP_F32) == P.FP_OK
    torch.cuda.synchronize()


@pytest.mark.parametrize("K", [10240, 16384])
@pytest.mark.parametrize("M", [9, 16])
def test_router_long_rows_split_k(K, M):
    """Past 8192 elements a row's 9..16-token workgroup would need more than
    8 K parts (its thread bound), so K is split across workgroups and the
    last to arrive adds the slices in slice order: every logit against the
    oracle under the fp32 rule, repeats, fused vs separate and graph replays
    bitwise equal."""
    x, ws = si.make_case(K, (256, 64), "bf16", M, seed=K + M)
    fp = _router(ws)
    assert fp.query(M)[0] == P.FP_PATH_SKINNY_SPLITK
    xg = to_gpu(x)
    ys = fp(xg)
    _check(ys, x, ws, "router K=%d M=%d" % (K, M))
    assert_bitwise_equal(ys, fp(xg), "repeat")
    assert_bitwise_equal(ys, fp.forward_separate(xg), "fused vs separate")
    outs = [torch.empty(M, n, dtype=torch.float32, device="cuda") for n in fp.N]
    fp(xg, out=outs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp(xg, out=outs)
    torch.cuda.synchronize()
    for seed in (1, 2):
        xn, _ = si.make_case(K, (256, 64), "bf16", M, seed=K + M + 100 * seed)
        xg.copy_(to_gpu(xn))
        g.replay()
        torch.cuda.synchronize()
        assert_bitwise_equal(outs, fp(xg), "replay %d" % seed)
        _check(outs, xn, ws, "router K=%d M=%d replay" % (K, M))


def _random_router_cases(n, seed):
    """Seeded router shapes: K a multiple of 8 from 64 to 16384, one or two
    projections of 1..4096 rows (at most 16M weight elements), M 1..16."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        K = 8 * int(round(np.exp(rng.uniform(np.log(8.0), np.log(2048.0)))))
        N = tuple(int(round(np.exp(rng.uniform(0.0, np.log(4096.0)))))
                  for _ in range(int(rng.integers(1, 3))))
        if sum(N) * K > 16_000_000:
            continue
        out.append((K, N, int(rng.integers(1, 17))))
    return out


@pytest.mark.parametrize("K,N,M", _random_router_cases(24, 5))
def test_router_on_random_shapes(K, N, M):
    """Every router shape is served (no row layout without a compiled
    kernel, no slice past the thread bound) and matches the oracle."""
    x, ws = si.make_case(K, N, "bf16", M, seed=K + 7 * M)
    fp = _router(ws)
    xg = to_gpu(x)
    assert fp.supported(xg), (K, N, M, fp.get_tiling(M))
    ys = fp(xg)
    _check(ys, x, ws, "router K=%d N=%s M=%d %s" % (K, N, M, fp.get_tiling(M)))
    assert_bitwise_equal(ys, fp.forward_separate(xg), "fused vs separate")


@pytest.mark.parametrize("M", [1, 8, 16])
def test_router_on_the_fused_wq_a_wkv_shape(M):
    """fp32 outputs over [1280, 512] x 5120: the cheapest row layout (7 rows
    per workgroup up to 8 tokens) has no compiled fp32-output kernel, so the
    search keeps to those that exist (these calls were refused before)."""
    x, ws = si.workload_case("crossover", M, 3)
    fp = _router(ws)
    xg = to_gpu(x)
    assert fp.supported(xg)
    assert fp.get_tiling(M)[4] in (1, 2, 4, 8)
    ys = fp(xg)
    _check(ys, x, ws, "router wq_a+wkv M=%d" % M)
    assert_bitwise_equal(ys, fp.forward_separate(xg), "fused vs separate")
