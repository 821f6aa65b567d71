"""Parity of the fused epilogues (through the C ABI) with the CPU oracle.

RMSNorm after the projection: q_norm over the q_a columns and kv_norm over
the kv columns that consume the fused wq_a/wkv projection ("tinygemm2 for
the DeepSeek-V4.1 hidden-state projections", TensorRT-LLM PR #20636,
Description).  SwiGLU of a row-concatenated gate/up pair, gate and up
rounded to bf16 first (dense-MLP commit of "Staircase: GLM-5.2 NVFP4
low-latency decode target for Rubin (TP16)", PR #20502).

Every element is compared with the oracle's unrounded fp64 result under the
derived bounds (``oracle.rmsnorm_bound`` / ``oracle.swiglu_bound``, pinned on
the CPU); the fused call (RMSNorm: the fused projection and one
normalisation launch; SwiGLU: one launch over gate/up row pairs) must be
bitwise equal to the unfused chain (one projection launch per projection,
then the standalone RMSNorm / SwiGLU kernel), to a repeat, and to graph
replays.  Exact-sum data (every fp32
partial sum exact) tightens the bounds to the rounding of the epilogue
alone.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
import projection_gemm_sparse_amd as P
from gpu_util import assert_bitwise_equal, out_bits, to_gpu

pytestmark = pytest.mark.gpu

EPS = float(np.float32(1e-6))


def _f64(t):
    return oracle.bf16_bits_to_f64(si.bits(t.cpu()))


def _check_norm(outs, x_cpu, ws, gammas, label, exact_sums=False):
    res = oracle.fused_rmsnorm(si.bits(x_cpu), [si.bits(w) for w in ws],
                               [None if g is None else si.bits(g) for g in gammas], EPS)
    torch.cuda.synchronize()
    for i, (o, r, g) in enumerate(zip(outs, res, gammas)):
        got = _f64(o)
        if g is None:
            ok, worst, idx = oracle.check_within_bound(got, r["y"], r["S"], oracle.BF16)
        else:
            bound = oracle.rmsnorm_bound(r, si.bits(g), EPS, exact_sums=exact_sums)
            ok, worst, idx = oracle.check_against(got, r["out"], bound)
        assert ok, "%s proj %d: worst |err|/bound %.3g at %s" % (label, i, worst, idx)


def _check_swiglu(h, x_cpu, ws, label, exact_sums=False):
    r = oracle.fused_swiglu(si.bits(x_cpu), si.bits(ws[0]), si.bits(ws[1]))
    torch.cuda.synchronize()
    ok, worst, idx = oracle.check_against(_f64(h), r["h"], oracle.swiglu_bound(r, exact_sums))
    assert ok, "%s: worst |err|/bound %.3g at %s" % (label, worst, idx)


# ------------------------------------------------------------------ RMSNorm
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("seed", [0, 1])
def test_rmsnorm_q_kv(M, seed):
    x, ws, gammas = si.norm_case(M, seed)
    fp = P.FusedProjection([to_gpu(w) for w in ws], max_M=8)
    xg = to_gpu(x)
    gg = [to_gpu(g) for g in gammas]
    outs = fp.forward_rmsnorm(xg, gg, EPS)
    _check_norm(outs, x, ws, gammas, "q_kv_norm M=%d seed=%d" % (M, seed))
    again = fp.forward_rmsnorm(xg, gg, EPS)
    assert_bitwise_equal(outs, again, "repeat")
    chain = fp.forward_rmsnorm_separate(xg, gg, EPS)
    assert_bitwise_equal(outs, chain, "fused vs unfused chain")


@pytest.mark.parametrize("M", [1, 5, 8])
def test_rmsnorm_one_projection_left_plain(M):
    x, ws, gammas = si.norm_case(M, 3)
    fp = P.FusedProjection([to_gpu(w) for w in ws], max_M=8)
    xg = to_gpu(x)
    outs = fp.forward_rmsnorm(xg, [to_gpu(gammas[0]), None], EPS)
    _check_norm(outs, x, ws, [gammas[0], None], "q only M=%d" % M)
    plain = fp(xg)
    assert_bitwise_equal([outs[1]], [plain[1]], "un-normalised projection = plain call")


@pytest.mark.parametrize("M", [1, 4, 8])
def test_rmsnorm_exact_sums(M):
    # every fp32 partial sum exact: the GPU's bf16 projection is RNE(exact)
    x, ws = si.sparse_int_case(5120, (1280, 512), M, 21)
    g = torch.Generator().manual_seed(21)
    gammas = [(1.0 + 0.1 * torch.randn(n, generator=g)).to(torch.bfloat16) for n in (1280, 512)]
    fp = P.FusedProjection([to_gpu(w) for w in ws], max_M=8)
    outs = fp.forward_rmsnorm(to_gpu(x), [to_gpu(t) for t in gammas], EPS)
    _check_norm(outs, x, ws, gammas, "exact sums M=%d" % M, exact_sums=True)


@pytest.mark.parametrize("M", [1, 4, 8])
def test_rmsnorm_three_way(M):
    x, ws = si.workload_case("fused_a_3way", M, 0)
    g = torch.Generator().manual_seed(5)
    gammas = [(1.0 + 0.1 * torch.randn(int(w.shape[0]), generator=g)).to(torch.bfloat16)
              for w in ws]
    fp = P.FusedProjection([to_gpu(w) for w in ws], max_M=8)
    xg = to_gpu(x)
    gg = [to_gpu(t) for t in gammas]
    outs = fp.forward_rmsnorm(xg, gg, EPS)
    _check_norm(outs, x, ws, gammas, "3-way M=%d" % M)
    assert_bitwise_equal(outs, fp.forward_rmsnorm_separate(xg, gg, EPS), "3-way chain")


def test_rmsnorm_strided_x():
    M = 4
    x, ws, gammas = si.norm_case(M, 0, ldx=5120 + 64)
    fp = P.FusedProjection([to_gpu(w) for w in ws], max_M=8)
    xg = to_gpu(x)[:, :5120]
    outs = fp.forward_rmsnorm(xg, [to_gpu(g) for g in gammas], EPS)
    _check_norm(outs, x[:, :5120].contiguous(), ws, gammas, "strided x")


def test_rmsnorm_graph_replay_equals_eager():
    M = 8
    x0, ws, gammas = si.norm_case(M, 0)
    fp = P.FusedProjection([to_gpu(w) for w in ws], max_M=8)
    gg = [to_gpu(g) for g in gammas]
    x_static = to_gpu(x0)
    outs = [torch.empty(M, n, dtype=torch.bfloat16, device="cuda") for n in fp.N]
    fp.forward_rmsnorm(x_static, gg, EPS, out=outs)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fp.forward_rmsnorm(x_static, gg, EPS, out=outs)
    torch.cuda.synchronize()
    for seed in (11, 12, 13):
        xn, _, _ = si.norm_case(M, seed)
        x_static.copy_(to_gpu(xn))
        graph.replay()
        torch.cuda.synchronize()
        eager = fp.forward_rmsnorm(x_static, gg, EPS)
        assert_bitwise_equal(outs, eager, "replay seed %d" % seed)
        _check_norm(outs, xn, ws, gammas, "replay seed %d" % seed)


def test_standalone_rmsnorm_in_place_and_bounds():
    M, N = 3, 1280
    g = torch.Generator().manual_seed(8)
    v = (torch.randn(M, N, generator=g) * 0.7).to(torch.bfloat16)
    gamma = (1.0 + 0.1 * torch.randn(N, generator=g)).to(torch.bfloat16)
    vg, gg = to_gpu(v), to_gpu(gamma)
    out = torch.empty_like(vg)
    st = P.fp_rmsnorm(vg.data_ptr(), M, N, gg.data_ptr(), EPS, out.data_ptr(), 0)
    assert st == P.FP_OK
    inplace = vg.clone()
    st = P.fp_rmsnorm(inplace.data_ptr(), M, N, gg.data_ptr(), EPS, inplace.data_ptr(), 0)
    assert st == P.FP_OK
    assert_bitwise_equal([out], [inplace], "in place")
    want, rinv = oracle.rmsnorm(si.bits(v), si.bits(gamma), EPS)
    # input exactly bf16: only the fp32 steps and the output rounding count
    r = {"y": oracle.bf16_bits_to_f64(si.bits(v)), "S": np.zeros((M, N)),
         "yb": si.bits(v), "out": want, "rinv": rinv}
    bound = oracle.rmsnorm_bound(r, si.bits(gamma), EPS, exact_sums=True)
    ok, worst, idx = oracle.check_against(_f64(out), want, bound)
    assert ok, (worst, idx)


@pytest.mark.parametrize("M", [9, 16])
def test_rmsnorm_beyond_eight_tokens(M):
    # the projection runs on the tile kernel, the normalisation launch is the same
    x, ws = si.workload_case("crossover", M, 0)
    g = torch.Generator().manual_seed(9)
    gammas = [(1.0 + 0.1 * torch.randn(n, generator=g)).to(torch.bfloat16) for n in (1280, 512)]
    fp = P.FusedProjection([to_gpu(w) for w in ws], max_M=16)
    xg = to_gpu(x)
    gg = [to_gpu(t) for t in gammas]
    outs = fp.forward_rmsnorm(xg, gg, EPS)
    _check_norm(outs, x, ws, gammas, "M=%d" % M)
    assert_bitwise_equal(outs, fp.forward_rmsnorm_separate(xg, gg, EPS), "chain M=%d" % M)


def test_rmsnorm_refusals():
    x, ws, gammas = si.norm_case(8, 0)
    fp = P.FusedProjection([to_gpu(w) for w in ws], max_M=16)
    g_dev = [to_gpu(g) for g in gammas]  # kept alive while their addresses are used
    gp = [g.data_ptr() for g in g_dev]
    x16 = to_gpu(si.workload_case("crossover", 16, 0)[0])
    outs = [torch.empty(16, n, dtype=torch.bfloat16, device="cuda") for n in fp.N]
    st = P.fp_forward_rmsnorm(x16.data_ptr(), 17, 5120, fp.plan, 0, gp, EPS,
                              [o.data_ptr() for o in outs])
    assert st == P.FP_ERR_UNSUPPORTED  # above the plan's max_M
    st = P.fp_forward_rmsnorm(x16.data_ptr(), 4, 5120, fp.plan, 0, gp, -1.0,
                              [o.data_ptr() for o in outs])
    assert st == P.FP_ERR_INVALID_ARG  # negative eps
    st = P.fp_rmsnorm(outs[0].data_ptr(), 2, 1284, gp[0], EPS, outs[1].data_ptr(), 0)
    assert st == P.FP_ERR_UNSUPPORTED  # width not a multiple of 8
    st = P.fp_rmsnorm(outs[0].data_ptr(), 2, 1280, gp[0], EPS, outs[0].data_ptr() + 16, 0)
    assert st == P.FP_ERR_INVALID_ARG  # partial overlap
    # an output overlapping a gain
    g_big = torch.empty(4 * 1280, dtype=torch.bfloat16, device="cuda")
    st = P.fp_forward_rmsnorm(x16.data_ptr(), 2, 5120, fp.plan, 0,
                              [g_big.data_ptr(), None], EPS,
                              [g_big.data_ptr() + 1280, outs[1].data_ptr()])  # inside the gain's 2560 bytes
    assert st == P.FP_ERR_INVALID_ARG
    torch.cuda.synchronize()


# ------------------------------------------------------------------- SwiGLU
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("seed", [0, 1])
def test_swiglu_gate_up(M, seed):
    x, ws = si.workload_case("gate_up_swiglu", M, seed)
    fp = P.FusedProjection([to_gpu(w) for w in ws], max_M=8)
    xg = to_gpu(x)
    h = fp.forward_swiglu(xg)
    _check_swiglu(h, x, ws, "gate/up M=%d seed=%d" % (M, seed))
    assert_bitwise_equal([h], [fp.forward_swiglu(xg)], "repeat")
    assert_bitwise_equal([h], [fp.forward_swiglu_separate(xg)], "fused vs unfused chain")


@pytest.mark.parametrize("M", [1, 8])
def test_swiglu_exact_sums(M):
    x, ws = si.sparse_int_case(6144, (768, 768), M, 31)
    fp = P.FusedProjection([to_gpu(w) for w in ws], max_M=8)
    h = fp.forward_swiglu(to_gpu(x))
    _check_swiglu(h, x, ws, "exact sums M=%d" % M, exact_sums=True)


def test_swiglu_graph_replay_equals_eager():
    M = 4
    x0, ws = si.workload_case("gate_up_swiglu", M, 0)
    fp = P.FusedProjection([to_gpu(w) for w in ws], max_M=8)
    x_static = to_gpu(x0)
    h = torch.empty(M, 768, dtype=torch.bfloat16, device="cuda")
    fp.forward_swiglu(x_static, out=h)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fp.forward_swiglu(x_static, out=h)
    torch.cuda.synchronize()
    for seed in (11, 12, 13):
        xn, _ = si.workload_case("gate_up_swiglu", M, seed)
        x_static.copy_(to_gpu(xn))
        graph.replay()
        torch.cuda.synchronize()
        assert_bitwise_equal([h], [fp.forward_swiglu(x_static)], "replay seed %d" % seed)
        _check_swiglu(h, xn, ws, "replay seed %d" % seed)


def test_swiglu_refusals():
    x, ws = si.workload_case("wq_a+wkv_m1", 1, 0)
    fp = P.FusedProjection([to_gpu(w) for w in ws], max_M=8)
    h = torch.empty(1, 1280, dtype=torch.bfloat16, device="cuda")
    # unequal widths: not a gate/up pair
    st = P.fp_forward_swiglu(to_gpu(x).data_ptr(), 1, 5120, fp.plan, 0, h.data_ptr())
    assert st == P.FP_ERR_INVALID_ARG
    a = torch.zeros(2, 16, dtype=torch.bfloat16, device="cuda")
    st = P.fp_swiglu(a.data_ptr(), a.data_ptr(), 2, 12, a.data_ptr(), 0)
    assert st == P.FP_ERR_UNSUPPORTED
    torch.cuda.synchronize()


def test_epilogue_launch_counts():
    """RMSNorm: the projection launch plus one normalisation launch for all
    normalised projections; SwiGLU: one launch."""
    from test_graph_gpu import _count_graph_nodes
    x, ws, gammas = si.norm_case(2, 0)
    fp = P.FusedProjection([to_gpu(w) for w in ws], max_M=8)
    xg = to_gpu(x)
    gg = [to_gpu(g) for g in gammas]
    outs = [torch.empty(2, n, dtype=torch.bfloat16, device="cuda") for n in fp.N]
    fp.forward_rmsnorm(xg, gg, EPS, out=outs)
    xs, wsw = si.workload_case("gate_up_swiglu", 2, 0)
    fs = P.FusedProjection([to_gpu(w) for w in wsw], max_M=8)
    xsg = to_gpu(xs)
    h = torch.empty(2, 768, dtype=torch.bfloat16, device="cuda")
    fs.forward_swiglu(xsg, out=h)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        n_norm = _count_graph_nodes(lambda: fp.forward_rmsnorm(xg, gg, EPS, out=outs, stream=s), s)
        n_swiglu = _count_graph_nodes(lambda: fs.forward_swiglu(xsg, out=h, stream=s), s)
    torch.cuda.synchronize()
    assert (n_norm, n_swiglu) == (2, 1)


def _random_epilogue_cases(n, seed, max_m, max_n):
    """Seeded (K, N, M): K a multiple of 8 from 64 to 8192, N a multiple of 8
    from 8 to max_n, at most 12M weight elements per projection pair."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        K = 8 * int(round(np.exp(rng.uniform(np.log(8.0), np.log(1024.0)))))
        N = 8 * int(round(np.exp(rng.uniform(0.0, np.log(max_n / 8.0)))))
        if 2 * N * K > 12_000_000:
            continue
        out.append((K, N, int(rng.integers(1, max_m + 1))))
    return out


@pytest.mark.parametrize("K,N,M", _random_epilogue_cases(16, 3, 8, 4096))
def test_swiglu_on_random_shapes(K, N, M):
    x, ws = si.make_case(K, (N, N), "bf16", M, seed=K + N + M)
    fp = P.FusedProjection([to_gpu(w) for w in ws], max_M=8)
    xg = to_gpu(x)
    h = fp.forward_swiglu(xg)
    _check_swiglu(h, x, ws, "gate/up K=%d N=%d M=%d" % (K, N, M))
    assert_bitwise_equal([h], [fp.forward_swiglu_separate(xg)], "fused vs unfused chain")


@pytest.mark.parametrize("K,N,M", _random_epilogue_cases(16, 4, 16, 2048))
def test_rmsnorm_on_random_shapes(K, N, M):
    # two projections, the first normalised (at most 2048 wide, the widest
    # normalised row), the second (N + 8 rows) plain
    x, ws = si.make_case(K, (N, N + 8), "bf16", M, seed=K + N + M)
    g = torch.Generator().manual_seed(K + N)
    gammas = [(1.0 + 0.1 * torch.randn(N, generator=g)).to(torch.bfloat16), None]
    fp = P.FusedProjection([to_gpu(w) for w in ws], max_M=16)
    xg = to_gpu(x)
    gg = [to_gpu(gammas[0]), None]
    outs = fp.forward_rmsnorm(xg, gg, EPS)
    _check_norm(outs, x, ws, gammas, "K=%d N=%d M=%d" % (K, N, M))
    assert_bitwise_equal(outs, fp.forward_rmsnorm_separate(xg, gg, EPS), "chain")
