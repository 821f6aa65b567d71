"""Parity of the NVFP4-weight projection (through the C ABI) with the oracle.

The pages' FP4 fused weight is an NVFP4 checkpoint ("Fuse QK down_proj with
indexer K + weight_proj for FP4 ckpt", PR #8771, first titled as NVFP4
only; the GLM-5.2 NVFP4 target of PR #20502), read as the public two-level
NVFP4 format: E2M1 codes two per byte (low nibble first), one E4M3 scale
per 16 elements, one fp32 scale per projection; packed rows of K/2 code
bytes then K/16 scales.  Each weight decodes exactly (E2M1 x E4M3 has at
most 6 significant bits) and each output's fp32 sum is multiplied by its
projection's tensor scale before the single rounding to bf16.

Checked: the dequantiser on all 256 code bytes at several E4M3 scales
(powers of two and not) and tensor scales against the exact values; every
projection element against the oracle's fp64 sum under the bf16 rule at
M = 1..8 (vector-ALU and matrix-core kernels, opt-in and default tilings)
with a different non-power-of-two tensor scale per projection; exact data
bit exact; three projections with strided x and reload; repeats, fused vs
one launch per projection and graph replays bitwise equal; RMSNorm on the
outputs; refusals.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
import projection_gemm_sparse_amd as P
from gpu_util import assert_bitwise_equal, to_gpu

pytestmark = pytest.mark.gpu

E4M3_SCALES = (0x38, 0x3C, 0x2B, 0x47, 0x01, 0x5E)  # 1, 1.5, 0.34375, 3.75, 2^-9, 28


def _plan(ws, gs, max_M=8):
    return P.FusedProjection([to_gpu(w) for w in ws], max_M=max_M, weight_format="nvfp4",
                             tensor_scales=gs)


def _small_tiling(K):
    steps = K // 64
    kt = 4 if steps <= 64 else 8 if steps <= 128 else 16
    return (P.FP_PATH_MFMA_SMALL, -(-steps // kt), kt, 1, 0, 0)


def _check(ys, x_cpu, ws, gs, K, label):
    torch.cuda.synchronize()
    for i, (y, w, g) in enumerate(zip(ys, ws, gs)):
        ref, s = oracle.linear_nvfp4(si.bits(x_cpu), si.bits(w), K, g)
        got = oracle.bf16_bits_to_f64(si.bits(y.cpu()))
        ok, worst, idx = oracle.check_within_bound(got, ref, s, oracle.BF16)
        assert ok, "%s proj %d: worst |err|/bound %.3g at %s" % (label, i, worst, idx)


def _bf16_bits_of_f32(v):
    """bf16 pattern of float32 value v, rounded to nearest even."""
    b = int(np.array([v], dtype=np.float32).view(np.uint32)[0])
    return ((b + 0x7FFF + ((b >> 16) & 1)) >> 16) & 0xFFFF


@pytest.mark.parametrize("g", [1.0, 0.013903140090405941, -2.5])
def test_dequantiser_all_code_bytes(g):
    K = 512
    rows = []
    for s in E4M3_SCALES:
        codes = np.tile(np.arange(256, dtype=np.uint8), K // 2 // 256)
        rows.append(np.concatenate([codes, np.full(K // 16, s, dtype=np.uint8)]))
    w = to_gpu(torch.from_numpy(np.stack(rows)))
    out = torch.empty(len(E4M3_SCALES), K, dtype=torch.bfloat16, device="cuda")
    assert P.fp_nvfp4_to_bf16(w.data_ptr(), len(E4M3_SCALES), K, g, out.data_ptr(), 0) == P.FP_OK
    torch.cuda.synchronize()
    got = si.bits(out.cpu())
    gf = np.float32(g)
    for r, s in enumerate(E4M3_SCALES):
        for k in range(K):  # all 256 code bytes, both nibbles
            byte = (k // 2) % 256
            code = (byte >> 4) if k % 2 else (byte & 0xF)
            exact = oracle.e2m1_value(code) * oracle.e4m3_value(s)
            assert float(np.float32(exact)) == exact  # E2M1 x E4M3 is exact in fp32
            want = _bf16_bits_of_f32(np.float32(exact) * gf)
            assert got[r, k] == want, "byte %02x k %d scale %02x g %r: got %04x want %04x" % (
                byte, k, s, g, got[r, k], want)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8, 9, 16])
def test_nvfp4_wq_a_wkv(M):
    x, ws, gs = si.nvfp4_case(M, 30 + M)
    fp = _plan(ws, gs, max_M=16)
    xg = to_gpu(x)
    ys = fp(xg)
    _check(ys, x, ws, gs, 5120, "nvfp4 default M=%d" % M)
    assert_bitwise_equal(ys, fp(xg), "repeat")
    assert_bitwise_equal(ys, fp.forward_separate(xg), "fused vs separate")


@pytest.mark.parametrize("path", ["skinny", "mfma_small"])
@pytest.mark.parametrize("M", [1, 4, 8])
def test_nvfp4_both_kernels(path, M):
    x, ws, gs = si.nvfp4_case(M, 50 + M)
    fp = _plan(ws, gs)
    t = (P.FP_PATH_SKINNY, 10, 1, 1, 0, 0) if path == "skinny" else _small_tiling(5120)
    assert fp.set_tiling(M, t) == P.FP_OK
    assert fp.query(M)[0] == (P.FP_PATH_SKINNY if path == "skinny" else P.FP_PATH_MFMA_SMALL)
    xg = to_gpu(x)
    ys = fp(xg)
    _check(ys, x, ws, gs, 5120, "nvfp4 %s M=%d" % (path, M))
    assert_bitwise_equal(ys, fp.forward_separate(xg), "fused vs separate")


@pytest.mark.parametrize("M", [1, 8])
def test_nvfp4_exact_data_bit_exact(M):
    # codes +-1/2, +-1, +-2 on sparse rows, block scales 1 and 2, tensor
    # scales 0.5 and 0.25: every product and fp32 partial sum exact, so the
    # outputs are RNE(exact sum)
    K, N, gs = 5120, (1280, 512), [0.5, 0.25]
    g = torch.Generator().manual_seed(29)
    ws = []
    for n in N:
        keep = torch.rand(n, K, generator=g) < 0.02
        nib = torch.tensor([0x1, 0x2, 0x4, 0x9, 0xA, 0xC], dtype=torch.int64)
        pick = nib[torch.randint(0, 6, (n, K), generator=g)]
        pick = torch.where(keep, pick, torch.zeros_like(pick))
        packed = pick[:, 0::2] | (pick[:, 1::2] << 4)
        sc = torch.tensor([0x38, 0x40], dtype=torch.int64)[torch.randint(0, 2, (n, K // 16),
                                                                          generator=g)]
        ws.append(torch.cat([packed, sc], 1).to(torch.uint8))
    x = (torch.randint(-255, 256, (M, K), generator=g).to(torch.float32) / 64).to(torch.bfloat16)
    for t in (None, _small_tiling(K)):
        fp = _plan(ws, gs)
        if t is not None:
            assert fp.set_tiling(M, t) == P.FP_OK
        ys = fp(to_gpu(x))
        torch.cuda.synchronize()
        for y, w, gg in zip(ys, ws, gs):
            ref, _ = oracle.linear_nvfp4(si.bits(x), si.bits(w), K, gg)
            assert np.array_equal(si.bits(y.cpu()), oracle.round_bf16(ref)), (M, t)


def test_nvfp4_three_way_strided_x_and_reload():
    K, N, M = 6144, (2048, 576, 128), 6
    x, ws, gs = si.nvfp4_case(M, 61, K=K, N=N, ldx=K + 64)
    fp = _plan(ws, gs)
    xg = to_gpu(x)[:, :K]
    ys = fp(xg)
    _check(ys, x[:, :K].contiguous(), ws, gs, K, "3-way")
    _, ws2, _ = si.nvfp4_case(M, 62, K=K, N=N)
    for v, w in zip(fp.views, ws2):
        v.copy_(to_gpu(w))
    ys2 = fp(xg)
    _check(ys2, x[:, :K].contiguous(), ws2, gs, K, "after reload")
    assert_bitwise_equal(ys2, fp.forward_separate(xg), "fused vs separate after reload")


@pytest.mark.parametrize("M", [3, 8])
def test_nvfp4_graph_replay_equals_eager(M):
    x0, ws, gs = si.nvfp4_case(M, 70)
    fp = _plan(ws, gs)
    x_static = to_gpu(x0)
    outs = [torch.empty(M, n, dtype=torch.bfloat16, device="cuda") for n in fp.N]
    fp(x_static, out=outs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp(x_static, out=outs)
    torch.cuda.synchronize()
    for seed in (71, 72, 73):
        xn, _, _ = si.nvfp4_case(M, seed)
        x_static.copy_(to_gpu(xn))
        g.replay()
        torch.cuda.synchronize()
        assert_bitwise_equal(outs, fp(x_static), "replay seed %d" % seed)
        _check(outs, xn, ws, gs, 5120, "replay seed %d" % seed)


@pytest.mark.parametrize("M", [4, 8])
def test_nvfp4_rmsnorm_epilogue(M):
    x, ws, gs = si.nvfp4_case(M, 80)
    gen = torch.Generator().manual_seed(80)
    gammas = [(1.0 + 0.1 * torch.randn(n, generator=gen)).to(torch.bfloat16) for n in (1280, 512)]
    fp = _plan(ws, gs)
    xg = to_gpu(x)
    gg = [to_gpu(t) for t in gammas]
    outs = fp.forward_rmsnorm(xg, gg, 1e-6)
    assert_bitwise_equal(outs, fp.forward_rmsnorm_separate(xg, gg, 1e-6), "chain")
    torch.cuda.synchronize()
    eps = float(np.float32(1e-6))
    for o, w, gm, g in zip(outs, ws, gammas, gs):
        y, s = oracle.linear_nvfp4(si.bits(x), si.bits(w), 5120, g)
        yb = oracle.round_bf16(y)
        out, rinv = oracle.rmsnorm(yb, si.bits(gm), eps)
        r = {"y": y, "S": s, "yb": yb, "out": out, "rinv": rinv}
        bound = oracle.rmsnorm_bound(r, si.bits(gm), eps)
        ok, worst, idx = oracle.check_against(oracle.bf16_bits_to_f64(si.bits(o.cpu())), out,
                                              bound)
        assert ok, (worst, idx)


def test_nvfp4_refusals():
    x, ws, gs = si.nvfp4_case(1, 0)
    fp = _plan(ws, gs, max_M=32)
    assert fp.supported(to_gpu(si.nvfp4_case(17, 0)[0])) is False  # above 16 tokens
    assert P.fp_plan_set_tensor_scales(fp.plan, [1.0, float("inf")]) == P.FP_ERR_INVALID_ARG
    assert P.fp_plan_set_tensor_scales(fp.plan, None) == P.FP_ERR_INVALID_ARG
    assert P.fp_plan_set_out_dtype(fp.plan, P.FP_F32) == P.FP_ERR_UNSUPPORTED
    # tensor scales belong to NVFP4 plans only
    xb, wb = si.workload_case("wq_a+wkv_m1", 1, 0)
    bf = P.FusedProjection([to_gpu(w) for w in wb], max_M=8)
    assert P.fp_plan_set_tensor_scales(bf.plan, [1.0, 1.0]) == P.FP_ERR_UNSUPPORTED
    # the refused calls changed nothing: results still match the scales given
    ys = fp(to_gpu(x))
    _check(ys, x, ws, gs, 5120, "after refusals")


@pytest.mark.parametrize("M", [9, 16])
def test_nvfp4_two_token_halves_at_k7168(M):
    # K = 7168: two token halves take sixteen K steps per wave (7 parts), as
    # eight steps would need more waves than their thread bound allows
    K = 7168
    x, ws, gs = si.nvfp4_case(M, 120 + M, K=K, N=(1536, 576))
    fp = _plan(ws, gs, max_M=16)
    assert fp.query(M)[0] == P.FP_PATH_MFMA_SMALL
    assert tuple(fp.get_tiling(M)[1:3]) == (7, 16)
    xg = to_gpu(x)
    ys = fp(xg)
    _check(ys, x, ws, gs, K, "nvfp4 K=7168 M=%d" % M)
    assert_bitwise_equal(ys, fp.forward_separate(xg), "fused vs separate")


@pytest.mark.parametrize("seed", range(8))
def test_nvfp4_default_routing_on_random_shapes(seed):
    rng = np.random.default_rng(900 + seed)
    while True:
        K = 512 * int(rng.integers(1, 17))
        N = tuple(int(round(np.exp(rng.uniform(0.0, np.log(3000.0)))))
                  for _ in range(int(rng.integers(1, 3))))
        if sum(N) * K <= 12_000_000:
            break
    M = int(rng.integers(1, 17))
    x, ws, gs = si.nvfp4_case(M, 130 + seed, K=K, N=N)
    fp = _plan(ws, gs, max_M=16)
    xg = to_gpu(x)
    assert fp.supported(xg), (K, N, M)
    ys = fp(xg)
    _check(ys, x, ws, gs, K, "nvfp4 K=%d N=%s M=%d %s" % (K, N, M, fp.get_tiling(M)))
    assert_bitwise_equal(ys, fp.forward_separate(xg), "fused vs separate")
