"""Parity of the matrix-core path for MX weights (through the C ABI) with
the oracle.

The MXFP8 / MXFP4 projections ("tinygemm2 for the DeepSeek-V4.1 hidden-state
projections", Description; "Fuse QK down_proj with indexer K + weight_proj
for FP4 ckpt", PR #8771), read as the open microscaling formats: packed rows
of codes then K/32 E8M0 scales.  The small-M matrix-core kernel decodes the
codes to bf16 in the registers that feed v_mfma_f32_16x16x32_bf16.

Checked, for both formats: every projection element against the oracle's
fp64 sum under the bf16 rule at M = 1..8 (opt-in tiling and the default),
on the DeepSeek shape, a three-way shape with strided x, ragged projections
and the shortest K; two token halves at M = 9..16; exact data bit exact;
repeats, fused vs one launch per projection and graph replays bitwise
equal; refusals above 16 tokens.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
import projection_gemm_sparse_amd as P
from gpu_util import assert_bitwise_equal, to_gpu

pytestmark = pytest.mark.gpu

CASES = {"mxfp8": (si.mxfp8_case, oracle.linear_mxfp8),
         "mxfp4": (si.mxfp4_case, oracle.linear_mxfp4)}


def _plan(ws, fmt, max_M=8):
    return P.FusedProjection([to_gpu(w) for w in ws], max_M=max_M, weight_format=fmt)


def _small_tiling(K):
    steps = K // 64          # MFMA steps of 64 k over K
    kt = 4 if steps <= 64 else 8 if steps <= 128 else 16
    return (P.FP_PATH_MFMA_SMALL, -(-steps // kt), kt, 1, 0, 0)


def _check(ys, x_cpu, ws, K, fmt, label):
    torch.cuda.synchronize()
    lin = CASES[fmt][1]
    for i, (y, w) in enumerate(zip(ys, ws)):
        ref, s = lin(si.bits(x_cpu), si.bits(w), K)
        got = oracle.bf16_bits_to_f64(si.bits(y.cpu()))
        ok, worst, idx = oracle.check_within_bound(got, ref, s, oracle.BF16)
        assert ok, "%s proj %d: worst |err|/bound %.3g at %s" % (label, i, worst, idx)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
def test_mx_small_mfma_wq_a_wkv(fmt, M):
    x, ws = CASES[fmt][0](M, 20 + M)
    fp = _plan(ws, fmt)
    assert fp.set_tiling(M, _small_tiling(5120)) == P.FP_OK
    assert fp.query(M)[0] == P.FP_PATH_MFMA_SMALL
    xg = to_gpu(x)
    ys = fp(xg)
    _check(ys, x, ws, 5120, fmt, "%s small-M MFMA M=%d" % (fmt, M))
    assert_bitwise_equal(ys, fp(xg), "repeat")
    assert_bitwise_equal(ys, fp.forward_separate(xg), "fused vs separate")


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("M", [1, 4, 5, 8])
def test_mx_default_path(fmt, M):
    x, ws = CASES[fmt][0](M, 40 + M)
    fp = _plan(ws, fmt)
    assert fp.query(M)[0] in (P.FP_PATH_SKINNY, P.FP_PATH_MFMA_SMALL)
    xg = to_gpu(x)
    ys = fp(xg)
    _check(ys, x, ws, 5120, fmt, "%s default M=%d" % (fmt, M))
    assert_bitwise_equal(ys, fp.forward_separate(xg), "fused vs separate")


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("shape", ["3way_strided", "ragged_k512", "k1024"])
def test_mx_small_mfma_shapes(fmt, shape):
    M = 6
    if shape == "3way_strided":
        K, N, ldx = 6144, (2048, 576, 128), 6144 + 64
    elif shape == "ragged_k512":
        K, N, ldx = 512, (37, 5, 70, 1), None
    else:
        K, N, ldx = 1024, (300, 29), None
    x, ws = CASES[fmt][0](M, 60, K=K, N=N, ldx=ldx)
    fp = _plan(ws, fmt)
    assert fp.set_tiling(M, _small_tiling(K)) == P.FP_OK
    xg = to_gpu(x)[:, :K]
    ys = fp(xg)
    _check(ys, x[:, :K].contiguous(), ws, K, fmt, "%s %s" % (fmt, shape))
    assert_bitwise_equal(ys, fp.forward_separate(xg), "fused vs separate")
    assert_bitwise_equal(ys, fp(xg.contiguous()), "strided vs contiguous x")


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("M", [5, 8])
def test_mx_small_mfma_exact_data(fmt, M):
    # weights of +-1/2, +-1, +-2 at scale 2^0 on sparse rows, x on a 1/64
    # grid: every product and fp32 partial sum exact, outputs = RNE(exact)
    K, N = 5120, (1280, 512)
    g = torch.Generator().manual_seed(23)
    ws = []
    for n in N:
        keep = torch.rand(n, K, generator=g) < 0.02
        if fmt == "mxfp8":
            codes = torch.tensor([0x30, 0x38, 0x40, 0xB0, 0xB8, 0xC0], dtype=torch.int64)
            pick = codes[torch.randint(0, 6, (n, K), generator=g)]
            pick = torch.where(keep, pick, torch.zeros_like(pick))
            packed = pick
        else:
            nib = torch.tensor([0x1, 0x2, 0x4, 0x9, 0xA, 0xC], dtype=torch.int64)
            pick = nib[torch.randint(0, 6, (n, K), generator=g)]
            pick = torch.where(keep, pick, torch.zeros_like(pick))
            packed = pick[:, 0::2] | (pick[:, 1::2] << 4)
        ws.append(torch.cat([packed, torch.full((n, K // 32), 127, dtype=torch.int64)], 1)
                  .to(torch.uint8))
    x = (torch.randint(-255, 256, (M, K), generator=g).to(torch.float32) / 64).to(torch.bfloat16)
    fp = _plan(ws, fmt)
    assert fp.set_tiling(M, _small_tiling(K)) == P.FP_OK
    ys = fp(to_gpu(x))
    torch.cuda.synchronize()
    lin = CASES[fmt][1]
    for y, w in zip(ys, ws):
        ref, _ = lin(si.bits(x), si.bits(w), K)
        assert np.array_equal(si.bits(y.cpu()), oracle.round_bf16(ref))


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_mx_small_mfma_graph_replay(fmt):
    M = 8
    x0, ws = CASES[fmt][0](M, 70)
    fp = _plan(ws, fmt)
    assert fp.set_tiling(M, _small_tiling(5120)) == P.FP_OK
    x_static = to_gpu(x0)
    outs = [torch.empty(M, n, dtype=torch.bfloat16, device="cuda") for n in fp.N]
    fp(x_static, out=outs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp(x_static, out=outs)
    torch.cuda.synchronize()
    for seed in (71, 72, 73):
        xn, _ = CASES[fmt][0](M, seed)
        x_static.copy_(to_gpu(xn))
        g.replay()
        torch.cuda.synchronize()
        assert_bitwise_equal(outs, fp(x_static), "replay seed %d" % seed)
        _check(outs, xn, ws, 5120, fmt, "replay seed %d" % seed)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("M", [9, 12, 16])
def test_mx_small_mfma_two_token_halves(fmt, M):
    # 9..16 tokens: the same kernel with two token halves (the default path)
    x, ws = CASES[fmt][0](M, 90 + M)
    fp = _plan(ws, fmt, max_M=16)
    assert fp.query(M)[0] == P.FP_PATH_MFMA_SMALL
    xg = to_gpu(x)
    ys = fp(xg)
    _check(ys, x, ws, 5120, fmt, "%s two halves M=%d" % (fmt, M))
    assert_bitwise_equal(ys, fp(xg), "repeat")
    assert_bitwise_equal(ys, fp.forward_separate(xg), "fused vs separate")


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_mx_small_mfma_refusals(fmt):
    x, ws = CASES[fmt][0](1, 0)
    fp = _plan(ws, fmt, max_M=32)
    # no path above 16 tokens for block-scaled weights, no tile kernel
    assert fp.set_tiling(17, _small_tiling(5120)) == P.FP_ERR_UNSUPPORTED
    assert fp.supported(to_gpu(CASES[fmt][0](17, 0)[0])) is False
    assert fp.set_tiling(8, (P.FP_PATH_MFMA, 4, 4, 9, 0, 2)) == P.FP_ERR_UNSUPPORTED
    assert fp.set_tiling(8, (P.FP_PATH_MFMA, 2, 0, 8, 0, 0)) == P.FP_ERR_UNSUPPORTED
    torch.cuda.synchronize()


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("M", [9, 13, 16])
def test_mx_two_token_halves_at_k7168(fmt, M):
    # K = 7168 (the DeepSeek hidden size): two token halves at eight K steps
    # per wave would need 14 K parts, more waves than the two-half form's
    # thread bound; the default takes sixteen steps per wave (7 parts)
    K = 7168
    x, ws = CASES[fmt][0](M, 110 + M, K=K, N=(1536, 576))
    fp = _plan(ws, fmt, max_M=16)
    assert fp.query(M)[0] == P.FP_PATH_MFMA_SMALL
    assert tuple(fp.get_tiling(M)[1:3]) == (7, 16)
    xg = to_gpu(x)
    ys = fp(xg)
    _check(ys, x, ws, K, fmt, "%s K=7168 M=%d" % (fmt, M))
    assert_bitwise_equal(ys, fp(xg), "repeat")
    assert_bitwise_equal(ys, fp.forward_separate(xg), "fused vs separate")


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_mx_two_token_halves_refused_past_k8192(fmt):
    # one workgroup spans K: past 8192 two token halves do not fit, and the
    # call is refused without a launch; 8 tokens are still served
    K = 8704
    x, ws = CASES[fmt][0](9, 5, K=K, N=(64, 7))
    fp = _plan(ws, fmt, max_M=16)
    xg = to_gpu(x)
    assert fp.supported(xg) is False
    assert fp.supported(xg[:8]) is True
    ys = fp(xg[:8])
    _check(ys, x[:8], ws, K, fmt, "%s K=8704 M=8" % fmt)


def _random_mx_cases(n, seed):
    """Seeded block-scaled shapes: K a multiple of 512 up to 8192, one or
    two projections of 1..3000 rows, M 1..16."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        K = 512 * int(rng.integers(1, 17))
        N = tuple(int(round(np.exp(rng.uniform(0.0, np.log(3000.0)))))
                  for _ in range(int(rng.integers(1, 3))))
        if sum(N) * K > 12_000_000:
            continue
        out.append((K, N, int(rng.integers(1, 17))))
    return out


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("K,N,M", _random_mx_cases(10, 8))
def test_mx_default_routing_on_random_shapes(fmt, K, N, M):
    x, ws = CASES[fmt][0](M, K + M, K=K, N=N)
    fp = _plan(ws, fmt, max_M=16)
    xg = to_gpu(x)
    assert fp.supported(xg), (fmt, K, N, M)
    ys = fp(xg)
    _check(ys, x, ws, K, fmt, "%s K=%d N=%s M=%d %s" % (fmt, K, N, M, fp.get_tiling(M)))
    assert_bitwise_equal(ys, fp.forward_separate(xg), "fused vs separate")
