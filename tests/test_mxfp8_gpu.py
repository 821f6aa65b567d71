"""Parity of the MXFP8-weight projection (through the C ABI) with the oracle.

The pages name MXFP8 projections for the DeepSeek-V4.1 wq_a / wkv weights
("tinygemm2 for the DeepSeek-V4.1 hidden-state projections", Description);
read as the open microscaling format (E4M3 codes, one E8M0 scale per 32
elements along K), packed rows of K codes then K/32 scales.  The weights
are half the bytes of bf16; activations and outputs stay bf16.

Checked: the decode (all 256 codes at several scales) bit-exact against the
oracle's exact values; every projection element against the oracle's fp64
sum under the bf16 rule; exact data bit exact; repeats, fused vs one launch
per projection and graph replays bitwise equal.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
import projection_gemm_sparse_amd as P
from gpu_util import assert_bitwise_equal, assert_matches_oracle, to_gpu

pytestmark = pytest.mark.gpu

SCALES = (1, 100, 112, 127, 140, 200)


def _plan(ws, max_M=8):
    return P.FusedProjection([to_gpu(w) for w in ws], max_M=max_M, weight_format="mxfp8")


def _check(ys, x_cpu, ws, K, label):
    torch.cuda.synchronize()
    for i, (y, w) in enumerate(zip(ys, ws)):
        ref, s = oracle.linear_mxfp8(si.bits(x_cpu), si.bits(w), K)
        got = oracle.bf16_bits_to_f64(si.bits(y.cpu()))
        ok, worst, idx = oracle.check_within_bound(got, ref, s, oracle.BF16)
        assert ok, "%s proj %d: worst |err|/bound %.3g at %s" % (label, i, worst, idx)


def test_decode_all_codes_bit_exact():
    K = 512
    rows = []
    for s in SCALES:
        codes = np.concatenate([np.arange(256), np.arange(256)]).astype(np.uint8)
        rows.append(np.concatenate([codes, np.full(K // 32, s, dtype=np.uint8)]))
    w = torch.from_numpy(np.stack(rows))
    wg = to_gpu(w)
    out = torch.empty(len(SCALES), K, dtype=torch.bfloat16, device="cuda")
    assert P.fp_mxfp8_to_bf16(wg.data_ptr(), len(SCALES), K, out.data_ptr(), 0) == P.FP_OK
    torch.cuda.synchronize()
    got = si.bits(out.cpu())
    for r, s in enumerate(SCALES):
        for k in range(K):
            c = k % 256
            v = oracle.e4m3_value(c) * oracle.e8m0_value(s)
            if np.isnan(v):
                assert (got[r, k] & 0x7F80) == 0x7F80 and (got[r, k] & 0x7F) != 0, (s, c)
                continue
            g = oracle.bf16_bits_to_f64(np.array([got[r, k]]))[0]
            if v == 0 or abs(v) >= 2.0 ** -126:
                # the served domain: the scaled value is exact in bf16
                want = oracle.round_bf16(np.array([v]))[0]
                assert oracle.bf16_bits_to_f64(np.array([want]))[0] == v
                assert got[r, k] == want, "code 0x%02x scale %d: got 0x%04x want 0x%04x" % (
                    c, s, got[r, k], want)
            else:
                # below bf16's normal range: within one subnormal quantum
                assert abs(g - v) <= 2.0 ** -133, (c, s, g, v)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("seed", [0, 1])
def test_mxfp8_wq_a_wkv(M, seed):
    x, ws = si.mxfp8_case(M, seed)
    fp = _plan(ws)
    assert fp.K == 5120 and fp.query(M)[0] in (P.FP_PATH_SKINNY, P.FP_PATH_MFMA_SMALL)
    xg = to_gpu(x)
    ys = fp(xg)
    _check(ys, x, ws, 5120, "mxfp8 M=%d seed=%d" % (M, seed))
    assert_bitwise_equal(ys, fp(xg), "repeat")
    assert_bitwise_equal(ys, fp.forward_separate(xg), "fused vs separate")


@pytest.mark.parametrize("M", [1, 8])
def test_mxfp8_exact_data_bit_exact(M):
    # codes of +-1/2, +-1, +-2 at scale 2^0, x on a 1/64 grid: every product
    # and every fp32 partial sum exact, so the outputs are RNE(exact sum)
    K, N = 5120, (1280, 512)
    g = torch.Generator().manual_seed(17)
    codes = torch.tensor([0x30, 0x38, 0x40, 0xB0, 0xB8, 0xC0], dtype=torch.int64)
    ws = []
    for n in N:
        pick = codes[torch.randint(0, 6, (n, K), generator=g)]
        keep = torch.rand(n, K, generator=g) < 0.02  # sparse rows keep sums small
        pick = torch.where(keep, pick, torch.zeros_like(pick))
        ws.append(torch.cat([pick, torch.full((n, K // 32), 127, dtype=torch.int64)], 1)
                  .to(torch.uint8))
    x = (torch.randint(-255, 256, (M, K), generator=g).to(torch.float32) / 64).to(torch.bfloat16)
    fp = _plan(ws)
    ys = fp(to_gpu(x))
    torch.cuda.synchronize()
    for y, w in zip(ys, ws):
        ref, _ = oracle.linear_mxfp8(si.bits(x), si.bits(w), K)
        assert np.array_equal(si.bits(y.cpu()), oracle.round_bf16(ref))


def test_mxfp8_three_way_strided_x_and_reload():
    # three projections at K = 6144, x with row stride K + 64, then new
    # weights written through the views
    K, N = 6144, (2048, 576, 128)
    M = 4
    x, ws = si.mxfp8_case(M, 2, K=K, N=N, ldx=K + 64)
    fp = _plan(ws)
    xg = to_gpu(x)[:, :K]
    ys = fp(xg)
    _check(ys, x[:, :K].contiguous(), ws, K, "3-way")
    _, ws2 = si.mxfp8_case(M, 3, K=K, N=N)
    for v, w in zip(fp.views, ws2):
        v.copy_(to_gpu(w))
    ys2 = fp(xg)
    _check(ys2, x[:, :K].contiguous(), ws2, K, "after reload")
    assert_bitwise_equal(ys2, fp.forward_separate(xg), "fused vs separate after reload")


def test_mxfp8_graph_replay_equals_eager():
    M = 8
    x0, ws = si.mxfp8_case(M, 0)
    fp = _plan(ws)
    x_static = to_gpu(x0)
    outs = [torch.empty(M, n, dtype=torch.bfloat16, device="cuda") for n in fp.N]
    fp(x_static, out=outs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp(x_static, out=outs)
    torch.cuda.synchronize()
    for seed in (11, 12, 13):
        xn, _ = si.mxfp8_case(M, seed)
        x_static.copy_(to_gpu(xn))
        g.replay()
        torch.cuda.synchronize()
        assert_bitwise_equal(outs, fp(x_static), "replay seed %d" % seed)
        _check(outs, xn, ws, 5120, "replay seed %d" % seed)


@pytest.mark.parametrize("M", [4, 8])
def test_mxfp8_rmsnorm_epilogue(M):
    # M = 4: the vector-ALU kernel; M = 8: the small-M matrix-core kernel
    x, ws = si.mxfp8_case(M, 4)
    g = torch.Generator().manual_seed(4)
    gammas = [(1.0 + 0.1 * torch.randn(n, generator=g)).to(torch.bfloat16) for n in (1280, 512)]
    fp = _plan(ws)
    xg = to_gpu(x)
    gg = [to_gpu(t) for t in gammas]
    outs = fp.forward_rmsnorm(xg, gg, 1e-6)
    assert_bitwise_equal(outs, fp.forward_rmsnorm_separate(xg, gg, 1e-6), "chain")
    torch.cuda.synchronize()
    eps = float(np.float32(1e-6))
    for o, w, gm in zip(outs, ws, gammas):
        y, s = oracle.linear_mxfp8(si.bits(x), si.bits(w), 5120)
        yb = oracle.round_bf16(y)
        out, rinv = oracle.rmsnorm(yb, si.bits(gm), eps)
        r = {"y": y, "S": s, "yb": yb, "out": out, "rinv": rinv}
        bound = oracle.rmsnorm_bound(r, si.bits(gm), eps)
        ok, worst, idx = oracle.check_against(oracle.bf16_bits_to_f64(si.bits(o.cpu())), out,
                                              bound)
        assert ok, (worst, idx)


def test_mxfp8_refusals():
    x, ws = si.mxfp8_case(1, 0)
    fp = _plan(ws, max_M=32)
    x17 = to_gpu(si.mxfp8_case(17, 0)[0])
    assert fp.supported(x17) is False  # above 16 tokens
    assert P.fp_plan_set_out_dtype(fp.plan, P.FP_F32) == P.FP_ERR_UNSUPPORTED
    buf = torch.empty(2, 544, dtype=torch.uint8, device="cuda")
    out = torch.empty(2, 528, dtype=torch.bfloat16, device="cuda")
    assert P.fp_mxfp8_to_bf16(buf.data_ptr(), 2, 528, out.data_ptr(), 0) == \
        P.FP_ERR_UNSUPPORTED  # K not a multiple of 512
    torch.cuda.synchronize()
