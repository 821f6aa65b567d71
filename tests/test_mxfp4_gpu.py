"""Parity of the MXFP4-weight projection (through the C ABI) with the oracle.

The FP4 form of the fused weight ("Fuse QK down_proj with indexer K +
weight_proj for FP4 ckpt", PR #8771), read as the microscaling FP4 format:
E2M1 codes, two per byte (element 2i in the low nibble), one E8M0 scale per
32 elements; packed rows of K/2 code bytes then K/32 scales, a quarter of
the bf16 bytes plus the scales.  Activations and outputs stay bf16.

Checked: the decode (all 256 code bytes at several scales) bit-exact
against the oracle's exact values, which also fixes the nibble order; every
projection element against the oracle's fp64 sum under the bf16 rule; exact
data bit exact; repeats, fused vs one launch per projection and graph
replays bitwise equal.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
import projection_gemm_sparse_amd as P
from gpu_util import assert_bitwise_equal, to_gpu

pytestmark = pytest.mark.gpu

SCALES = (1, 100, 118, 127, 140, 240)


def _plan(ws, max_M=8):
    return P.FusedProjection([to_gpu(w) for w in ws], max_M=max_M, weight_format="mxfp4")


def _check(ys, x_cpu, ws, K, label):
    torch.cuda.synchronize()
    for i, (y, w) in enumerate(zip(ys, ws)):
        ref, s = oracle.linear_mxfp4(si.bits(x_cpu), si.bits(w), K)
        got = oracle.bf16_bits_to_f64(si.bits(y.cpu()))
        ok, worst, idx = oracle.check_within_bound(got, ref, s, oracle.BF16)
        assert ok, "%s proj %d: worst |err|/bound %.3g at %s" % (label, i, worst, idx)


def test_decode_all_code_bytes_bit_exact():
    K = 512
    rows = []
    for s in SCALES:
        codes = np.arange(256).astype(np.uint8)
        rows.append(np.concatenate([codes, np.full(K // 32, s, dtype=np.uint8)]))
    w = to_gpu(torch.from_numpy(np.stack(rows)))
    out = torch.empty(len(SCALES), K, dtype=torch.bfloat16, device="cuda")
    assert P.fp_mxfp4_to_bf16(w.data_ptr(), len(SCALES), K, out.data_ptr(), 0) == P.FP_OK
    torch.cuda.synchronize()
    got = si.bits(out.cpu())
    for r, s in enumerate(SCALES):
        for k in range(K):
            byte = k // 2
            code = (byte >> 4) if k % 2 else (byte & 0xF)
            v = oracle.e2m1_value(code) * oracle.e8m0_value(s)
            g = oracle.bf16_bits_to_f64(np.array([got[r, k]]))[0]
            if v == 0 or abs(v) >= 2.0 ** -126:
                want = oracle.round_bf16(np.array([v]))[0]
                assert oracle.bf16_bits_to_f64(np.array([want]))[0] == v
                assert got[r, k] == want, "byte 0x%02x elem %d scale %d: 0x%04x vs 0x%04x" % (
                    byte, k % 2, s, got[r, k], want)
            else:
                assert abs(g - v) <= 2.0 ** -133, (byte, s, g, v)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
@pytest.mark.parametrize("seed", [0, 1])
def test_mxfp4_wq_a_wkv(M, seed):
    x, ws = si.mxfp4_case(M, seed)
    fp = _plan(ws)
    assert fp.K == 5120 and fp.query(M)[0] in (P.FP_PATH_SKINNY, P.FP_PATH_MFMA_SMALL)
    xg = to_gpu(x)
    ys = fp(xg)
    _check(ys, x, ws, 5120, "mxfp4 M=%d seed=%d" % (M, seed))
    assert_bitwise_equal(ys, fp(xg), "repeat")
    assert_bitwise_equal(ys, fp.forward_separate(xg), "fused vs separate")


@pytest.mark.parametrize("M", [1, 8])
def test_mxfp4_exact_data_bit_exact(M):
    # codes of +-1/2, +-1, +-2 at scale 2^0, x on a 1/64 grid, sparse rows:
    # every fp32 partial sum exact, so the outputs are RNE(exact sum)
    K, N = 5120, (1280, 512)
    g = torch.Generator().manual_seed(19)
    vals = torch.tensor([0x1, 0x2, 0x4, 0x9, 0xA, 0xC], dtype=torch.int64)
    ws = []
    for n in N:
        c = vals[torch.randint(0, 6, (n, K), generator=g)]
        keep = torch.rand(n, K, generator=g) < 0.02
        c = torch.where(keep, c, torch.zeros_like(c))
        packed = c[:, 0::2] | (c[:, 1::2] << 4)
        ws.append(torch.cat([packed, torch.full((n, K // 32), 127, dtype=torch.int64)], 1)
                  .to(torch.uint8))
    x = (torch.randint(-255, 256, (M, K), generator=g).to(torch.float32) / 64).to(torch.bfloat16)
    fp = _plan(ws)
    ys = fp(to_gpu(x))
    torch.cuda.synchronize()
    for y, w in zip(ys, ws):
        ref, _ = oracle.linear_mxfp4(si.bits(x), si.bits(w), K)
        assert np.array_equal(si.bits(y.cpu()), oracle.round_bf16(ref))


def test_mxfp4_three_way_strided_x_graph_replay():
    K, N = 6144, (2048, 576, 128)
    M = 5
    x0, ws = si.mxfp4_case(M, 2, K=K, N=N, ldx=K + 64)
    fp = _plan(ws)
    x_static = to_gpu(x0)
    xv = x_static[:, :K]
    outs = [torch.empty(M, n, dtype=torch.bfloat16, device="cuda") for n in N]
    fp(xv, out=outs)
    _check(outs, x0[:, :K].contiguous(), ws, K, "3-way strided")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp(xv, out=outs)
    torch.cuda.synchronize()
    for seed in (11, 12):
        xn, _ = si.mxfp4_case(M, seed, K=K, N=N, ldx=K + 64)
        x_static.copy_(to_gpu(xn))
        g.replay()
        torch.cuda.synchronize()
        assert_bitwise_equal(outs, fp(xv), "replay seed %d" % seed)
        _check(outs, xn[:, :K].contiguous(), ws, K, "replay seed %d" % seed)


def test_mxfp4_refusals_and_format_inference():
    x, ws = si.mxfp4_case(1, 0)
    fp = P.FusedProjection([to_gpu(w) for w in ws], max_M=32)  # 2720 = 17 * 160: mxfp4
    assert fp.fp_dtype == P.FP_MXFP4 and fp.K == 5120
    x17 = to_gpu(si.mxfp4_case(17, 0)[0])
    assert fp.supported(x17) is False  # above 16 tokens
    assert P.fp_plan_set_out_dtype(fp.plan, P.FP_F32) == P.FP_ERR_UNSUPPORTED
    torch.cuda.synchronize()
