"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Every workload cell is checked element by element against the oracle's
fp64 result under the acceptance bound (bf16: 2^-7 * S + 1e-6, fp32:
1e-5 * S + 1e-7, S = sum_k |x_k w_k|); fused and one-launch-per-projection
outputs must be bitwise equal, and so must repeats.  Integer-valued data
must be bit exact (every partial sum is an exact integer below 2^24).
"""
import os

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
import projection_gemm_sparse_amd as P
from gpu_util import (BF16, F32, assert_bitwise_equal, assert_matches_oracle, out_bits,
                      to_gpu)

pytestmark = pytest.mark.gpu


def _plan(ws_cpu, max_M=8, workspace_bytes=None):
    return P.FusedProjection([to_gpu(w) for w in ws_cpu], max_M=max_M,
                             workspace_bytes=workspace_bytes)


def _check_case(fp, x_cpu, ws_cpu, label, rows=None, separate=True):
    x = to_gpu(x_cpu)
    if x_cpu.shape[1] != fp.K:
        x = x[:, :fp.K]
    ys = fp(x)
    assert_matches_oracle(ys, x_cpu[:, :fp.K].contiguous(), ws_cpu, rows=rows, label=label)
    ys2 = fp(x)
    assert_bitwise_equal(ys, ys2, label + " repeat")
    if separate:
        ysep = fp.forward_separate(x)
        assert_bitwise_equal(ys, ysep, label + " fused vs separate")
    return ys


def test_library_is_the_in_tree_build():
    import os
    here = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    assert os.path.dirname(os.path.abspath(P.LIB_PATH)) == os.path.join(
        here, "projection_gemm_sparse_amd")
    assert torch.cuda.is_available()


# ---- wq_a + wkv, one token (K=5120, [1280, 512], bf16, seed 0)
def test_wq_a_wkv_m1():
    x, ws = si.workload_case("wq_a+wkv_m1", 1, 0)
    fp = _plan(ws)
    assert fp.query(1) == (P.FP_PATH_SKINNY, 1, 2)
    _check_case(fp, x, ws, "wq_a+wkv M=1")


# ---- M in {2, 4, 8}, seeds 1-3
@pytest.mark.parametrize("M", [2, 4, 8])
@pytest.mark.parametrize("seed", [1, 2, 3])
def test_wq_a_wkv_m2_8(M, seed):
    x, ws = si.workload_case("wq_a+wkv_m2_8", M, seed)
    fp = _plan(ws)
    _check_case(fp, x, ws, "wq_a+wkv M=%d seed=%d" % (M, seed))


# ---- fp32 indexer fusion (K=7168, [128, 64]): the default tiling (each
#      row in one workgroup) and forced K splits across workgroups
@pytest.mark.parametrize("M", [1, 4, 8])
@pytest.mark.parametrize("seed", [0, 1, 2, 3])
@pytest.mark.parametrize("tiling", [None, (P.FP_PATH_SKINNY_SPLITK, 7, 1, 4, 0, 0),
                                    (P.FP_PATH_SKINNY_SPLITK, 2, 2, 7, 1, 3)],
                         ids=["default", "split4", "split7"])
def test_indexer_fp32(M, seed, tiling):
    x, ws = si.workload_case("indexer_f32", M, seed)
    fp = _plan(ws, workspace_bytes=1 << 20)
    if tiling is not None:
        assert fp.set_tiling(M, tiling) == P.FP_OK
        assert fp.query(M)[0] == P.FP_PATH_SKINNY_SPLITK
    _check_case(fp, x, ws, "indexer fp32 M=%d seed=%d tiling=%s" % (M, seed, tiling))


# ---- three-way fused-A (K=6144, [2048, 576, 128]), M 1..8
@pytest.mark.parametrize("M", range(1, 9))
def test_fused_a_three_way(M):
    x, ws = si.workload_case("fused_a_3way", M, 0)
    fp = _plan(ws)
    _check_case(fp, x, ws, "fused-A M=%d" % M)


# ---- crossover sweep, strided x (row stride K + 64); sampled token rows
#      for large M (the oracle's cost grows with M; rows are independent)
@pytest.mark.parametrize("M", [1, 2, 4, 8, 9, 16, 17, 24, 32, 64, 128])
def test_crossover_sweep_strided_x(M):
    K = 5120
    x_full, ws = si.workload_case("crossover", M, 0, ldx=K + 64)
    fp = _plan(ws, max_M=128)
    x = to_gpu(x_full)[:, :K]
    assert x.stride(0) == K + 64
    ys = fp(x)
    rows = None if M <= 16 else sorted({0, 1, M // 2, M - 2, M - 1} | set(range(3, M, 13)))
    assert_matches_oracle(ys, x_full[:, :K].contiguous(), ws, rows=rows,
                          label="crossover M=%d" % M)
    assert_bitwise_equal(ys, fp.forward_separate(x), "crossover M=%d fused/sep" % M)
    # contiguous x gives the same bits as the strided view
    assert_bitwise_equal(ys, fp(x.contiguous()), "crossover M=%d strided/contig" % M)


# ---- small shapes: several tiles, ragged tails, odd projection sizes
@pytest.mark.parametrize("dt", [BF16, F32])
@pytest.mark.parametrize("M", [1, 2, 3, 5, 7, 8, 9, 17, 33])
def test_ragged_small_shapes(dt, M):
    if dt == F32 and M > 8:
        pytest.skip("fp32 is served for M <= 8")
    K = 136 if dt == BF16 else 132
    N = (37, 5, 70, 1)
    x, ws = si.make_case(K, N, "bf16" if dt == BF16 else "f32", M, seed=40 + M,
                         w_dist="uniform_inv_sqrt_k" if dt == BF16 else "normal_0.02")
    fp = _plan(ws, max_M=64)
    _check_case(fp, x, ws, "ragged %s M=%d" % (dt, M))


@pytest.mark.parametrize("dt", [BF16, F32])
@pytest.mark.parametrize("K", [8, 1032, 20480])
def test_k_extremes(dt, K):
    if dt == F32:
        K = K // 2 if K > 8 else 4
    N = (300, 29)
    x, ws = si.make_case(K, N, "bf16" if dt == BF16 else "f32", 3, seed=K,
                         w_dist="uniform_inv_sqrt_k" if dt == BF16 else "normal_0.02")
    fp = _plan(ws, max_M=16)
    _check_case(fp, x, ws, "K=%d %s" % (K, dt))


# ---- integer data: bit exact on every path
@pytest.mark.parametrize("dt,K,N,M", [
    (BF16, 5120, (1280, 512), 1), (BF16, 5120, (1280, 512), 8),
    (BF16, 5120, (1280, 512), 32), (BF16, 6144, (2048, 576, 128), 5),
    (F32, 7168, (128, 64), 4), (F32, 7168, (128, 64), 1)])
def test_integer_data_bit_exact(dt, K, N, M):
    x, ws = si.make_case(K, N, "bf16" if dt == BF16 else "f32", M, seed=7,
                         w_dist="int4", x_dist="int4")
    fp = _plan(ws, max_M=32)
    ys = fp(to_gpu(x))
    got = out_bits(ys)
    xi = x.float().numpy().astype(np.int64)
    for w, g in zip(ws, got):
        exact = (xi @ w.float().numpy().astype(np.int64).T).astype(np.float64)
        if dt == BF16:
            want = oracle.round_bf16(exact)
        else:
            want = exact.astype(np.float32).view(np.uint32)
        assert np.array_equal(g, want)


# ---- every tiling the kernels accept passes; fused == separate under each
@pytest.mark.parametrize("M", [1, 4, 8, 16, 24])
def test_tilings_all_pass(M):
    x, ws = si.workload_case("crossover", M, 3)
    fp = _plan(ws, max_M=24, workspace_bytes=64 << 20)
    xg = to_gpu(x)
    tilings = [
        (P.FP_PATH_SKINNY, 10, 1, 1, 0, 0),
        (P.FP_PATH_SKINNY, 5, 2, 1, 0, 0),
        (P.FP_PATH_SKINNY, 5, 1, 2, 0, 0),
        (P.FP_PATH_SKINNY, 2, 1, 5, 1, 0),
        (P.FP_PATH_SKINNY, 4, 2, 2, 0, 2),
        (P.FP_PATH_SKINNY, 10, 1, 1, 1, 1),
        (P.FP_PATH_SKINNY, 1, 10, 1, 1, 7),  # whole rows per wave, no barrier
        (P.FP_PATH_SKINNY, 1, 10, 1, 2, 3),
        (P.FP_PATH_SKINNY, 2, 5, 1, 1, 5),
        (P.FP_PATH_MFMA, 2, 40, 4, 0, 0),   # tile kernel: row tiles, register
        (P.FP_PATH_MFMA, 4, 20, 8, 0, 0),   # bound of k steps, slices
        (P.FP_PATH_MFMA, 8, 8, 20, 0, 0),
        (P.FP_PATH_MFMA, 2, 8, 20, 0, 0),
        (P.FP_PATH_MFMA, 2, 40, 5, 0, 0),
        (P.FP_PATH_MFMA, 2, 20, 9, 0, 0),   # uneven slices (160 steps / 9)
        (P.FP_PATH_MFMA, 2, 8, 160, 0, 0),  # one k step per slice
        (P.FP_PATH_MFMA_SMALL, 10, 8, 1, 0, 0),
        (P.FP_PATH_MFMA_SMALL, 5, 16, 1, 8, 1),
        (P.FP_PATH_MFMA_SMALL, 5, 16, 1, 3, 2),  # two row groups of 3 rows
        (P.FP_PATH_MFMA_SMALL, 16, 8, 1, 1, 0),  # more K parts than needed
        (P.FP_PATH_MFMA_SMALL, 10, 8, 1, 12, 1),  # two tiles of 6 rows per wave
        (P.FP_PATH_MFMA_SMALL, 5, 16, 1, 16, 1),  # two tiles of 8 rows per wave
    ]
    ran = 0
    for t in tilings:
        st = fp.set_tiling(M, t)
        if st != P.FP_OK:
            # skinny tilings above M = 8, tile tilings at M <= 8 (and above
            # 16 tokens where their slice of 32 token rows exceeds LDS) and
            # small-M MFMA workgroups above the register bound of their
            # token halves are refused
            assert st == P.FP_ERR_UNSUPPORTED, (t, st)
            assert ((t[0] in (P.FP_PATH_SKINNY, P.FP_PATH_SKINNY_SPLITK)
                     and (M > 8 or (t[2] > 2 and M > 2)))
                    or (t[0] == P.FP_PATH_MFMA and (M <= 8 or (M > 16 and t[2] >= 20)))
                    or (t[0] == P.FP_PATH_MFMA_SMALL and M > 8
                        and (max(1, t[5]) * t[1] * 64 >
                             _smfma_thread_cap(t[2], 3 if M > 16 else 2, 2 if t[4] > 8 else 1)
                             or (M > 16 and t[4] > 8)))), (t, st)
            continue
        ran += 1
        ys = fp(xg)
        assert_matches_oracle(ys, x, ws, label="tiling %s M=%d" % (t, M))
        assert_bitwise_equal(ys, fp.forward_separate(xg), "tiling %s fused/sep" % (t,))
    assert ran >= 4
    fp.set_tiling(M, None)


# ---- edge cases
def test_m_zero_launches_nothing():
    x, ws = si.workload_case("wq_a+wkv_m1", 1, 0)
    fp = _plan(ws)
    sentinel = [torch.full((1, n), 3.0, dtype=BF16, device="cuda") for n in fp.N]
    x0 = to_gpu(x)[:0]
    assert P.fp_forward(x0.data_ptr() or 0, 0, fp.K, fp.plan, 0,
                        [y.data_ptr() for y in sentinel]) == P.FP_OK
    torch.cuda.synchronize()
    assert all(bool((y == 3.0).all()) for y in sentinel)
    assert fp.query(0) == (P.FP_PATH_NONE, 0, 0)


def test_max_m_sampled():
    M = 256
    x, ws = si.make_case(1024, (300, 77), "bf16", M, seed=5)
    fp = _plan(ws, max_M=256)
    ys = fp(to_gpu(x))
    rows = [0, 1, 100, 127, 128, 200, 254, 255]
    assert_matches_oracle(ys, x, ws, rows=rows, label="M=256")


def test_unsupported_inputs_are_refused_without_launch():
    x, ws = si.workload_case("wq_a+wkv_m1", 2, 0)
    fp = _plan(ws, max_M=8)
    xg = to_gpu(x)
    outs = [torch.full((2, n), 7.0, dtype=BF16, device="cuda") for n in fp.N]
    ptrs = [o.data_ptr() for o in outs]
    # misaligned x (2-byte offset)
    buf = torch.zeros(2 * 5120 + 8, dtype=BF16, device="cuda")
    assert P.fp_forward(buf.data_ptr() + 2, 2, 5120, fp.plan, 0, ptrs) == P.FP_ERR_UNSUPPORTED
    # row stride not a multiple of 16 bytes
    assert P.fp_forward(xg.data_ptr(), 2, 5121, fp.plan, 0, ptrs) == P.FP_ERR_UNSUPPORTED
    # ldx < K
    assert P.fp_forward(xg.data_ptr(), 2, 5000, fp.plan, 0, ptrs) == P.FP_ERR_INVALID_ARG
    # M above max_M
    assert P.fp_forward(xg.data_ptr(), 9, 5120, fp.plan, 0, ptrs) == P.FP_ERR_UNSUPPORTED
    # output overlapping x
    assert P.fp_forward(xg.data_ptr(), 2, 5120, fp.plan, 0,
                        [xg.data_ptr(), ptrs[1]]) == P.FP_ERR_INVALID_ARG
    # outputs overlapping each other
    assert P.fp_forward(xg.data_ptr(), 2, 5120, fp.plan, 0,
                        [ptrs[0], ptrs[0]]) == P.FP_ERR_INVALID_ARG
    torch.cuda.synchronize()
    assert all(bool((o == 7.0).all()) for o in outs)
    assert fp.supported(xg) and not fp.supported(to_gpu(si.workload_case("wq_a+wkv_m1", 9, 0)[0]))


def test_single_row_projections_and_one_projection():
    x, ws = si.make_case(5120, (1,), "bf16", 4, seed=9)
    _check_case(_plan(ws), x, ws, "one row")
    x, ws = si.make_case(5120, (1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1, 1), "bf16", 3, seed=9)
    _check_case(_plan(ws), x, ws, "16 single-row projections")


# ---- the small-M matrix-core kernel (opt-in tiling) on every workload shape
def _smfma_thread_cap(kt, mh, tt=1):
    """Largest workgroup of the small-M matrix-core kernel: its register
    estimate per lane (tt row tiles per wave), 4 waves per SIMD at most."""
    if mh + tt >= 4:
        regs = 4 * kt * (mh + tt) + 24
    else:
        regs = 4 * kt * (mh + tt) + 24 + 16 * (mh - 1) + 4 * (tt - 1)
    return 256 * max(1, min(4, 512 // regs))


def _small_mfma_tiling(K, esize=2):
    kc = K * esize // 16
    steps = -(-kc // 8)
    kt = 4 if steps <= 64 else 8 if steps <= 128 else 16
    return (P.FP_PATH_MFMA_SMALL, -(-steps // kt), kt, 1, 0, 0)


@pytest.mark.parametrize("case", ["wq_a+wkv", "fused_a_3way", "ragged", "single_rows", "k8"])
@pytest.mark.parametrize("M", [1, 2, 3, 5, 8, 9, 12, 16, 17, 20, 24])
def test_small_mfma_path(case, M):
    if case == "wq_a+wkv":
        x, ws = si.workload_case("wq_a+wkv_m2_8", M, 1)
    elif case == "fused_a_3way":
        x, ws = si.workload_case("fused_a_3way", M, 0)
    elif case == "ragged":
        x, ws = si.make_case(136, (37, 5, 70, 1), "bf16", M, seed=60 + M)
    elif case == "single_rows":
        x, ws = si.make_case(1024, (1,) * 16, "bf16", M, seed=61 + M)
    else:
        x, ws = si.make_case(8, (300, 29), "bf16", M, seed=62 + M)
    fp = _plan(ws, max_M=24)
    assert fp.set_tiling(M, _small_mfma_tiling(fp.K)) == P.FP_OK
    assert fp.query(M)[0] == P.FP_PATH_MFMA_SMALL
    _check_case(fp, x, ws, "small-M MFMA %s M=%d" % (case, M))


# ---- two row tiles per wave (rows 10..16: two tiles of rows / 2 sharing the
#      activation operand): same per-row order as one tile, so the outputs
#      are bitwise those of one tile of rows / 2, and within the bound
@pytest.mark.parametrize("case", ["fused_a_3way", "ragged", "single_rows", "k8", "page_2784"])
@pytest.mark.parametrize("M", [1, 3, 5, 8, 9, 12, 13, 16])
def test_small_mfma_two_tiles_per_wave(case, M):
    if case == "fused_a_3way":
        x, ws = si.workload_case("fused_a_3way", M, 2)
    elif case == "ragged":
        x, ws = si.make_case(136, (37, 5, 70, 1), "bf16", M, seed=70 + M)
    elif case == "single_rows":
        x, ws = si.make_case(1024, (1,) * 16, "bf16", M, seed=71 + M)
    elif case == "k8":
        x, ws = si.make_case(8, (300, 29), "bf16", M, seed=72 + M)
    else:
        K, N = _page_shape("glm_fused_a_indexer")
        x, ws = si.make_case(K, N, "bf16", M, seed=73 + M)
    fp = _plan(ws, max_M=16)
    base = _small_mfma_tiling(fp.K)
    mh = 2 if M > 8 else 1
    xg = to_gpu(x)
    ref = None
    for rows, groups in ((10, 1), (12, 1), (14, 2), (16, 1), (6, 1)):
        st = fp.set_tiling(M, base[:4] + (rows, groups))
        if groups * base[1] * 64 > _smfma_thread_cap(base[2], mh, 2 if rows > 8 else 1):
            assert st == P.FP_ERR_UNSUPPORTED, (rows, groups)
            continue
        assert st == P.FP_OK, (rows, groups)
        assert fp.query(M)[0] == P.FP_PATH_MFMA_SMALL
        label = "two tiles %s M=%d rows=%d G=%d" % (case, M, rows, groups)
        ys = _check_case(fp, x, ws, label)
        if ref is None:
            ref = ys
        else:
            assert_bitwise_equal(ys, ref, label + " vs rows=10")
    fp.set_tiling(M, None)


def test_small_mfma_two_tiles_refused_where_unsupported():
    x, ws = si.workload_case("fused_a_3way", 9, 0)
    fp = _plan(ws, max_M=16)
    base = _small_mfma_tiling(fp.K)
    # odd row counts above 8, more than 16 rows, a workgroup past the
    # two-tile two-half thread bound (16 K parts of 64 lanes > 768)
    assert fp.set_tiling(8, base[:4] + (11, 1)) == P.FP_ERR_UNSUPPORTED
    assert fp.set_tiling(8, base[:4] + (18, 1)) == P.FP_ERR_UNSUPPORTED
    assert fp.set_tiling(9, (P.FP_PATH_MFMA_SMALL, 16, 8, 1, 12, 1)) == P.FP_ERR_UNSUPPORTED
    assert fp.set_tiling(8, base[:4] + (12, 1)) == P.FP_OK
    assert fp.set_tiling(9, base[:4] + (12, 1)) == P.FP_OK
    fp.set_tiling(8, None)
    fp.set_tiling(9, None)


# ---- the split tile path finishes its K slices either in the launch (last
#      workgroup of each row block) or in a second launch over the whole GPU;
#      both add the slices in slice order: bitwise equal
@pytest.mark.parametrize("M", [16, 64, 128])
def test_tile_finish_in_launch_equals_second_launch(M):
    x, ws = si.workload_case("crossover", M, 6)
    fp = _plan(ws, max_M=128)
    fp.set_mfma_min_m(9)  # the tile kernel also at M = 16
    xg = to_gpu(x)
    t = list(fp.get_tiling(M))
    assert t[0] == P.FP_PATH_MFMA and t[3] > 1 and t[5] in (1, 2)
    outs = {}
    for g in (1, 2):
        assert fp.set_tiling(M, tuple(t[:5] + [g])) == P.FP_OK
        outs[g] = fp(xg)
        assert_matches_oracle(outs[g], x, ws, label="finish %d M=%d" % (g, M))
        assert_bitwise_equal(outs[g], fp.forward_separate(xg), "finish %d fused/sep" % g)
        assert fp.query(M)[1] == g
    assert_bitwise_equal(outs[1], outs[2], "in-launch vs second-launch finish")
    fp.set_tiling(M, None)


# ---- the ring tile kernel (an MFMA tiling whose chunks field is a ring
#      depth of 3, 4 or 6 stage buffers; 64-row blocks)
def _ring(stages, S, finish=0):
    return (P.FP_PATH_MFMA, 4, stages, S, 0, finish)


@pytest.mark.parametrize("M", [17, 64, 128])
@pytest.mark.parametrize("stages", [3, 4, 6])
def test_ring_tile_full_shape(M, stages):
    x, ws = si.workload_case("crossover", M, 11)
    fp = _plan(ws, max_M=128, workspace_bytes=64 << 20)
    xg = to_gpu(x)
    rows = sorted({0, 1, M // 2, M - 1} | set(range(3, M, 29)))
    ran = compared = 0
    for S in (1, 9, 13):
        for finish in (1, 2):
            if S == 1 and finish == 2:
                continue
            st = fp.set_tiling(M, _ring(stages, S, finish))
            if st != P.FP_OK:
                # a ring of 6 stages of 256-token blocks does not fit in LDS
                assert st == P.FP_ERR_UNSUPPORTED and stages == 6 and M > 64, (M, stages, S)
                continue
            ran += 1
            label = "ring M=%d stages=%d S=%d finish=%d" % (M, stages, S, finish)
            ys = _check_case(fp, x, ws, label, rows=rows)
            # the tile kernel with the same slices adds in the same order
            # (where a slice of its activations fits in LDS)
            if fp.set_tiling(M, (P.FP_PATH_MFMA, 2, 0, S, 0, finish)) == P.FP_OK:
                assert_bitwise_equal(ys, fp(xg), label + " vs tile kernel")
                compared += 1
    fp.set_tiling(M, None)
    assert ran >= 1 or stages == 6
    assert compared >= 1 or ran == 0


@pytest.mark.parametrize("M", [2, 9, 16, 33, 100])
def test_ring_tile_ragged(M):
    K, N = 136, (37, 5, 70, 1)
    x, ws = si.make_case(K, N, "bf16", M, seed=70 + M)
    fp = _plan(ws, max_M=128, workspace_bytes=16 << 20)
    for stages in (3, 4):
        for S in (1, 2, 5):  # 5 slices of 17 steps' worth: some slices empty
            assert fp.set_tiling(M, _ring(stages, S)) == P.FP_OK
            _check_case(fp, x, ws, "ring ragged M=%d stages=%d S=%d" % (M, stages, S))
    fp.set_tiling(M, None)


def test_ring_tile_max_m_and_strided_x():
    M, K = 256, 1024
    x, ws = si.make_case(K, (300, 77), "bf16", M, seed=71, ldx=K + 64)
    fp = _plan(ws, max_M=256, workspace_bytes=64 << 20)
    rows = [0, 1, 100, 127, 128, 200, 254, 255]
    for S in (1, 3):
        for finish in (1, 2):
            if S == 1 and finish == 2:
                continue
            assert fp.set_tiling(M, _ring(3, S, finish)) == P.FP_OK
            _check_case(fp, x, ws, "ring M=256 S=%d finish=%d" % (S, finish), rows=rows)
    fp.set_tiling(M, None)


# ---- the weight-resident tile kernel (an MFMA tiling whose chunks field is
#      2; 64-row blocks, the slice's weights resident in LDS, activations
#      through a ring filled by producer waves): same bits as the ring tile
#      kernel for the same slices, either finish
def _wres(S, finish):
    return (P.FP_PATH_MFMA, 4, 2, S, 0, finish)


@pytest.mark.parametrize("M", [17, 32, 40, 64, 100, 128, 200])
def test_weight_resident_tile_kernel(M):
    x, ws = si.workload_case("crossover", M, 12)
    fp = _plan(ws, max_M=256, workspace_bytes=64 << 20)
    xg = to_gpu(x)
    rows = sorted({0, 1, M // 2, M - 1} | set(range(3, M, 29)))
    ran = 0
    for S in (5, 7, 9, 12):
        for finish in (1, 2):
            st = fp.set_tiling(M, _wres(S, finish))
            if st != P.FP_OK:
                # a slice longer than the LDS holds (few slices, many tokens)
                assert st == P.FP_ERR_UNSUPPORTED, (M, S, st)
                continue
            ran += 1
            label = "wres M=%d S=%d finish=%d" % (M, S, finish)
            ys = fp(xg)
            assert_matches_oracle(ys, x, ws, rows=rows, label=label)
            assert_bitwise_equal(ys, fp.forward_separate(xg), label + " fused/sep")
            assert_bitwise_equal(ys, fp(xg), label + " repeat")
            assert fp.set_tiling(M, _ring(3 if M > 128 else 4, S, finish)) == P.FP_OK
            assert_bitwise_equal(ys, fp(xg), label + " vs ring tile kernel")
    assert ran >= 2, M
    fp.set_tiling(M, None)


def test_weight_resident_tile_kernel_ragged_rows():
    # row counts that leave a partial 64-row block and 16-row tile, K with a
    # partial last stage (K = 5120 + 32)
    K, N, M = 5152, (100, 37, 200), 48
    x, ws = si.make_case(K, N, "bf16", M, seed=5)
    fp = _plan(ws, max_M=64, workspace_bytes=32 << 20)
    xg = to_gpu(x)
    for S in (6, 9):
        for finish in (1, 2):
            assert fp.set_tiling(M, _wres(S, finish)) == P.FP_OK
            ys = fp(xg)
            assert_matches_oracle(ys, x, ws, label="wres ragged S=%d f=%d" % (S, finish))
            assert_bitwise_equal(ys, fp.forward_separate(xg), "wres ragged fused/sep")
    fp.set_tiling(M, None)


# ---- outputs that start 2 bytes past an 8-byte boundary: the tile kernels
#      store four rows of one token as one 8-byte run only where the address
#      allows it and fall back to one store per row elsewhere, with the same
#      values (both finishes and the unsplit ring launch)
@pytest.mark.parametrize("M", [17, 32, 64, 128])
def test_tile_outputs_at_two_byte_offsets(M):
    x, ws = si.workload_case("crossover", M, 13)
    fp = _plan(ws, max_M=128, workspace_bytes=64 << 20)
    xg = to_gpu(x)
    rows = sorted({0, 1, M // 2, M - 1})
    cases = [None, _ring(4, 1, 1), _ring(4, 9, 1), _ring(4, 9, 2), _wres(9, 1), _wres(9, 2)]
    for t in cases:
        if fp.set_tiling(M, t) != P.FP_OK:
            assert t is not None and t[2] == 2, (M, t)  # weight-resident slices too long
            continue
        label = "outputs at +2 bytes M=%d tiling %s" % (M, t)
        ref = fp(xg)
        assert_matches_oracle(ref, x, ws, rows=rows, label=label)
        bufs = [torch.full((M * n + 1,), float("nan"), dtype=torch.bfloat16, device=xg.device)
                for n in fp.N]
        out = [b[1:].view(M, n) for b, n in zip(bufs, fp.N)]
        assert all(o.data_ptr() % 8 == 2 for o in out)
        fp.forward(xg, out=out)
        assert_bitwise_equal(out, ref, label)
        assert all(torch.isnan(b[0]) for b in bufs), label + ": wrote before the output"
    fp.set_tiling(M, None)


# ---- the pages' own fused-A shapes at hidden 6144 (pinned as concatenation
#      shapes in tests/golden/page_shapes.txt): 2624 rows = 2048 + 512 + 64,
#      and 2784 rows with the 160 indexer rows appended as a fourth
#      projection; every token count the fused call serves by default up to
#      16, each kernel on these row counts, and graph replay of the 2784-row
#      plan
def _page_shape(name):
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "page_shapes.txt")
    for ln in open(path):
        f = ln.split()
        if f and f[0] == name:
            eq = f.index("=")
            return int(f[1]), tuple(int(v) for v in f[2:eq])
    raise KeyError(name)


@pytest.mark.parametrize("name", ["glm_fused_a", "glm_fused_a_indexer"])
@pytest.mark.parametrize("M", [1, 3, 5, 8, 13, 16])
def test_page_fused_a_shapes_through_the_kernels(name, M):
    K, N = _page_shape(name)
    x, ws = si.make_case(K, N, "bf16", M, seed=31 + M)
    fp = _plan(ws, max_M=16)
    _check_case(fp, x, ws, "%s M=%d" % (name, M))


# M = 4: vector-ALU kernel; 8 and 16: small-M kernel with two row tiles per
# wave (one and two token halves); 32: ring tile kernel and the
# second-launch finish.  K = 7168 over 2112 rows at 12 tokens: the ring
# tile kernel with its in-launch finish.
@pytest.mark.parametrize("case,M", [("page", 4), ("page", 8), ("page", 16), ("page", 32),
                                    ("k7168", 12)])
def test_page_fused_a_indexer_shape_graph_replay(case, M):
    if case == "page":
        K, N = _page_shape("glm_fused_a_indexer")
    else:
        K, N = 7168, (1536, 576)
    x0, ws = si.make_case(K, N, "bf16", M, seed=40)
    fp = _plan(ws, max_M=max(8, M))
    xs = to_gpu(x0)
    outs = [torch.empty(M, n, dtype=BF16, device="cuda") for n in N]
    fp(xs, out=outs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fp(xs, out=outs)
    for seed in (41, 42, 43):
        xn, _ = si.make_case(K, N, "bf16", M, seed=seed)
        xs.copy_(to_gpu(xn))
        g.replay()
        torch.cuda.synchronize()
        assert_bitwise_equal(outs, fp(xs), "%s replay M=%d seed %d" % (case, M, seed))
        assert_matches_oracle(outs, xn, ws, label="%s replay M=%d" % (case, M))


# ---- plans past one round of small-M or tile workgroups: the ring tile
#      kernel from 9 tokens on the three-way fused-A shape, and the tile
#      kernels where a two-half small-M workgroup would exceed its thread
#      bound (K = 7168); defaults, against the oracle
@pytest.mark.parametrize("M", [9, 16, 17, 32, 48, 64])
def test_three_way_defaults_above_eight_tokens(M):
    x, ws = si.make_case(6144, (2048, 576, 128), "bf16", M, seed=90 + M)
    fp = _plan(ws, max_M=M)
    assert fp.query(M)[0] == (P.FP_PATH_MFMA_SMALL if M <= 16 else P.FP_PATH_MFMA)
    _check_case(fp, x, ws, "three-way default M=%d" % M)


@pytest.mark.parametrize("N", [(1536,), (1536, 576)])
@pytest.mark.parametrize("M", [9, 12, 16])
def test_long_k_two_halves_defaults(N, M):
    x, ws = si.make_case(7168, N, "bf16", M, seed=80 + M)
    fp = _plan(ws, max_M=16)
    assert fp.query(M)[0] == P.FP_PATH_MFMA
    _check_case(fp, x, ws, "K=7168 %s M=%d" % (N, M))


@pytest.mark.parametrize("K,N", [(5120, (1280, 512)), (3712, (5, 3585, 263))])
@pytest.mark.parametrize("M", [5, 8])
def test_fp32_long_rows_at_five_to_eight_tokens(K, N, M):
    """fp32 with long rows at 5..8 tokens: the row layout keeps to
    workgroups that fit the kernel's thread bound (these calls were refused
    while a seven-row layout that does not fit won on cost)."""
    x, ws = si.make_case(K, N, "f32", M, seed=300 + M, w_dist="normal_0.02")
    fp = _plan(ws, max_M=8)
    assert fp.query(M)[0] == P.FP_PATH_SKINNY
    _check_case(fp, x, ws, "f32 K=%d %s M=%d" % (K, N, M))


def _random_routing_cases(n, seed):
    """Seeded bf16 shapes (K a multiple of 8 from 64 to 8192, one to three
    projections of 4..4096 rows, at most 12M weight elements) and two token
    counts each, drawn around the kernels' boundaries."""
    rng = np.random.default_rng(seed)
    ms = [1, 2, 3, 4, 5, 7, 8, 9, 12, 16, 17, 24, 25, 31, 32, 33, 48, 64, 65, 96, 128]
    out = []
    while len(out) < n:
        K = 8 * int(round(np.exp(rng.uniform(np.log(8.0), np.log(1024.0)))))
        N = tuple(int(round(np.exp(rng.uniform(np.log(4.0), np.log(4096.0)))))
                  for _ in range(int(rng.integers(1, 4))))
        if sum(N) * K > 12_000_000:
            continue
        for M in rng.choice(ms, size=2, replace=False):
            out.append((K, N, int(M)))
    return out


@pytest.mark.parametrize("K,N,M", _random_routing_cases(40, 7) + _random_routing_cases(40, 11))
def test_default_routing_on_random_shapes(K, N, M):
    """Whatever kernel and layout the default routing picks for a shape no
    other test names: oracle parity (sampled token rows above 16), repeats
    and fused vs one launch per projection bitwise equal, with contiguous
    and strided activations."""
    # two in three cases read x through a padded row stride (ldx = K + 8 or
    # K + 16 elements, the pad filled with a sentinel)
    ldx = K + 8 * ((K + M) % 3)
    x, ws = si.make_case(K, N, "bf16", M, seed=K + M, ldx=ldx)
    fp = _plan(ws, max_M=max(8, M))
    rows = None if M <= 16 else sorted({0, 1, M // 2, M - 1} | set(range(3, M, 17)))
    _check_case(fp, x, ws, "K=%d ldx=%d N=%s M=%d %s" % (K, ldx, N, M, fp.get_tiling(M)),
                rows=rows)
