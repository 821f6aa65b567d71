"""fp_forward_noalloc: the fused call with its split-K state in the
library's static device scratch instead of the plan's workspace.

It must give fp_forward's outputs bit for bit (same tilings, same kernels),
on consecutive calls whose sizes shrink (the scratch keeps the previous
call's partials and must leave its counters at zero), across plans of
different row counts sharing the one scratch, and refuse a call whose
split-K partials do not fit, with no launch.  Every call goes through the
C ABI."""
import pytest
import torch

import synthetic_inputs as si
import projection_gemm_sparse_amd as P
from gpu_util import assert_bitwise_equal, assert_matches_oracle, to_gpu

pytestmark = pytest.mark.gpu


def _calls(fp, x, M):
    """fp_forward and fp_forward_noalloc on the same input, into separate
    outputs; returns both output lists."""
    L = P._lib
    dt = fp.out_dtype
    ya = [torch.full((M, n), 7.0, dtype=dt, device="cuda") for n in fp.N]
    yb = [torch.full((M, n), -7.0, dtype=dt, device="cuda") for n in fp.N]
    h = torch.cuda.current_stream().cuda_stream
    L.check(L.fp_forward(x.data_ptr(), M, x.stride(0), fp.plan, h, [y.data_ptr() for y in ya]),
            "fp_forward")
    L.check(L.fp_forward_noalloc(x.data_ptr(), M, x.stride(0), fp.plan, h,
                                 [y.data_ptr() for y in yb]), "fp_forward_noalloc")
    torch.cuda.synchronize()
    return ya, yb


def _rows(M):
    return None if M <= 16 else sorted({0, M // 2, M - 1})


@pytest.mark.parametrize("name,Ms,tiling", [
    # ring tile kernel (second-launch finish), then the tile kernel with an
    # in-launch finish (arrival counters), then the small-M kernel (no split)
    ("crossover", (64, 20, 4), None),
    # fp32 indexer with a forced skinny K split (partials + counters)
    ("indexer_f32", (8, 3), (P.FP_PATH_SKINNY_SPLITK, 7, 1, 4, 0, 0)),
    # three-way fused-A (2752 rows): ring tile kernel with 9 slices and the
    # second-launch finish, then its in-launch finish, then the small-M
    # kernel with two row tiles per wave
    ("fused_a_3way", (64, 16, 8), None),
])
def test_noalloc_equals_fp_forward_on_shrinking_calls(name, Ms, tiling):
    x0, ws = si.workload_case(name, max(Ms), 0)
    # forced split tilings need more workspace than the defaults
    fp = P.FusedProjection([to_gpu(w) for w in ws], max_M=max(8, max(Ms)),
                           workspace_bytes=1 << 20)
    for M in Ms:
        if tiling is not None:
            P._lib.check(fp.set_tiling(M, tiling), "set_tiling")
    for M in Ms:
        xc, _ = si.workload_case(name, M, 40 + M)
        x = to_gpu(xc)
        ya, yb = _calls(fp, x, M)
        assert_bitwise_equal(ya, yb, "%s M=%d noalloc vs fp_forward" % (name, M))
        assert_matches_oracle(yb, xc, ws, rows=_rows(M), label="%s M=%d noalloc" % (name, M))
    fp.close()


def test_plans_of_different_rows_share_the_scratch():
    # a 2752-row plan, then a 1792-row plan, then the first again, each with
    # split tile launches: every call's counters must start at zero
    xa0, wsa = si.workload_case("fused_a_3way", 32, 0)
    xb0, wsb = si.workload_case("crossover", 32, 0)
    fa = P.FusedProjection([to_gpu(w) for w in wsa], max_M=32)
    fb = P.FusedProjection([to_gpu(w) for w in wsb], max_M=32)
    assert fa.get_tiling(32)[3] > 1 and fb.get_tiling(32)[3] > 1 and fa.get_tiling(17)[3] > 1
    for fp, ws, name, M in ((fa, wsa, "fused_a_3way", 32), (fb, wsb, "crossover", 32),
                            (fa, wsa, "fused_a_3way", 17)):
        xc, _ = si.workload_case(name, M, 90 + M)
        ya, yb = _calls(fp, to_gpu(xc), M)
        assert_bitwise_equal(ya, yb, "%s M=%d shared scratch" % (name, M))
        assert_matches_oracle(yb, xc, ws, rows=_rows(M), label="%s M=%d shared" % (name, M))
    fa.close()
    fb.close()


def test_partials_beyond_the_scratch_are_refused_without_launch():
    # 12 K slices of the ring tile kernel at 256 tokens on 2752 rows:
    # 12 * 2752 * 256 * 4 B = 33.8 MB of partials, more than the scratch
    # holds (the plan's own workspace is made large enough for fp_forward)
    x0, ws = si.workload_case("fused_a_3way", 1, 0)
    fp = P.FusedProjection([to_gpu(w) for w in ws], max_M=256, workspace_bytes=40 << 20)
    M = 256
    P._lib.check(fp.set_tiling(M, (P.FP_PATH_MFMA, 4, 3, 12, 0, 0)), "set_tiling")
    x = torch.zeros(M, fp.K, dtype=torch.bfloat16, device="cuda")
    sentinel = [torch.full((M, n), 3.0, dtype=torch.bfloat16, device="cuda") for n in fp.N]
    h = torch.cuda.current_stream().cuda_stream
    st = P._lib.fp_forward_noalloc(x.data_ptr(), M, fp.K, fp.plan, h,
                                   [y.data_ptr() for y in sentinel])
    torch.cuda.synchronize()
    assert st == P.FP_ERR_WORKSPACE
    for y in sentinel:
        assert bool((y == 3.0).all()), "a refused call wrote its outputs"
    fp.close()


def _random_cases(n, seed):
    """Seeded bf16 shapes (K a multiple of 8 from 64 to 8192, one to three
    projections of 4..4096 rows, at most 12M weight elements) with a token
    count around the kernels' boundaries."""
    import numpy as np
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        K = 8 * int(round(np.exp(rng.uniform(np.log(8.0), np.log(1024.0)))))
        N = tuple(int(round(np.exp(rng.uniform(np.log(4.0), np.log(4096.0)))))
                  for _ in range(int(rng.integers(1, 4))))
        if sum(N) * K > 12_000_000:
            continue
        out.append((K, N, int(rng.choice([5, 9, 17, 25, 32, 48, 64, 100, 128]))))
    return out


@pytest.mark.parametrize("K,N,M", _random_cases(12, 17))
def test_noalloc_on_random_shapes(K, N, M):
    """The default tiling of shapes no other test names: fp_forward's bits,
    or FP_ERR_WORKSPACE with the outputs untouched where the split-K
    partials exceed the scratch."""
    xc, ws = si.make_case(K, N, "bf16", M, seed=K + M)
    fp = P.FusedProjection([to_gpu(w) for w in ws], max_M=max(8, M))
    x = to_gpu(xc)
    L = P._lib
    ya = [torch.full((M, n), 7.0, dtype=torch.bfloat16, device="cuda") for n in fp.N]
    yb = [torch.full((M, n), -7.0, dtype=torch.bfloat16, device="cuda") for n in fp.N]
    h = torch.cuda.current_stream().cuda_stream
    L.check(L.fp_forward(x.data_ptr(), M, x.stride(0), fp.plan, h, [y.data_ptr() for y in ya]),
            "fp_forward")
    st = L.fp_forward_noalloc(x.data_ptr(), M, x.stride(0), fp.plan, h,
                              [y.data_ptr() for y in yb])
    torch.cuda.synchronize()
    label = "K=%d N=%s M=%d %s" % (K, N, M, fp.get_tiling(M))
    if st == P.FP_ERR_WORKSPACE:
        assert fp.get_tiling(M)[3] > 1, label
        for y in yb:
            assert bool((y == -7.0).all()), "a refused call wrote its outputs: " + label
    else:
        assert st == P.FP_OK, label
        assert_bitwise_equal(ya, yb, label + " noalloc vs fp_forward")
        assert_matches_oracle(yb, xc, ws, rows=_rows(M), label=label + " noalloc")
    fp.close()
