"""Views into the concatenated weight, in-place reloads and replaced weights.

"tinygemm2 for the DeepSeek-V4.1 hidden-state projections" (TensorRT-LLM
PR #20636), Description and Test Coverage: both Linear weights become views
of the concatenated tensor; a checkpoint reload writes through the views and
keeps the fused call; a replaced Parameter falls back to separate calls.
"""
import pytest
import torch

import synthetic_inputs as si
import projection_gemm_sparse_amd as P
from gpu_util import assert_bitwise_equal, assert_matches_oracle, to_gpu

pytestmark = pytest.mark.gpu


def _setup(name="crossover", M=4, max_M=128):
    x, ws = si.workload_case(name, M, 0)
    fp = P.FusedProjection([to_gpu(w) for w in ws], max_M=max_M)
    return fp, x, ws


def test_views_alias_the_concatenated_weight():
    fp, x, ws = _setup()
    assert len(fp.views) == 2
    for v, off, w in zip(fp.views, fp.offsets, ws):
        assert v.data_ptr() == fp.w_cat.data_ptr() + off * fp.K * fp.w_cat.element_size()
        assert v.is_contiguous() and tuple(v.shape) == tuple(w.shape)
        assert torch.equal(v.cpu().view(torch.int16), w.view(torch.int16))
    assert fp.offsets == [0, 1280]
    assert all(fp.aliases_intact(fp.views))


@pytest.mark.parametrize("M", [1, 4, 8, 32])
def test_inplace_reload_through_views_keeps_fused_path(M):
    fp, _, _ = _setup(M=M)
    # new checkpoint (new seed), written through the views in place
    x2, ws2 = si.workload_case("crossover", M, 77)
    for v, w in zip(fp.views, ws2):
        v.copy_(to_gpu(w))
    assert all(fp.aliases_intact(fp.views))
    ys = fp.forward_modules(to_gpu(x2), fp.views)
    assert_matches_oracle(ys, x2, ws2, label="reloaded M=%d" % M)
    assert_bitwise_equal(ys, fp(to_gpu(x2)), "reload fused")


def test_replaced_parameter_falls_back_to_separate():
    fp, x, ws = _setup(M=2)
    x2, ws2 = si.workload_case("crossover", 2, 5)
    new_wkv = to_gpu(ws2[1]).clone()  # a new tensor: no longer a view
    weights = [fp.views[0], new_wkv]
    assert fp.aliases_intact(weights) == [True, False]
    ys = fp.forward_modules(to_gpu(x), weights)
    # projection 0 from the view, projection 1 from the replacement
    assert_matches_oracle(ys, x, [ws[0], ws2[1]], label="replaced wkv")
    # and the view itself is untouched
    assert_bitwise_equal([fp.views[1]], [to_gpu(ws[1])], "view untouched")


def test_plan_destroy_and_stale_handle():
    fp, x, _ = _setup(M=1)
    plan = fp.plan
    fp.close()
    xg = to_gpu(x)
    outs = [torch.empty(1, n, dtype=torch.bfloat16, device="cuda") for n in fp.N]
    assert P.fp_forward(xg.data_ptr(), 1, fp.K, plan, 0,
                        [o.data_ptr() for o in outs]) == P.FP_ERR_INVALID_ARG
