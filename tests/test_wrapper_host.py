"""The torch-side wrapper's host logic (no GPU): tensors it allocates for
work enqueued on a caller's stream are held for that stream, so the caching
allocator cannot reuse their memory before the work has run."""
import torch

import projection_gemm_sparse_amd as P
from projection_gemm_sparse_amd import fused
from projection_gemm_sparse_amd import _lib as L


class _Stream:
    """Stands in for a torch.cuda.Stream (has a cuda_stream handle)."""
    cuda_stream = 12345


class _Tensor:
    """A device tensor stand-in: records record_stream calls."""
    def __init__(self, ptr):
        self.ptr, self.held = ptr, []

    def data_ptr(self):
        return self.ptr

    def record_stream(self, s):
        self.held.append(s)


def _bare(monkeypatch, calls):
    fp = object.__new__(P.FusedProjection)
    fp.N, fp.K, fp.row_cols, fp.plan = [4, 2], 8, 8, 777
    fp.w_dtype = torch.bfloat16
    fp.dtype = fp.out_dtype = torch.bfloat16
    fp.device = torch.device("cpu")
    monkeypatch.setattr(fp, "_check_x", lambda x: None)
    monkeypatch.setattr(L, "fp_forward_separate",
                        lambda *a: calls.append(("separate",) + a) or L.FP_OK)
    monkeypatch.setattr(L, "fp_forward", lambda *a: calls.append(("fused",) + a) or L.FP_OK)
    return fp


def test_replaced_weight_temporary_is_held_for_the_stream(monkeypatch):
    calls = []
    fp = _bare(monkeypatch, calls)
    tmp = _Tensor(0x2000)

    class _W:
        """A replaced, non-contiguous weight: .detach().contiguous() makes tmp."""
        shape, dtype, device = (2, 8), torch.bfloat16, torch.device("cpu")

        def detach(self):
            return self

        def contiguous(self):
            return tmp

    monkeypatch.setattr(fp, "aliases_intact", lambda ws: [True, False])
    monkeypatch.setattr(fp, "forward_separate",
                        lambda x, out=None, w_override=None, stream=None:
                        calls.append(("sep", w_override, stream)) or out)
    s = _Stream()
    fp.forward_modules(object(), [object(), _W()], out=["y0", "y1"], stream=s)
    assert calls[-1][1][1] is tmp and calls[-1][2] is s
    assert tmp.held == [s]


def test_outputs_allocated_for_another_stream_are_held(monkeypatch):
    held = []
    monkeypatch.setattr(fused, "_hold_for_stream", lambda ts, st: held.append((list(ts), st)))
    calls = []
    fp = _bare(monkeypatch, calls)
    s = _Stream()
    ys = fp._outputs(3, None, s)
    assert [tuple(y.shape) for y in ys] == [(3, 4), (3, 2)]
    assert held and held[-1][1] is s and len(held[-1][0]) == 2
    # caller-provided outputs are the caller's to keep alive
    held.clear()
    assert fp._outputs(3, ["a", "b"], s) == ["a", "b"]
    assert not held


def test_hold_is_a_no_op_on_the_current_stream():
    t = _Tensor(1)
    fused._hold_for_stream([t], None)
    fused._hold_for_stream([t], 0x1234)  # a raw handle: nothing to record on
    assert t.held == []
    s = _Stream()
    fused._hold_for_stream([t, None], s)
    assert t.held == [s]
