"""Torch-side owner of a fused projection plan.

The load-time half of "tinygemm2 for the DeepSeek-V4.1 hidden-state
projections" (TensorRT-LLM PR #20636), Description: the projection weights
that read the same activations are copied once into one row-concatenated
buffer, and every projection gets a view into it (no second copy is kept);
checkpoint reloads that write through the views keep the fused path valid,
while a weight that no longer aliases its view (a replaced Parameter) is
served by the one-launch-per-projection path with that weight.

Torch only allocates device memory (the concatenated weight, the workspace
and the outputs) and supplies the stream; every arithmetic step runs in
libfusedproj's HIP kernels through the C ABI.
"""
from __future__ import annotations

import torch

from . import _lib as L

_DTYPES = {torch.bfloat16: L.FP_BF16, torch.float32: L.FP_F32}
# MXFP8 weights arrive as packed uint8 rows: K E4M3 codes, then K/32 E8M0
# scales (K + K/32 bytes per row)


def _stream_handle(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return int(s.cuda_stream)


def _hold_for_stream(tensors, stream) -> None:
    """Tensors allocated here (on the current stream's pool) and used by work
    enqueued on another ``stream``: mark them in use by that stream, so the
    caching allocator does not hand their memory out again before that work
    has run (torch's record_stream)."""
    if stream is None or not hasattr(stream, "cuda_stream"):
        return
    for t in tensors:
        if t is not None:
            t.record_stream(stream)


class FusedProjection:
    """Fuses projections ``weights[i]`` ([N_i, K], one dtype, on one GPU).

    ``copy_weights=True`` copies the given tensors into the concatenated
    buffer; the caller may then rebind its module weights to ``views``.
    MXFP8 weights are uint8 tensors of packed rows [N_i, K + K/32] (the K
    E4M3 codes, then the K/32 E8M0 scales), MXFP4 weights packed rows
    [N_i, K/2 + K/32] (two E2M1 codes per byte, low nibble first, then the
    scales), NVFP4 weights packed rows [N_i, K/2 + K/16] (two E2M1 codes
    per byte, low nibble first, then one E4M3 scale per 16 elements) with
    one fp32 ``tensor_scales[i]`` per projection (default 1);
    ``weight_format`` ("mxfp8", "mxfp4" or "nvfp4") names the format of
    uint8 weights when their width does not tell it.  Activations and
    outputs are then bf16.
    """

    def __init__(self, weights, max_M: int = 8, stream=None, copy_weights: bool = True,
                 workspace_bytes: int | None = None, out_dtype=None,
                 weight_format: str | None = None, tensor_scales=None):
        if not weights:
            raise ValueError("at least one projection")
        w0 = weights[0]
        if w0.dtype not in _DTYPES and w0.dtype != torch.uint8:
            raise TypeError("weights must be bfloat16, float32 or packed MXFP8 (uint8), got %s"
                            % w0.dtype)
        if not w0.is_cuda:
            raise ValueError("weights must be on a GPU")
        self.w_dtype = w0.dtype
        if w0.dtype == torch.uint8:
            cols = int(w0.shape[1])
            fits = {"mxfp8": cols % 33 == 0, "mxfp4": cols % 17 == 0, "nvfp4": cols % 9 == 0}
            fmt = weight_format
            if fmt is None:
                cand = [f for f, ok in fits.items() if ok]
                if len(cand) != 1:
                    raise ValueError("packed rows of %d bytes: pass weight_format" % cols)
                fmt = cand[0]
            if fmt not in fits or not fits[fmt]:
                raise ValueError("packed %s rows cannot be %d bytes wide" % (fmt, cols))
            self.dtype = torch.bfloat16  # activations and outputs
            self.fp_dtype = {"mxfp8": L.FP_MXFP8, "mxfp4": L.FP_MXFP4,
                             "nvfp4": L.FP_NVFP4}[fmt]
            self.K = {"mxfp8": cols // 33 * 32, "mxfp4": cols // 17 * 32,
                      "nvfp4": cols // 9 * 16}[fmt]
        else:
            self.dtype = w0.dtype
            self.fp_dtype = _DTYPES[w0.dtype]
            self.K = int(w0.shape[1])
        self.device = w0.device
        self.row_cols = int(w0.shape[1])
        self.N = [int(w.shape[0]) for w in weights]
        for w in weights:
            if w.dtype != self.w_dtype or w.device != self.device or w.dim() != 2 \
                    or int(w.shape[1]) != self.row_cols:
                raise ValueError("all weights must be [N_i, K] of one dtype on one device")
        self.max_M = int(max_M)
        self.n_total = sum(self.N)
        # plan creation under no_grad: the concatenated buffer must not keep
        # an autograd graph alive (lesson of PR #20502's commit log)
        with torch.no_grad():
            self.w_cat = torch.empty(self.n_total, self.row_cols, dtype=self.w_dtype,
                                     device=self.device)
            self.ws_bytes = L.fp_workspace_bytes(self.fp_dtype, self.K, self.N, self.max_M)
            if self.ws_bytes == 0:
                raise L.FusedProjError(L.FP_ERR_INVALID_ARG, "fp_workspace_bytes")
            if workspace_bytes is not None:
                # a larger workspace admits tilings with more K splits
                self.ws_bytes = max(self.ws_bytes, int(workspace_bytes))
            self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
            src = None
            if copy_weights:
                keep = [w.detach().contiguous() for w in weights]  # alive until copied
                src = [w.data_ptr() for w in keep]
            st, plan = L.fp_plan_create(self.fp_dtype, self.K, self.N, src,
                                        self.w_cat.data_ptr(), self.workspace.data_ptr(),
                                        self.ws_bytes, self.max_M, _stream_handle(stream))
            L.check(st, "fp_plan_create")
            if copy_weights:
                # the copies are stream-ordered; keep the sources alive until done
                (torch.cuda.current_stream() if stream is None else stream).synchronize()
                del keep
        self.plan = plan
        self.tensor_scales = None
        if tensor_scales is not None:
            if len(tensor_scales) != len(self.N):
                raise ValueError("one tensor scale per projection")
            L.check(L.fp_plan_set_tensor_scales(plan, list(tensor_scales)),
                    "fp_plan_set_tensor_scales")
            self.tensor_scales = [float(v) for v in tensor_scales]
        self.out_dtype = self.dtype if out_dtype is None else out_dtype
        if self.out_dtype != self.dtype:
            if self.out_dtype not in _DTYPES:
                raise TypeError("out_dtype must be bfloat16 or float32")
            L.check(L.fp_plan_set_out_dtype(plan, _DTYPES[self.out_dtype]),
                    "fp_plan_set_out_dtype")
        self.offsets = []
        self.views = []
        for i in range(len(self.N)):
            st, ptr, off, rows = L.fp_plan_view(plan, i)
            L.check(st, "fp_plan_view")
            view = self.w_cat.narrow(0, off, rows)
            assert view.data_ptr() == ptr
            self.offsets.append(off)
            self.views.append(view)

    # ----------------------------------------------------------------- guard
    def aliases_intact(self, weights) -> list:
        """Per projection: does ``weights[i]`` still alias its view (same
        storage address, shape and dense strides)?  A replaced Parameter
        fails this and must go to the separate path with an override."""
        out = []
        for w, v in zip(weights, self.views):
            out.append(w.data_ptr() == v.data_ptr() and tuple(w.shape) == tuple(v.shape)
                       and w.stride() == v.stride() and w.dtype == v.dtype)
        return out

    def supported(self, x: torch.Tensor) -> bool:
        if x.dim() != 2 or x.dtype != self.dtype or x.device != self.device \
                or x.stride(1) != 1 or int(x.shape[1]) != self.K:
            return False
        return L.fp_supported(self.plan, int(x.shape[0]), x.data_ptr(), int(x.stride(0))) == L.FP_OK

    # ---------------------------------------------------------------- calls
    def _outputs(self, M: int, out, stream=None):
        if out is not None:
            return out
        ys = [torch.empty(M, n, dtype=self.out_dtype, device=self.device) for n in self.N]
        _hold_for_stream(ys, stream)
        return ys

    def _check_x(self, x):
        if x.dim() != 2 or int(x.shape[1]) != self.K or x.stride(1) != 1:
            raise ValueError("x must be [M, K] with unit column stride")
        if x.dtype != self.dtype or x.device != self.device:
            raise ValueError("x dtype/device differ from the plan's")

    def forward(self, x: torch.Tensor, out=None, stream=None):
        """Fused call: returns one dense [M, N_i] tensor per projection."""
        self._check_x(x)
        M = int(x.shape[0])
        ys = self._outputs(M, out, stream)
        st = L.fp_forward(x.data_ptr(), M, int(x.stride(0)), self.plan,
                          _stream_handle(stream), [y.data_ptr() for y in ys])
        L.check(st, "fp_forward")
        return ys

    __call__ = forward

    def forward_separate(self, x: torch.Tensor, out=None, w_override=None, stream=None):
        """One launch per projection; ``w_override[i]`` (a [N_i, K] tensor)
        replaces projection i's view."""
        self._check_x(x)
        M = int(x.shape[0])
        ys = self._outputs(M, out, stream)
        ov = None
        if w_override is not None:
            ov = []
            for i, w in enumerate(w_override):
                if w is None:
                    ov.append(None)
                    continue
                if tuple(w.shape) != (self.N[i], self.row_cols) or not w.is_contiguous() \
                        or w.dtype != self.w_dtype or w.device != self.device:
                    raise ValueError("override %d must be a dense [%d, %d] tensor"
                                     % (i, self.N[i], self.row_cols))
                ov.append(w.data_ptr())
        st = L.fp_forward_separate(x.data_ptr(), M, int(x.stride(0)), self.plan,
                                   _stream_handle(stream), [y.data_ptr() for y in ys], ov)
        L.check(st, "fp_forward_separate")
        return ys

    def forward_modules(self, x: torch.Tensor, weights, out=None, stream=None):
        """Dispatch as a module would: the fused call while every weight
        aliases its view, else the separate path with the replaced weights."""
        intact = self.aliases_intact(weights)
        if all(intact):
            return self.forward(x, out=out, stream=stream)
        ov = [None if ok else w.detach().contiguous() for ok, w in zip(intact, weights)]
        # a non-contiguous replaced weight gets a contiguous temporary that
        # the separate launches on `stream` read after this call returns
        _hold_for_stream([t for t, w in zip(ov, weights) if t is not None and t is not w],
                         stream)
        return self.forward_separate(x, out=out, w_override=ov, stream=stream)

    # ------------------------------------------------------------ epilogues
    def _gains(self, gammas):
        if len(gammas) != len(self.N):
            raise ValueError("one gain (or None) per projection")
        ptrs = []
        for i, g in enumerate(gammas):
            if g is None:
                ptrs.append(None)
                continue
            if g.dtype != torch.bfloat16 or g.device != self.device or g.dim() != 1 \
                    or int(g.shape[0]) != self.N[i] or not g.is_contiguous():
                raise ValueError("gain %d must be a dense bf16 [%d] tensor" % (i, self.N[i]))
            ptrs.append(g.data_ptr())
        return ptrs

    def forward_rmsnorm(self, x: torch.Tensor, gammas, eps: float, out=None, stream=None):
        """Fused projection + RMSNorm: projection i is normalised with gain
        ``gammas[i]`` (bf16 [N_i]) or returned as is when that entry is None."""
        self._check_x(x)
        M = int(x.shape[0])
        ys = self._outputs(M, out, stream)
        st = L.fp_forward_rmsnorm(x.data_ptr(), M, int(x.stride(0)), self.plan,
                                  _stream_handle(stream), self._gains(gammas), eps,
                                  [y.data_ptr() for y in ys])
        L.check(st, "fp_forward_rmsnorm")
        return ys

    def forward_rmsnorm_separate(self, x: torch.Tensor, gammas, eps: float, stream=None):
        """The unfused chain: one projection launch per projection, then one
        RMSNorm launch per normalised projection (in place)."""
        ptrs = self._gains(gammas)
        ys = self.forward_separate(x, stream=stream)
        M = int(x.shape[0])
        for i, g in enumerate(ptrs):
            if g is None:
                continue
            st = L.fp_rmsnorm(ys[i].data_ptr(), M, self.N[i], g, eps, ys[i].data_ptr(),
                              _stream_handle(stream))
            L.check(st, "fp_rmsnorm")
        return ys

    def forward_swiglu(self, x: torch.Tensor, out=None, stream=None):
        """Fused gate/up + SwiGLU (a plan of two equal-width projections,
        gate first): returns h, dense [M, N]."""
        self._check_x(x)
        M = int(x.shape[0])
        h = out
        if h is None:
            h = torch.empty(M, self.N[0], dtype=self.dtype, device=self.device)
            _hold_for_stream([h], stream)
        st = L.fp_forward_swiglu(x.data_ptr(), M, int(x.stride(0)), self.plan,
                                 _stream_handle(stream), h.data_ptr())
        L.check(st, "fp_forward_swiglu")
        return h

    def forward_swiglu_separate(self, x: torch.Tensor, stream=None):
        """The unfused chain: gate and up launches, then one SwiGLU launch
        (written over the gate output)."""
        g, u = self.forward_separate(x, stream=stream)
        M = int(x.shape[0])
        st = L.fp_swiglu(g.data_ptr(), u.data_ptr(), M, self.N[0], g.data_ptr(),
                         _stream_handle(stream))
        L.check(st, "fp_swiglu")
        return g

    # ----------------------------------------------------------- tuning/query
    def query(self, M: int):
        st, path, lf, ls = L.fp_plan_query(self.plan, M)
        L.check(st, "fp_plan_query")
        return path, lf, ls

    def set_tiling(self, M: int, tiling) -> int:
        return L.fp_plan_set_tiling(self.plan, M, tiling)

    def get_tiling(self, M: int, n_rows: int | None = None):
        st, t = L.fp_plan_get_tiling(self.plan, M, self.n_total if n_rows is None else n_rows)
        L.check(st, "fp_plan_get_tiling")
        return t

    def set_mfma_min_m(self, m: int) -> None:
        L.check(L.fp_plan_set_mfma_min_m(self.plan, m), "fp_plan_set_mfma_min_m")

    def close(self) -> None:
        if getattr(self, "plan", None) is not None:
            L.fp_plan_destroy(self.plan)
            self.plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
