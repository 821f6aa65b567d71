"""MI355X-native fused decode-time hidden-state projection.

Several linear projections that read the same activations have their weights
row-concatenated once into one buffer; one skinny GEMM computes all of them
and returns each projection as a dense [M, N_i] tensor ("tinygemm2 for the
DeepSeek-V4.1 hidden-state projections", TensorRT-LLM PR #20636,
Description).  The compute path is libfusedproj (HIP kernels for gfx950,
C ABI in include/fusedproj.h); this package binds it and owns device memory
through torch.  Importing it fails if the library is not built.
"""
from . import _lib
from ._lib import (FP_BF16, FP_F32, FP_MXFP8, FP_MXFP4, FP_NVFP4, FP_OK, FP_ERR_INVALID_ARG, FP_ERR_UNSUPPORTED,
                   FP_ERR_HIP, FP_ERR_WORKSPACE, FP_PATH_NONE, FP_PATH_SKINNY,
                   FP_PATH_SKINNY_SPLITK, FP_PATH_MFMA, FP_PATH_MFMA_SMALL, FP_MAX_M, FP_MAX_PROJ,
                   FusedProjError, LIB_PATH, fp_workspace_bytes, fp_plan_create,
                   fp_plan_view, fp_plan_destroy, fp_supported, fp_forward,
                   fp_forward_separate, fp_forward_rmsnorm, fp_mxfp8_to_bf16,
                   fp_mxfp4_to_bf16, fp_nvfp4_to_bf16, fp_plan_set_tensor_scales,
                   fp_stream_read, fp_stream_read_shaped, fp_forward_noalloc,
                   fp_forward_swiglu, fp_rmsnorm, fp_swiglu, fp_plan_query, fp_plan_set_out_dtype,
                   fp_plan_set_mfma_min_m,
                   fp_plan_set_tiling, fp_plan_get_tiling, fp_default_tiling,
                   fp_status_str, fp_last_hip_error)
from .fused import FusedProjection

__all__ = [n for n in dir() if not n.startswith("__")]
