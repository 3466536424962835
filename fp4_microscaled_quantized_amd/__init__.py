"""fp4_microscaled_quantized_amd: fully-FP4 (MXFP4 / NVFP4) quantized linear
layer for AMD MI355X (gfx950).

The computation lives in ``libfp4mx.so`` (HIP kernels behind a C ABI declared
in ``include/fp4mx.h``); ``binding`` is its thin ctypes wrapper.
"""
from .binding import (COL, QUEST_CLIP, ROW, RTN, SR, FP4LinearFunction, LinearCtx, MXTensor, NVTensor,  # noqa: F401
                      gemm, gemm_bf16, gemm_unmask_irht, hadamard_quantize, hadamard_quantize_dual, lib, linear_bwd, linear_fwd,
                      nv_gemm, nv_linear_bwd, nv_linear_bwd_ctx, nv_linear_fwd, nv_linear_fwd_ctx, nv_msedn_quantize,
                      nv_msedn_requantize, NvCtx, nv_quantize46, nv_sr_quantize, quantize,
                      quest_linear_bwd, quest_linear_fwd, quest_quantize, QuestCtx, requantize, sign_mask,
                      unmask_inverse_hadamard)
