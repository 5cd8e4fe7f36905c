"""FP8-Dynamic quantized linear layer for AMD MI355X (gfx950).

The compute path is the HIP library libfp8dq.so (C-ABI declared in
include/fp8dq.h); this package only builds it and marshals torch tensors to
it. Entry points keep the C names:

    fp8_quant_act, fp8_quant_weight_block, fp8_gemm, fp8_gemm_block,
    fp8_linear, fp8_linear_block, fp8_linear_noalloc, fp8_workspace_bytes,
    fp8_status_string,
    fp8_silu_mul_quant, fp8_rmsnorm_quant, fp8_silu_mul, fp8_rmsnorm,
    fp8_calib_scale,
    fp8_calib_workspace_bytes, fp8_quant_static, fp8_kv_cache_quant

lm_head is not quantized by this method; nothing here applies to it.
"""
from ._binding import (  # noqa: F401
    AUTO, DECODE_MAX_M, FORCE_DECODE, FORCE_PREFILL, GROUP, RMS_EPS, Fp8dqError,
    fp8_calib_scale, fp8_calib_workspace_bytes, fp8_gemm, fp8_gemm_block,
    fp8_kv_cache_quant, fp8_linear, fp8_linear_block, fp8_linear_noalloc, fp8_quant_act,
    fp8_quant_static,
    fp8_quant_weight_block, fp8_rmsnorm, fp8_rmsnorm_quant, fp8_silu_mul, fp8_silu_mul_quant,
    fp8_status_string,
    fp8_workspace_bytes, fp8dq_version, header_functions, lib,
)
