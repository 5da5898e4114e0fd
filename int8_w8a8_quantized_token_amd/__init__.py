"""MI355X-native (gfx950) W8A8 INT8 linear layer.

Per-token dynamic activation quantization, an int8 x int8 -> int32 MFMA GEMM
against per-output-channel int8 weights, and a dequantizing bf16 epilogue,
exposed through the C ABI in include/w8a8.h (libw8a8.so) and mirrored here
function for function.
"""
from .binding import (  # noqa: F401
    HIST_BINS,
    NOALLOC_MAX_BYTES,
    QUANT_LEVELS,
    W8A8Error,
    header_functions,
    lib,
    w8a8_abi_version,
    w8a8_activation_histogram,
    w8a8_calibrate_entropy,
    w8a8_calibrate_minmax,
    w8a8_channel_absmax,
    w8a8_fold_gamma,
    w8a8_gemm,
    w8a8_gemm_i32,
    w8a8_gptq_factor,
    w8a8_gptq_factor_workspace_bytes,
    w8a8_gptq_hessian,
    w8a8_gptq_quantize,
    w8a8_gptq_quantize_workspace_bytes,
    w8a8_linear,
    w8a8_linear_noalloc,
    w8a8_linear_static,
    w8a8_linear_workspace_bytes,
    w8a8_quantize_act,
    w8a8_quantize_act_static,
    w8a8_quantize_weight,
    w8a8_residual_add,
    w8a8_rmsnorm_quantize,
    w8a8_silu_mul_quantize,
    w8a8_smoothing_factors,
    w8a8_status_string,
)
