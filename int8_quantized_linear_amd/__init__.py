"""int8 quantized linear layer for AMD Instinct MI355X (gfx950).

Python names match the C ABI of ``include/i8ql.h``.  The HIP library ``libi8ql.so`` is loaded
on first use (``load_library``); importing the package touches neither the GPU nor HIP.
"""
from ._binding import (EXPORTS, GROUP_SIZE, NORM_MAX_K, ROUTE_MAX_EXPERTS,  # noqa: F401
                       ROUTE_MAX_K, SILU_MAX_N, rmsnorm_bf16,
                       rmsnorm_quantize_per_token_int8, silu_mul_bf16,
                       silu_mul_quantize_per_token_int8,
                       W8A8_MAX_SPLITS, W8A8_NUM_CONFIGS, W8A8_SCRATCH_BYTES, I8qlError,
                       grouped_w8a16_gemm,
                       grouped_w8a16_silu_gemm, load_library, moe_combine, moe_route_topk,
                       quantize_per_channel_int8, quantize_per_group_int8,
                       quantize_per_token_int8, quantize_per_token_int8_multi, w8a8_gemm,
                       w8a8_gemm_choose_config,
                       w8a8_gemm_choose_plan, w8a8_gemm_config_info, w8a8_gemm_g128,
                       w8a8_gemm_noalloc,
                       w8a8_gemm_with_config,
                       w8a8_gemm_with_plan, w8a8_gemm_workspace_size, w8a8_workspace,
                       w8a16_gemm, w8a16_gemm_g128)
