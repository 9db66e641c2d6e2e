"""int8 quantized linear layer for AMD Instinct MI355X (gfx950).

Python names match the C ABI of ``include/i8ql.h``.  The HIP library ``libi8ql.so`` is loaded
on first use (``load_library``); importing the package touches neither the GPU nor HIP.
"""
from ._binding import (EXPORTS, W8A8_NUM_CONFIGS, I8qlError, grouped_w8a16_gemm,  # noqa: F401
                       load_library, quantize_per_channel_int8, quantize_per_token_int8,
                       w8a8_gemm, w8a8_gemm_choose_config, w8a8_gemm_config_info,
                       w8a8_gemm_with_config, w8a16_gemm)
