"""int8 quantized linear layer for AMD Instinct MI355X (gfx950).

Python names match the C ABI of ``include/i8ql.h``.  The HIP library ``libi8ql.so`` is loaded
on first use (``load_library``); importing the package touches neither the GPU nor HIP.
"""
from ._binding import (EXPORTS, I8qlError, grouped_w8a16_gemm, load_library,  # noqa: F401
                       quantize_per_channel_int8, quantize_per_token_int8, w8a8_gemm,
                       w8a16_gemm)
