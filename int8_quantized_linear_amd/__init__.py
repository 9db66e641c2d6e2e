"""int8 quantized linear layer for AMD Instinct MI355X (gfx950): Python binding.

The binding lives in ``_binding`` and is loaded on first use; importing this package does
not touch the GPU or the HIP library.
"""
