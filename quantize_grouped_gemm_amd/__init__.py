"""MXFP8 training hot path for MI355X (gfx950).

The compute lives in hand-written HIP kernels behind the C ABI declared in
``include/mxfp8.h`` (``libmxfp8.so``); ``quantize_grouped_gemm_amd.mx`` is the
thin Python binding over it. PyTorch is used only for device memory and
streams.
"""
