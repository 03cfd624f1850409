"""NVFP4 W4A4 quantized linear and routed-expert MoE for MI355X (gfx950).

The compute lives in ``libnvfp4.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/nvfp4.h``).  ``moe_nvfp4_quantize_amd.nvfp4`` is the thin
Python binding over it; importing this package does not load the library, so the
input generators in ``workloads`` work on a machine without a GPU.
"""

__all__ = ["nvfp4", "workloads"]
