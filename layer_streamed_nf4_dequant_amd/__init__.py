"""Exact layer-streamed NF4 LoRA on MI355X (gfx950).

The compute path lives in the native library ``liblsnf4.so`` (HIP kernels for gfx950 behind a
C ABI declared in ``include/lsnf4.h``); ``layer_streamed_nf4_dequant_amd.lib`` is a thin ctypes
binding to it.  PyTorch is used only to own device memory and streams.  There is no CPU
fallback: if the native library is missing, every call raises.

Submodules are imported on demand so that the input generators and configs can be used
without loading the native library.
"""

__all__ = ["configs", "inputs", "lib", "stack"]
