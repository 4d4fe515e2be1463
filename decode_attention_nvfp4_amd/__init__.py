"""NVFP4 KV cache for AMD Instinct MI355X (gfx950).

The compute path is a C-ABI shared library (``libnvfp4kv.so``, hand-written
HIP kernels) declared in ``include/nvfp4kv.h``; ``decode_attention_nvfp4_amd.api``
is a thin ctypes binding over it that takes PyTorch device tensors.  Importing
this package loads nothing; the library is loaded on first use and its absence
raises an error (there is no CPU fallback).
"""

__all__ = ["api", "workloads"]
