"""MosaicKV decode hot path for AMD Instinct MI355X (gfx950).

The C ABI is include/mkv.h, implemented by libmkv.so (HIP kernels + host
C++). `_lib` binds it 1:1 with ctypes; `cache.Cache` wraps device buffers
held in torch tensors. Importing `_lib` or `cache` loads libmkv.so and fails
if it is missing: there is no other implementation.
"""
__all__ = ["_lib", "cache", "layout", "bytes_model"]
