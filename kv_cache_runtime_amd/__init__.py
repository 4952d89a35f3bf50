"""Paged, folded causal attention for AMD Instinct MI355X (gfx950).

The compute lives in libatlas.so (HIP kernels behind the C ABI declared in
include/atlas.h); `kv_cache_runtime_amd.atlas` is its ctypes binding.
"""
