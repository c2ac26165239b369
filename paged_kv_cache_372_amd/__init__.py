"""Paged-KV decode attention for AMD MI355X (gfx950).

The compute path is a C-ABI library of hand-written HIP kernels
(``libpagedkv.so``); this package holds its Python binding and the host-side
block manager.  Importing the package does not load the library: the first
call into ``paged_kv_cache_372_amd.ops`` does, and fails loudly if it has not
been built.
"""
__all__ = ["blocks", "ops"]
