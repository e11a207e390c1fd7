"""MI355X-native paged decode attention.

The compute path is a C-ABI HIP library built for gfx950
(``libpa_gfx950.so`` next to this file; declarations in ``include/pa.h``).
:mod:`paged_kv_cache_331_amd.pa` is a thin ctypes binding over it: argument
marshalling only. :mod:`paged_kv_cache_331_amd.workloads` draws the seeded
synthetic inputs.
"""
__all__ = ["pa", "workloads"]
