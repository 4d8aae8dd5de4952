"""cache_gather_amd — the sparse-KV hot-cache decode step on MI355X (gfx950).

`cache_gather_amd.hc` is the ctypes binding of the C-ABI library libhc.so
(include/hc.h); `cache_gather_amd.workload` draws the seeded synthetic inputs.
"""
