"""MI355X-native paged KV cache: paged KV append and PagedAttention decode / chunked prefill.

The compute path is the HIP library ``libpagedattn.so`` (gfx950 kernels behind a C ABI,
declared in ``include/pagedattn.h``); ``paged_kv_cache_461_amd.ops`` is a thin ctypes
binding over it.  ``workloads`` holds the seeded synthetic input generators.
"""
