"""fp4_kv_cache_amd: paged decode attention over a 4-bit microscaling KV cache on MI355X (gfx950).

The compute lives in the C-ABI library ``libfp4kv.so`` (HIP kernels for
gfx950); ``fp4_kv_cache_amd.lib`` is the thin ctypes binding with the same
entry-point names.  ``workloads`` holds the seeded synthetic inputs.
"""
