"""MI355X-native paged KV-cache decode: the slot write and PagedAttention decode.

The compute path is the C-ABI library ``libpa.so`` (hand-written HIP kernels
for gfx950); ``paged_kv_cache_261_amd.pa`` is its thin ctypes binding and
``paged_kv_cache_261_amd.synthetic`` builds seeded decode workloads.
"""
