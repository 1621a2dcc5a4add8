"""MI355X-native paged KV cache: decode attention over a pool of 16-token
blocks, the paged cache write and the copy-on-write block copy.

The compute runs in hand-written HIP kernels for gfx950 behind a C ABI
(``include/pa.h``, built into ``paged_kv_cache_401_amd/libpa.so``).  The
Python layer (``ops``) only marshals torch tensors to that ABI; it raises if
the library is missing.  ``blocks`` is the host block manager and
``workloads`` draws seeded synthetic inputs.
"""
__all__ = ["ops", "blocks", "workloads"]
