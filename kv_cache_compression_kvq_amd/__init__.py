"""kvq: low-bit KV-cache compression and decode attention for MI355X (gfx950).

The compute path is the HIP library ``libkvq.so`` built from ``csrc/``; the
Python binding in ``abi`` only marshals pointers, sizes and streams. Importing
this package does not load the library; ``kv_cache_compression_kvq_amd.abi``
does, and fails loudly if it has not been built.
"""
__all__ = ["abi", "bytes_model", "synth"]
