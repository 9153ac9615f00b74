"""MI355X-native split-KV MLA decode over a paged FP8 E4M3 cache.

The compute path is a C-ABI shared library (``libmla_decode.so``, HIP kernels for
gfx950) declared in ``include/mla_decode.h``; ``decode_attention_gather_amd.mla`` is
its thin ctypes binding. Importing this package loads nothing; the binding raises if
the built library is missing.
"""
__all__ = ["mla", "inputs"]
