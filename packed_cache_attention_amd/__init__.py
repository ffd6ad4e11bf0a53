"""MI355X-native Block-GTQ key-cache quantization and packed-cache decode attention.

The compute path is the HIP library ``libkvq.so`` (C ABI declared in
``include/kvq.h``); ``packed_cache_attention_amd.kvq`` is its thin ctypes
binding.  Importing this package loads nothing: ``kvq`` loads the library on
first use and fails loudly when it has not been built.
"""
__all__ = ["kvq", "synth"]
