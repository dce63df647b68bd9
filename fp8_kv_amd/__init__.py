"""MI355X-native paged grouped-query attention with FP16 / FP8-E4M3 KV.

The compute lives in the C-ABI library ``libpgqa.so`` (hand-written HIP for
gfx950, declared in ``include/pgqa.h``); ``fp8_kv_amd.pgqa`` is its thin
ctypes binding.  Importing this package loads nothing: the binding loads the
library on first use and raises if it is missing.
"""
__all__ = ["pgqa", "inputs"]
