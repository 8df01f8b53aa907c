"""MI355X-native CSA2 global-branch hot path (FP4 KV cache).

The compute lives in ``libcsa2.so`` (hand-written HIP kernels for gfx950 behind a C ABI
declared in ``include/csa2.h``).  ``fp4_kv_cache_csa2_amd.csa2`` is the thin Python
binding over it; importing this package does not load the library.
"""
__all__ = ["csa2", "synth"]
