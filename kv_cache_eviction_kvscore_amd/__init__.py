"""MI355X-native (gfx950) output-perturbation KV-cache eviction scoring.

The compute path is the C-ABI library ``libkvscore.so`` (hand-written HIP kernels);
``kv_cache_eviction_kvscore_amd.api`` is a thin ctypes binding over it that passes
torch-owned device pointers and torch's current HIP stream. Importing this package
does not load the library; the binding loads it on first use and raises if it is
missing.
"""
__all__ = ["configs", "synth"]
