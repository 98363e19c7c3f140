"""MoE expert offload with a fixed-size HBM expert-slot cache, for MI355X (gfx950).

The compute path lives in the HIP/C++ shared library ``libmoe_pool.so`` (C ABI,
``include/moe_pool.h``); ``expert_slot_cache_amd.binding`` is a thin ctypes layer
over it.  ``expert_slot_cache_amd.synth`` holds the seeded synthetic inputs.
Importing the package loads nothing; the library is loaded on first use of the
binding and its absence is an error, never a fallback.
"""

__all__ = ["binding", "synth"]
