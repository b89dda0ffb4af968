"""Batched-decode PagedAttention for AMD MI355X (gfx950).

The compute path is a C-ABI HIP library (``libpagedkv.so``, declared in
``include/pagedkv.h``); ``_lib`` is its thin ctypes binding.  ``synth``
draws seeded synthetic decode batches and ``pool`` is host-side block
bookkeeping.  Importing the package does not load the library; the first
call into ``_lib`` does, and fails loudly if it has not been built.
"""

__all__ = ["synth", "pool", "roofline"]
