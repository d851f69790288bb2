"""MI355X-native batched Lloyd k-means: FlashAssign + sort-inverse update on gfx950.

The compute path is the HIP shared library ``libflashkm.so`` (C-ABI declared in
``include/flashkm.h``); ``exact_lloyd_means_02_amd.flashkm`` is the thin ctypes binding.
Importing this package does not load the library; the binding does, and it raises if
the library is missing.
"""
