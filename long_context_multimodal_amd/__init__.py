"""MI355X-native per-rank MM-SP chunked causal attention.

The compute lives in ``libmmsp.so`` (hand-written HIP kernels for gfx950 behind
the C-ABI declared in ``include/mmsp.h``).  :mod:`.mmsp` is a thin ctypes
binding with the same names; :mod:`.workloads` draws the seeded synthetic
inputs.  Importing the package does not load the library: the binding loads it
on first use and raises if it is missing.
"""

__all__ = ["mmsp", "workloads"]
