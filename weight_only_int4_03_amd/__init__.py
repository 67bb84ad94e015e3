"""MI355X-native W4A16 weight-only INT4 GEMM (gfx950, wave64).

The compute path is the HIP library ``libw4a16.so`` built from ``csrc/``; the
Python module :mod:`weight_only_int4_03_amd.w4a16` is a thin ctypes binding
over its C ABI (``include/w4a16.h``).  Importing this package loads nothing;
the binding loads the library on first use and raises if it is missing.
"""
__all__ = ["w4a16", "synth"]
