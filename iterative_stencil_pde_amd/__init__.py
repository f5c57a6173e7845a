"""Persistent-kernel Jacobi engine for AMD MI355X (gfx950).

The engine is the C-ABI library ``_libpk.so`` built from ``csrc/`` (declared in
``include/pk.h`` at the repository root). ``pk`` is its thin ctypes binding,
``inputs`` builds the seeded synthetic workloads. Importing this package loads
nothing native; the binding loads the library on first use and raises if it is
missing (there is no CPU fallback).
"""

__all__ = ["pk", "inputs"]
