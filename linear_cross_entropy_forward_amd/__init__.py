"""flash-CCE ORPO head for MI355X (gfx950).

The compute path is the HIP library ``libflashcce.so`` (C-ABI, declared in
``include/flashcce.h``); :mod:`linear_cross_entropy_forward_amd.binding` is a
thin ctypes layer over it.  Importing this package loads nothing; the first
call through the binding loads the library and raises if it is missing.
"""
__all__ = ["binding", "workloads"]
