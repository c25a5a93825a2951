"""SAGA + Atop-N sparse decode attention for MI355X (gfx950).

The compute lives in a C-ABI shared library of hand-written HIP kernels
(``csrc/``, declared in ``include/saga.h``).  ``saga`` is a thin ctypes binding
over it; ``workload`` draws seeded synthetic inputs.  Nothing is loaded at
import time: the binding opens the library on first use and raises if it is
missing -- there is no CPU fallback.
"""

__all__ = ["saga", "workload"]
