"""HSMLA attention forward pass for AMD Instinct MI355X (gfx950).

The compute lives in libhsmla.so (hand-written HIP kernels behind the C ABI
of include/hsmla.h); ``hsmla`` is its ctypes binding and ``device`` moves
host arrays into device tensors for it.
"""

from . import hsmla  # noqa: F401
