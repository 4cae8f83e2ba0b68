"""MI355X (gfx950) prefill forward pass of a decoder-only transformer.

The computation lives in libfwd.so (HIP kernels behind the C ABI of
include/fwd.h); ``fwd`` is its ctypes binding. Importing the package loads nothing.
"""
from . import fwd  # noqa: F401

__all__ = ["fwd"]
