"""MI355X (gfx950) DoRA hot path: factored row norm, fused compose, backward.

The computation lives in libdora.so (HIP kernels behind the C ABI declared in
include/dora.h).  ``ops`` is the torch binding with the same names,
``module.DoRALinear`` the autograd layer; both import torch lazily.
"""
from ._lib import LIB_PATH, DoraError, lib  # noqa: F401

__all__ = ["LIB_PATH", "DoraError", "lib"]
