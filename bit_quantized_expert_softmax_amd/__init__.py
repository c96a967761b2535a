"""libmoedecode for AMD MI355X: decode-time int4 MoE layer with an LFU expert cache.

The library itself is ``libmoedecode.so`` (C ABI in ``include/moedecode.h``,
HIP kernels in ``csrc/``); ``api`` is its ctypes binding with the same names.
Importing this package does not load the library; the first call does, and
fails loudly when it has not been built.
"""
from . import api  # noqa: F401
from .api import MoeError  # noqa: F401
