"""KVSculpt cache-distillation optimizer for MI355X (gfx950).

The compute lives in libkvsculpt.so (hand-written HIP kernels behind a C
ABI, declared in include/kvsculpt.h); this package is the thin ctypes
binding with the same entry-point names (``_lib``).  Importing it does not
touch the GPU; calling an entry point needs the built library and a GPU.
"""
from ._lib import *  # noqa: F401,F403
from ._lib import __all__  # noqa: F401
