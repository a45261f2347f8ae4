"""SAF hybrid attention layer for AMD MI355X (gfx950).

The compute lives in the HIP library ``libsaf_hybrid.so`` (C ABI in
``include/saf_hybrid.h``); this package holds its sources (``csrc/``), the
build script and a thin ctypes binding.  Importing the binding requires the
built library -- there is no CPU fallback.
"""

import importlib

__all__ = ["autograd", "binding", "build"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
