"""MI355X-native FP8 MoE expert grouped GEMM.

The compute runs in the HIP library ``libmxsg.so`` (built from ``csrc/``
for gfx950); this package is its thin Python binding (``api``). Importing
the package loads nothing; the first call into ``api`` loads the library
and raises if it is missing or no GPU is present.
"""
import importlib

__all__ = ["api", "workloads"]


def __getattr__(name):
    if name in ("api", "workloads", "_lib"):
        return importlib.import_module("." + name, __name__)
    raise AttributeError(name)
