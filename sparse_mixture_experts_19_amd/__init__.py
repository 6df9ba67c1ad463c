"""MI355X-native (gfx950) sparse top-k MoE FFN forward.

The compute lives in ``libmoe_mi355x.so`` (hand-written HIP kernels behind a
C ABI, declared in ``include/moe_mi355x.h``).  ``binding`` wraps that ABI for
torch tensors; it is imported lazily so that the input generator in
``workloads`` can be used without the library.
"""
import importlib

__all__ = ["workloads", "binding"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
