"""MI355X-native ball-tree partition, ball attention and Ball Sparse Attention.

The compute path is the HIP library ``libbtsparse.so`` built from ``csrc/``
for gfx950; ``ops`` is a thin ctypes binding over its C ABI (``include/bt.h``).
The library is loaded on first call of a binding, so importing the package (or
its ``synth`` input generators) never needs a GPU.
"""
import importlib

__all__ = ["ops", "synth"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
