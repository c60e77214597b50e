"""MI355X-native W4A16 Mixture-of-Experts expert layer.

The compute path is hand-written HIP for gfx950 in ``csrc/``, built into the
C-ABI library ``libmoe_w4a16.so``; ``ops`` binds it with ctypes (argument
marshalling only). PyTorch provides device memory and streams.

Importing the package does not load the native library; the first call into
``ops`` does, and raises if the library is missing.
"""
import importlib

__all__ = ["ops", "inputs"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
