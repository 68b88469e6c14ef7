"""MI355X-native Float8Linear with tensorwise scaling.

The compute path is the C-ABI library libf8lin.so (hand-written HIP for
gfx950, built from csrc/); `f8lin` is its thin ctypes binding and loads it on
first attribute access, failing loudly if it is not built.  `inputs` holds the
seeded synthetic workloads.
"""
import importlib

__all__ = ["f8lin", "inputs", "module"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
