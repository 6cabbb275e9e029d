"""Exact tiled attention (BF16) for MI355X / gfx950.

The compute path is the C-ABI library libfa_gfx950.so (include/fa_gfx950.h),
built from csrc/ by build_lib.py; ``attention`` is a thin torch binding of it.
Imports are lazy so that the input generators can be used without torch or the
library.
"""
__all__ = ["attention", "inputs", "workload", "build_lib"]


def __getattr__(name):
    import importlib
    if name in __all__:
        return importlib.import_module(f".{name}", __name__)
    raise AttributeError(name)
