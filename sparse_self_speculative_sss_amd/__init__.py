"""Sparse self-speculative decode attention for AMD MI355X (gfx950).

The compute lives in the HIP library ``libsss.so`` (built from ``csrc/``)
behind a C ABI (``include/sss.h``); :mod:`.sss` is the thin ctypes binding.
The binding is imported lazily so that the input generator in
:mod:`.workload` can be used on machines without a GPU.
"""
import importlib

__all__ = ["sss", "workload"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f".{name}", __name__)
    raise AttributeError(name)
