"""MI355X-native LongCat Sparse Attention (LSA) hot path.

The compute lives in ``liblsa.so`` (hand-written HIP kernels for gfx950 behind a C ABI declared
in ``include/lsa.h``).  ``long_context_sparse_lightning_amd.lsa`` is the thin ctypes binding;
submodules are imported on first use so that host-only tooling (the input generator) works
without a GPU.
"""
import importlib

__all__ = ["lsa", "inputs"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
