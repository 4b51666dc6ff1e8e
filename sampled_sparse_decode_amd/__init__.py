"""libsanta: SANTA++ sampled-team decode attention for AMD MI355X (gfx950).

The compute lives in a C-ABI shared library (``libsanta.so``, hand-written HIP
kernels); ``sampled_sparse_decode_amd.santa`` is a thin ctypes binding that
marshals torch tensors and the current HIP stream into it. Importing this
package loads nothing; the library is loaded on first use of the binding and
a missing or unloadable library raises an error (there is no fallback path).
"""
import importlib

__all__ = ["santa", "workloads"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
