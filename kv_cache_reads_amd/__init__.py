"""Top-K+phi residual-mass-accounting decode for AMD MI355X (gfx950).

The compute lives in librma.so (hand-written HIP kernels behind a C ABI, see
include/rma.h); `kv_cache_reads_amd.rma` is the thin ctypes binding over it.
Submodules load lazily so that the input generator can be used without the
library.
"""
__all__ = ["rma", "workload"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
