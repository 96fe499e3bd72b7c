"""KIVI-style quantized KV-cache append and decode attention for MI355X (gfx950).

The compute path is libkvq.so (hand-written HIP kernels behind the C ABI in
include/kvq.h). This package holds its ctypes binding (`binding`), a torch-facing
cache wrapper (`cache.QuantizedKVCache`), the build script (`build`) and the
seeded synthetic workloads (`workloads`). Importing the package does not load
the library; the first call into it does, and fails loudly if it is not built.
"""

__all__ = ["binding", "cache", "workloads", "build"]


def __getattr__(name):
    if name == "QuantizedKVCache":
        from .cache import QuantizedKVCache
        return QuantizedKVCache
    raise AttributeError(name)
