"""Sparse KV-cache decode step for MI355X (gfx950).

score -> top-k -> delta/LRU working set (+ miss fetch) -> split-K GQA
attention, as hand-written HIP kernels behind the C ABI declared in
``include/sparse_kv.h`` (``libsparse_kv.so``).  ``binding`` is the Python
binding of that ABI, ``step`` a per-layer buffer helper, ``synth`` the
seeded synthetic workloads.  Submodules load on first use so that the input
generator does not pull in torch or the GPU library.
"""

import importlib

__all__ = ["binding", "step", "synth", "build"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
