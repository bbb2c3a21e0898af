"""MI355X (gfx950) gated sparse attention hot path: indexer -> Top-K -> gated sparse attention.

The compute runs in hand-written HIP kernels behind the C ABI declared in
``include/sparse_attn.h``; ``binding`` marshals torch tensors into those calls.
Importing the package does not load the shared library; the first call does,
and fails loudly if it has not been built.
"""
import importlib

__all__ = ["binding", "workloads"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
