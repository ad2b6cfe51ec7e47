"""LoSA per-denoising-step attention on MI355X (gfx950).

The compute path is the C-ABI library ``liblosa.so`` (hand-written HIP kernels,
declared in ``include/losa.h``).  ``sparse_attention_block_amd.binding`` is the
thin Python binding with the same entry-point names; ``workloads`` holds the
seeded synthetic inputs.  Submodules load on first use, so the input
generators work on machines without the built library.
"""
import importlib

__all__ = ["binding", "workloads"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
