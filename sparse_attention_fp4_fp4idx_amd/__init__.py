"""MI355X-native FP4 lightning-indexer hot path.

The compute lives in ``libfp4idx.so`` (hand-written HIP for gfx950, C ABI
declared in ``include/fp4idx.h``).  ``fp4idx`` is the thin Python binding
(argument marshalling only); ``workloads`` draws seeded synthetic inputs.
Submodules are imported on first use so that ``workloads`` works without a
GPU.
"""
import importlib

__all__ = ["fp4idx", "workloads"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
