"""MI355X-native staircase block-diffusion attention.

The compute path is the C-ABI library ``libbdattn.so`` (hand-written HIP
kernels for gfx950); ``binding`` marshals torch tensors into it. The binding
is imported lazily so that host-only users (workload generation, planning
tests) do not need a GPU.
"""
import importlib

__all__ = ["binding", "workloads"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
