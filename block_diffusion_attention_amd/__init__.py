"""MI355X-native staircase block-diffusion attention.

The compute path is the C-ABI library ``libbdattn.so`` (hand-written HIP
kernels for gfx950); ``binding`` marshals torch tensors into it. The binding
is imported lazily so that host-only users (workload generation, planning
tests) do not need a GPU.
"""
__all__ = ["binding", "workloads"]


def __getattr__(name):
    if name == "binding":
        from . import binding as _b
        return _b
    if name == "workloads":
        from . import workloads as _w
        return _w
    raise AttributeError(name)
