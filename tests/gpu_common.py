"""Helpers for GPU parity tests: run a workload through the C ABI, and the oracle beside it."""
from __future__ import annotations

import numpy as np
import torch

from oracle import bd_oracle as orc


def to_dev(x, dtype):
    if x is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").to(dtype).contiguous()


def nan_like(shape, dtype):
    """An output buffer filled with NaN, so that any element a kernel fails to
    write shows up in the comparison instead of keeping a stale value."""
    return torch.full(shape, float("nan"), dtype=dtype, device="cuda")


def run_gpu(wl, flags=0, backward=True):
    """Forward (and backward) of a workload through libbdattn; numpy float64 results.
    Every output starts out NaN-filled."""
    from block_diffusion_attention_amd import binding as b
    plan = b.Plan(wl.meta, flags).upload("cuda")
    dt = plan.dtype
    q, k, v = to_dev(wl.q, dt), to_dev(wl.k, dt), to_dev(wl.v, dt)
    o = nan_like(q.shape, dt)
    lse = nan_like((plan.tq, wl.meta.num_q_heads), torch.float32)
    o, lse = b.fwd(plan, q, k, v, o, lse)
    out = {"o": o, "lse": lse}
    if backward and wl.do is not None:
        do = to_dev(wl.do, dt)
        dq, dk, dv = nan_like(q.shape, dt), nan_like(k.shape, dt), nan_like(v.shape, dt)
        dq, dk, dv = b.bwd(plan, q, k, v, o, lse, do, dq, dk, dv)
        out.update(dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return {n: t.float().cpu().numpy().astype(np.float64) for n, t in out.items()}, plan


def run_oracle(wl, backward=True, segments=None):
    o, lse = orc.attention_fwd(wl.q, wl.k, wl.v, wl.meta, scale=wl.meta.softmax_scale, segments=segments)
    out = {"o": o, "lse": lse}
    if backward and wl.do is not None:
        dq, dk, dv = orc.attention_bwd(wl.q, wl.k, wl.v, wl.do, wl.meta, scale=wl.meta.softmax_scale,
                                       segments=segments)
        out.update(dq=dq, dk=dk, dv=dv)
    return out
