"""The rescale stress inputs reach the forward kernels' running-maximum rescale.

Checked on the CPU from the inputs alone, by replaying the kernels' key-tile
order: for most target rows a later tile of the same work item scores at least
12 log2 units above the item's first tile (the kernels rescale beyond 8).
The GPU parity test of these inputs runs the same check first.
"""
import numpy as np
import pytest

from rescale_common import GROWTH, RESCALE_SLACK, growth, stress_workload

SPLIT_TILES = 4


def reached(kind, tps):
    wl = stress_workload(kind)
    g, is_canvas = growth(wl, tps)
    C = wl.meta.ctx_len[0]
    if kind == "context":
        # clean rows that see tile 2 (L > 128) and canvases with b >= 5
        target = np.zeros(len(is_canvas), bool)
        target[:C] = np.arange(C) >= 128
        target[C:] = np.repeat(np.array(wl.meta.canvas_block_idx[0]) * 32 > 128, 32)
    else:
        target = is_canvas.copy()
    frac = float((g[target] >= GROWTH).mean())
    return frac, g, target


@pytest.mark.parametrize("kind", ["context", "canvas"])
@pytest.mark.parametrize("tps", [None, SPLIT_TILES])
def test_stress_inputs_reach_the_rescale(kind, tps):
    frac, g, target = reached(kind, tps)
    assert frac >= 0.6, f"{kind} tps={tps}: only {frac:.2f} of the target rows grow by {GROWTH}"


def test_plain_inputs_do_not_reach_it():
    # the same shapes without the shifts stay well inside the slack: the stress is
    # what makes the branch run
    from block_diffusion_attention_amd import workloads as W
    from rescale_common import STRESS_META
    meta = W.Meta(**STRESS_META)
    wl = W.random_workload(np.random.default_rng(0), meta, sigma=0.3)
    g, _ = growth(wl)
    assert np.nanmax(g[np.isfinite(g)]) < RESCALE_SLACK
