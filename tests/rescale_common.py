"""Inputs that drive the bf16 forward kernels through their running-maximum
rescale, and a CPU replay of the order in which those kernels visit key tiles.

The forward kernels keep a running row maximum m (log2 units of the scaled
scores) and only raise it when a later 64-key tile's maximum exceeds it by more
than 8; the first visited tile sets m with a zero accumulator, so only a later
tile that scores far above the first one takes the branch with alpha != 0.
The stress inputs give every query a shared direction u and shift chosen keys
along u, so that their scores rise by a known amount:

  * "context": keys of context tile 2 (positions 128..191) shifted by 5 u and
    of tile 6 (positions 384..447) by 10 u; queries carry 24 u, so tile 2 scores
    ~120 raw (15 log2 units at scale 1/sqrt(128)) above tile 0, and tile 6 as
    much again above tile 2 (and above tile 4, where a 4-tile split starts);
  * "canvas": the keys of every canvas's own block shifted by 5 u, so each
    canvas row's last tile scores ~15 log2 units above its first context tile.
The shift sits mostly on the queries: a large offset shared by the keys a row
sees cancels in dQ = scale * sum_j dS_j k_j (sum_j dS_j = 0), so the bf16
rounding of dS would dominate dQ's relative error (2.6 % at a key offset of
60 u against 0.5 % here, in a CPU replay of that rounding).

``growth`` recomputes from the inputs, per query row and per launched work item,
how far a later tile's maximum lies above the item's first tile, so a test can
assert that the branch is reached instead of assuming it.
"""
from __future__ import annotations

import math

import numpy as np

from block_diffusion_attention_amd import workloads as W

KEY_TILE = 64          # keys per main-loop step of the forward kernels
RESCALE_SLACK = 8.0    # log2 units the running maximum may lag before it is raised
GROWTH = 12.0          # growth the stress inputs are required to reach (log2 units)

# one segment: a 512-token context (16 blocks of 32, 8 key tiles) in replay mode
# and four canvases; 8 query heads over 2 kv heads, head_dim 128
STRESS_META = dict(ctx_len=[512], ctx_q_begin=[0], canvas_block_idx=[[16, 12, 9, 3]], block_size=32,
                   num_q_heads=8, num_kv_heads=2, head_dim=128, dtype="bf16")


def stress_workload(kind: str, seed: int = 0) -> W.Workload:
    meta = W.Meta(**{k: (list(map(list, v)) if k == "canvas_block_idx" else v) for k, v in STRESS_META.items()})
    rng = np.random.default_rng(seed)
    # dO at a quarter scale: the high-scoring keys collect most of the weight of
    # ~500 rows x 4 heads, and with unit dO their dV reaches ~8, where the bf16
    # rounding of the output alone (spacing 1/16) exceeds the 2e-2 bar
    wl = W.random_workload(rng, meta, sigma=0.3, name=f"rescale-{kind}", do_sigma=0.25)
    D = meta.head_dim
    u = np.full(D, 1.0 / math.sqrt(D), np.float32)
    q = wl.q + np.float32(24.0) * u
    k = wl.k.copy()
    C, B = meta.ctx_len[0], meta.block_size
    if kind == "context":
        k[128:192] += np.float32(5.0) * u
        k[384:448] += np.float32(10.0) * u
    elif kind == "canvas":
        k[C:C + len(meta.canvas_block_idx[0]) * B] += np.float32(5.0) * u
    else:
        raise ValueError(kind)
    wl.q = W.round_bf16(q)
    wl.k = W.round_bf16(k)
    return wl


def _row_tiles(meta):
    """Per query token: (visible clean-key limit L, own canvas key range or None).
    One segment, block-causal rows, grid offset 0 (the stress meta)."""
    C, q0, B = meta.ctx_len[0], meta.ctx_q_begin[0], meta.block_size
    rows = []
    for t in range(q0, C):
        rows.append(((t // B + 1) * B, None))
    for c, b in enumerate(meta.canvas_block_idx[0]):
        own = (C + c * B, C + (c + 1) * B)
        for _ in range(B):
            rows.append((b * B, own))
    return rows


def growth(wl: W.Workload, tiles_per_split=None):
    """Largest rise of a later tile's maximum over the first tile's, per
    (query token, head) and work item, in log2 units, as the kernels see it.

    Returns (growth [Tq, Hq] max over the row's items, is_canvas [Tq]).
    The tile list of a row is its context tiles 0 .. ceil(L/64) - 1 followed by
    its own canvas tiles; with a split size, a work item covers tiles
    [j*tps, (j+1)*tps) of that list (every row of these stress tiles has the
    tile's largest limit, so the row's list is the tile's list).
    """
    m = wl.meta
    G = m.num_q_heads // m.num_kv_heads
    c = m.scale / math.log(2.0)             # scale * log2(e)
    q = wl.q.astype(np.float64)
    k = wl.k.astype(np.float64)
    rows = _row_tiles(m)
    out = np.full((len(rows), m.num_q_heads), -np.inf)
    is_canvas = np.array([own is not None for _, own in rows])
    for i, (L, own) in enumerate(rows):
        tiles = [np.arange(t0, min(t0 + KEY_TILE, L)) for t0 in range(0, L, KEY_TILE)]
        if own is not None:
            tiles += [np.arange(t0, min(t0 + KEY_TILE, own[1])) for t0 in range(own[0], own[1], KEY_TILE)]
        tps = tiles_per_split if (tiles_per_split and len(tiles) > tiles_per_split) else len(tiles)
        for h in range(m.num_q_heads):
            s = c * (k[:, h // G] @ q[i, h])
            tmax = np.array([s[t].max() for t in tiles])
            for j0 in range(0, len(tiles), tps):
                part = tmax[j0:j0 + tps]
                if len(part) > 1:
                    out[i, h] = max(out[i, h], float(part[1:].max() - part[0]))
    return out, is_canvas
