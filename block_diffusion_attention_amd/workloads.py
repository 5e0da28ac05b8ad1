"""Seeded synthetic workloads for staircase block-diffusion attention.

This module only draws metadata and input tensors; it holds none of the
attention arithmetic, so the GPU path and the CPU oracle can both consume its
output without sharing any of the method's code.

Packed layout of one segment (the boundary's contract):
  keys    : [ C clean context tokens | m canvases of B tokens ]
  queries : [ clean tokens from position q0 to C | the same m canvases ]
Replay rows (q0 = 0) make the context tokens queries too; the single-request
denoising step (q0 = C) queries only with the canvas, and the commit-folded
step (q0 = C - B) with the just-finished block and the next canvas.

The five named workloads follow the shapes the method is used at: packed
replay rows of captured canvases after their clean contexts, and one
denoising step over a long context (ORL section 3.2, appendix D.2/D.3, and
appendix F.1 "Kernels" for the single-request shape). Draw order for
``make_config``: metadata, then Q, K, V (standard normal float32 times sigma),
then dO (standard normal); bf16 workloads are rounded to bf16 with
round-to-nearest-even and kept as float32 arrays holding exact bf16 values.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

DTYPE_BF16 = "bf16"
DTYPE_FP32 = "fp32"


@dataclasses.dataclass
class Meta:
    """Per-segment metadata of one packed batch."""
    ctx_len: List[int]                 # C_s; C_s + o_s a multiple of block_size
    ctx_q_begin: List[int]             # q0_s in [0, C_s]
    canvas_block_idx: List[List[int]]  # per segment, block index b in [0, (C_s+o_s)/B], any order
    block_size: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str = DTYPE_BF16
    softmax_scale: float = 0.0         # <= 0 means 1/sqrt(head_dim)
    # o_s in [0, B): the segment's block grid starts o_s positions before its
    # first context token (a prompt whose length is not a multiple of B followed
    # by whole blocks); None means 0 for every segment
    block_offset: Optional[List[int]] = None
    clean_causal: bool = False         # clean queries see clean keys token-causally

    def offset(self, s: int) -> int:
        return 0 if self.block_offset is None else int(self.block_offset[s])

    @property
    def num_segments(self) -> int:
        return len(self.ctx_len)

    @property
    def canvas_offsets(self) -> List[int]:
        off = [0]
        for c in self.canvas_block_idx:
            off.append(off[-1] + len(c))
        return off

    @property
    def flat_canvas_block_idx(self) -> List[int]:
        return [int(b) for c in self.canvas_block_idx for b in c]

    def seg_q_tokens(self, s: int) -> int:
        return (self.ctx_len[s] - self.ctx_q_begin[s]) + len(self.canvas_block_idx[s]) * self.block_size

    def seg_k_tokens(self, s: int) -> int:
        return self.ctx_len[s] + len(self.canvas_block_idx[s]) * self.block_size

    @property
    def tq(self) -> int:
        return sum(self.seg_q_tokens(s) for s in range(self.num_segments))

    @property
    def tk(self) -> int:
        return sum(self.seg_k_tokens(s) for s in range(self.num_segments))

    def q_offsets(self) -> List[int]:
        off = [0]
        for s in range(self.num_segments):
            off.append(off[-1] + self.seg_q_tokens(s))
        return off

    def k_offsets(self) -> List[int]:
        off = [0]
        for s in range(self.num_segments):
            off.append(off[-1] + self.seg_k_tokens(s))
        return off

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale > 0 else 1.0 / math.sqrt(self.head_dim)


@dataclasses.dataclass
class Workload:
    name: str
    meta: Meta
    q: np.ndarray          # [Tq, Hq, D] float32 (exact bf16 values for bf16 workloads)
    k: np.ndarray          # [Tk, Hkv, D]
    v: np.ndarray          # [Tk, Hkv, D]
    do: Optional[np.ndarray]  # [Tq, Hq, D] or None
    passes: str            # "fwd" or "fwd+bwd"


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def _normal(rng, shape, sigma, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x = x * np.float32(sigma)
    return round_bf16(x) if dtype == DTYPE_BF16 else x


def draw_tensors(meta: Meta, rng, sigma: float, with_do: bool, do_sigma: float = 1.0):
    """Q, K, V (and dO) for ``meta`` from ``rng`` in the fixed draw order."""
    hq, hkv, d = meta.num_q_heads, meta.num_kv_heads, meta.head_dim
    q = _normal(rng, (meta.tq, hq, d), sigma, meta.dtype)
    k = _normal(rng, (meta.tk, hkv, d), sigma, meta.dtype)
    v = _normal(rng, (meta.tk, hkv, d), sigma, meta.dtype)
    do = _normal(rng, (meta.tq, hq, d), do_sigma, meta.dtype) if with_do else None
    return q, k, v, do


CONFIG_NAMES = {
    1: "tiny-fp32-fwd",
    2: "denoise-step-2048ctx-32q8kv-d128",
    3: "packed-replay-16seg-32q8kv-d128",
    4: "staircase-4096ctx-24canvas-32q8kv-d128",
    5: "large-pack-4x8192ctx-16canvas-32q8kv-d128",
    6: "commit-folded-step-2031ctx-offset17-32q8kv-d128",
}


def config_meta(k: int, rng) -> Meta:
    """Metadata of named workload ``k`` (1..6), drawn from ``rng``."""
    if k == 1:
        return Meta([64], [0], [[4]], 16, 2, 1, 64, DTYPE_FP32)
    if k == 2:
        return Meta([2048], [2048], [[64]], 32, 32, 8, 128, DTYPE_BF16)
    if k == 3:
        n = rng.integers(8, 129, size=16)
        return Meta([int(32 * x) for x in n], [0] * 16, [[int(x)] for x in n], 32, 32, 8, 128, DTYPE_BF16)
    if k == 4:
        b = rng.choice(np.arange(1, 129), size=24, replace=False)
        return Meta([4096], [0], [[int(x) for x in b]], 32, 32, 8, 128, DTYPE_BF16)
    if k == 5:
        cv = [[int(x) for x in rng.choice(np.arange(1, 257), size=16, replace=False)] for _ in range(4)]
        return Meta([8192] * 4, [0] * 4, cv, 32, 32, 8, 128, DTYPE_BF16)
    if k == 6:
        # commit-folded step of one request: a 2031-token context (a prompt that
        # leaves the block grid 17 positions short, then whole blocks of 32), the
        # block just finished (its 32 tokens as token-causal queries) and the next
        # canvas, in one pass over the KV arena
        return Meta([2031], [1999], [[64]], 32, 32, 8, 128, DTYPE_BF16, block_offset=[17], clean_causal=True)
    raise ValueError(f"unknown workload {k}")


def make_config(k: int, seed: Optional[int] = None, with_do: Optional[bool] = None) -> Workload:
    """Named workload ``k`` (1..6) with seed (default k)."""
    rng = np.random.default_rng(k if seed is None else seed)
    meta = config_meta(k, rng)
    sigma = 1.0 if k == 1 else 1.0 / math.sqrt(128.0)
    passes = "fwd+bwd" if k in (3, 4, 5) else "fwd"
    if with_do is None:
        with_do = k in (1, 3, 4, 5)
    q, kk, v, do = draw_tensors(meta, rng, sigma, with_do)
    return Workload(CONFIG_NAMES[k], meta, q, kk, v, do, passes)


def random_meta(rng, *, max_segments=3, max_blocks=5, block_sizes=(1, 2, 3, 4), max_canvases=3,
                hq=2, hkv=1, d=8, dtype=DTYPE_FP32, canvas_only_prob=0.3, allow_empty_ctx=True,
                offsets=False, clean_causal=False) -> Meta:
    """Small random metadata for exhaustive and randomized checks.

    ``offsets`` draws a block-grid offset o in [0, B) per segment (the context
    then holds n*B - o tokens); ``clean_causal`` sets the token-causal clean rule.
    """
    B = int(rng.choice(block_sizes))
    S = int(rng.integers(1, max_segments + 1))
    ctx, q0s, cvs, offs = [], [], [], []
    for _ in range(S):
        n = int(rng.integers(0 if allow_empty_ctx else 1, max_blocks + 1))
        o = int(rng.integers(0, B)) if (offsets and n > 0) else 0
        offs.append(o)
        C = n * B - o
        m = int(rng.integers(0, max_canvases + 1))
        cv = [int(x) for x in rng.integers(0, n + 1, size=m)]
        if rng.random() < canvas_only_prob:
            q0 = C
        else:
            q0 = int(rng.integers(0, C + 1)) if rng.random() < 0.3 else 0
        if (C - q0) + m * B == 0:       # keep at least one query per segment
            cv = [n]
        ctx.append(C); q0s.append(q0); cvs.append(cv)
    return Meta(ctx, q0s, cvs, B, hq, hkv, d, dtype, block_offset=offs if offsets else None,
                clean_causal=clean_causal)


def random_workload(rng, meta: Meta, sigma: float = 1.0, with_do: bool = True, name="random",
                    do_sigma: float = 1.0) -> Workload:
    q, k, v, do = draw_tensors(meta, rng, sigma, with_do, do_sigma)
    return Workload(name, meta, q, k, v, do, "fwd+bwd" if with_do else "fwd")


def segment_slice(wl: Workload, s: int) -> Workload:
    """The one-segment workload made of segment ``s`` of ``wl`` (same tensors, sliced)."""
    m = wl.meta
    qo, ko = m.q_offsets(), m.k_offsets()
    sub = Meta([m.ctx_len[s]], [m.ctx_q_begin[s]], [list(m.canvas_block_idx[s])], m.block_size,
               m.num_q_heads, m.num_kv_heads, m.head_dim, m.dtype, m.softmax_scale,
               None if m.block_offset is None else [m.offset(s)], m.clean_causal)
    q = wl.q[qo[s]:qo[s + 1]]
    k = wl.k[ko[s]:ko[s + 1]]
    v = wl.v[ko[s]:ko[s + 1]]
    do = None if wl.do is None else wl.do[qo[s]:qo[s + 1]]
    return Workload(f"{wl.name}[seg{s}]", sub, q, k, v, do, wl.passes)


def kv_group_slice(wl: Workload, g: int) -> Workload:
    """The workload restricted to kv head ``g`` and its query heads."""
    m = wl.meta
    G = m.num_q_heads // m.num_kv_heads
    sub = dataclasses.replace(m, num_q_heads=G, num_kv_heads=1,
                              canvas_block_idx=[list(c) for c in m.canvas_block_idx],
                              block_offset=None if m.block_offset is None else list(m.block_offset))
    hs = slice(g * G, (g + 1) * G)
    return Workload(f"{wl.name}[kv{g}]", sub, wl.q[:, hs], wl.k[:, g:g + 1], wl.v[:, g:g + 1],
                    None if wl.do is None else wl.do[:, hs], wl.passes)


# ---------------------------------------------------------------- vocabulary logits

AEC_VOCAB = 151936          # a 152k-entry vocabulary (the pages give no size)


@dataclasses.dataclass
class AecWorkload:
    """Logits of the canvas positions of a replay batch, their unresolved
    masks, and adjacent state pairs with captured source entropies."""
    name: str
    logits: np.ndarray         # [N, row_stride] float32 (exact bf16 values for bf16)
    vocab: int
    unresolved: np.ndarray     # [N] uint8
    state_rows: np.ndarray     # [S+1] int32
    pair_next: np.ndarray      # [P] int32
    pair_h_source: np.ndarray  # [P] float32
    pair_weight: np.ndarray    # [P] float32
    rho: float
    gate_max: float
    dtype: str


def aec_workload(seed: int, n_states: int = 16, block: int = 32, vocab: int = AEC_VOCAB,
                 row_stride: Optional[int] = None, dtype: str = DTYPE_BF16, rho: float = 0.1,
                 gate_max: float = math.inf, states_per_response: int = 4) -> AecWorkload:
    """Seeded synthetic logits for ``n_states`` states of ``block`` positions.

    Draw order: per-row temperature tau ~ U[0.5, 6]; logits N(0, 1) * tau; for
    about one row in ten, one entry raised by U[10, 30]; unresolved flags
    (probability 0.6; the fourth state fully resolved); captured source means
    U[0.05, 1] for the pairs (s, s+1) inside each response of
    ``states_per_response`` consecutive states, weighted 1 / (pairs of the
    response). Columns past the vocabulary hold 30000, which a kernel that read
    them would notice.
    """
    rng = np.random.default_rng(seed)
    N = n_states * block
    width = 8 if dtype == DTYPE_BF16 else 4
    stride = row_stride or -(-vocab // width) * width
    tau = rng.uniform(0.5, 6.0, size=N).astype(np.float32)
    z = rng.standard_normal((N, vocab), dtype=np.float32)
    z *= tau[:, None]
    peaky = np.nonzero(rng.random(N) < 0.1)[0]
    for i in peaky:
        z[i, int(rng.integers(vocab))] += np.float32(rng.uniform(10.0, 30.0))
    logits = np.full((N, stride), 30000.0, dtype=np.float32)
    logits[:, :vocab] = z
    if dtype == DTYPE_BF16:
        logits = round_bf16(logits)
    unresolved = (rng.random(N) < 0.6).astype(np.uint8)
    if n_states > 3:
        unresolved[3 * block:4 * block] = 0
    state_rows = (np.arange(n_states + 1) * block).astype(np.int32)
    nxt, hs, w = [], [], []
    for r0 in range(0, n_states, states_per_response):
        members = list(range(r0, min(n_states, r0 + states_per_response)))
        pairs = list(zip(members, members[1:]))
        for _src, dst in pairs:
            nxt.append(dst)
            hs.append(rng.uniform(0.05, 1.0))
            w.append(1.0 / len(pairs))
    return AecWorkload(f"aec-{n_states}x{block}-V{vocab}-{dtype}", logits, vocab, unresolved, state_rows,
                       np.array(nxt, np.int32), np.array(hs, np.float32), np.array(w, np.float32),
                       float(rho), float(gate_max), dtype)
