"""Plain fp64 CPU oracle for staircase block-diffusion attention.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The GPU
library never calls it, and it imports nothing from the GPU library.

What is computed (ORL paper, section 3.2 "Staircase attention kernel" and the
appendix D.2 paragraph on the kernel): masked softmax attention over packed,
mutually invisible documents under block-diffusion visibility, and its analytic
gradients. Every value is computed in float64 from the inputs as given.

Packed layout of one segment (document), the interface both sides agree on:
  keys    : [ C clean context tokens | m canvases of B tokens each ]
  queries : [ clean tokens from position q0 to C | the same m canvases ]
A replay row (ORL section 3.1, section 3.2 "Packed and cost-balanced state
training") puts each captured canvas after its clean context; q0 = 0 makes every
context token a query as well (replay), q0 = C leaves only the canvases as
queries (the single-request denoising step, appendix F.1 "Kernels").

Readings of points the pages leave open (each one is a single place below):
  * clean queries see clean keys block-causally: key block <= query block,
    bidirectional inside a block (the pages only say clean queries never see
    noisy keys); with ``meta.clean_causal`` they see clean keys token-causally
    (key position <= query position), the reading of the causal commit pass
    that writes a finished block's keys and values (ORL appendix F.1, the
    single-request engine's block loop);
  * a canvas with block index b sees the clean blocks 0..b-1 and its own B
    tokens; b ranges over 0..(C+o)/B;
  * the block grid of a segment may start o positions (0 <= o < B) before its
    first context token, so that a prompt whose length is not a multiple of B is
    followed by whole blocks: context position p lies in block (p + o) // B, the
    first block holds B - o tokens and C + o is a multiple of B (o = 0 unless
    ``meta.block_offset`` says otherwise);
  * the commit-folded step (ORL section 3.3 "Commit folding": one pass over the
    finished block and the next canvas) is q0 = C - B with one canvas b = (C+o)/B;
  * query head h reads kv head h // (Hq / Hkv);
  * scale defaults to 1/sqrt(D); LSE is the natural-log log-sum-exp of the
    scaled scores.

Functions with parity pins (see tests/test_oracle_*.py): ``visible`` and
``dense_mask`` (hand-worked golden mask, library SDPA special cases),
``attention_fwd_dense``/``attention_bwd_dense`` (library SDPA with an explicit
mask, closed forms, finite differences), ``attention_fwd``/``attention_bwd``
(range form, checked element-wise against the dense form), ``visible_pairs``
(count of the dense mask).
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "segment_layout", "query_roles", "key_roles", "visible", "dense_mask",
    "visible_pairs", "attention_fwd_dense", "attention_bwd_dense",
    "attention_fwd", "attention_bwd",
]


# --------------------------------------------------------------------------
# metadata -> packed token roles
# --------------------------------------------------------------------------

def _canvas_lists(meta):
    """Per-segment canvas block indices as plain lists."""
    return [list(map(int, c)) for c in meta.canvas_block_idx]


def _offset(meta, s):
    """Block-grid offset o of segment s (0 when the metadata gives none)."""
    off = getattr(meta, "block_offset", None)
    return 0 if off is None else int(off[s])


def segment_layout(meta):
    """Per segment: (C, q0, canvases, q_offset, k_offset) in packed token units."""
    out = []
    qo = ko = 0
    B = int(meta.block_size)
    for s, C in enumerate(meta.ctx_len):
        C = int(C)
        q0 = int(meta.ctx_q_begin[s])
        cv = _canvas_lists(meta)[s]
        out.append((C, q0, cv, qo, ko))
        qo += (C - q0) + len(cv) * B
        ko += C + len(cv) * B
    return out


def query_roles(meta):
    """One tuple per packed query token: (segment, is_canvas, pos, canvas_id, b).

    pos is the context position for clean tokens and the offset inside the
    canvas for canvas tokens; canvas_id is the canvas' index in its segment
    (-1 for clean tokens) and b its block index (-1 for clean tokens).
    """
    B = int(meta.block_size)
    roles = []
    for s, (C, q0, cv, _qo, _ko) in enumerate(segment_layout(meta)):
        for p in range(q0, C):
            roles.append((s, False, p, -1, -1))
        for c, b in enumerate(cv):
            for t in range(B):
                roles.append((s, True, t, c, b))
    return roles


def key_roles(meta):
    """One tuple per packed key token, same fields as ``query_roles``."""
    B = int(meta.block_size)
    roles = []
    for s, (C, _q0, cv, _qo, _ko) in enumerate(segment_layout(meta)):
        for p in range(C):
            roles.append((s, False, p, -1, -1))
        for c, b in enumerate(cv):
            for t in range(B):
                roles.append((s, True, t, c, b))
    return roles


def visible(qr, kr, block_size, block_offset=0, clean_causal=False):
    """Block-diffusion visibility of key role ``kr`` from query role ``qr``.

    ORL section 3.2 "Staircase attention kernel" / appendix D.2. A canvas
    query at block b attends to clean keys of its document whose block index is
    below b, and to every token of its own canvas; nothing else (not the clean
    copy of block b, not later clean blocks, not other canvases, not other
    documents). A clean query attends to clean keys only, up to the end of its
    own block (or up to itself under the token-causal rule).
    ``block_offset`` is the offset o of the query's segment (context position p
    lies in block (p + o) // B); ``clean_causal`` selects token-causal clean
    rows.
    """
    qs, q_canvas, qpos, qc, qb = qr
    ks, k_canvas, kpos, kc, _kb = kr
    if qs != ks:                       # packed documents are mutually invisible
        return False

    def block(p):
        return (p + block_offset) // block_size

    if not q_canvas:                   # clean query: clean keys, block- or token-causal
        if k_canvas:
            return False
        return kpos <= qpos if clean_causal else block(kpos) <= block(qpos)
    if not k_canvas:                   # canvas query, clean key: blocks before b
        return block(kpos) < qb
    return kc == qc                    # canvas key: only its own canvas


def dense_mask(meta):
    """Boolean [Tq, Tk] visibility matrix built pair by pair (small inputs only)."""
    qr = query_roles(meta)
    kr = key_roles(meta)
    B = int(meta.block_size)
    causal = bool(getattr(meta, "clean_causal", False))
    m = np.zeros((len(qr), len(kr)), dtype=bool)
    for i, a in enumerate(qr):
        o = _offset(meta, a[0])
        for j, b in enumerate(kr):
            m[i, j] = visible(a, b, B, o, causal)
    return m


def visible_pairs(meta):
    """Number of visible (query token, key token) pairs, per query head.

    Counted from the visibility sets of ``_groups`` (one set per group of queries
    that see the same keys); the tests check it against ``dense_mask(meta).sum()``.
    """
    total = 0
    for _s, qidx, kidx in _groups(meta):
        total += len(qidx) * len(kidx)
    return total


# --------------------------------------------------------------------------
# dense form: explicit mask, one query head at a time
# --------------------------------------------------------------------------

def _scale(meta, scale):
    return (1.0 / math.sqrt(int(meta.head_dim))) if (scale is None or scale <= 0) else float(scale)


def attention_fwd_dense(q, k, v, meta, scale=None, mask=None):
    """O and LSE by the definition, with an explicit [Tq, Tk] mask.

    q [Tq, Hq, D], k/v [Tk, Hkv, D] (any real dtype, used as float64).
    Returns o [Tq, Hq, D] float64 and lse [Tq, Hq] float64.
    """
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
    sc = _scale(meta, scale)
    if mask is None:
        mask = dense_mask(meta)
    Tq, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    o = np.zeros((Tq, Hq, D))
    lse = np.zeros((Tq, Hq))
    for h in range(Hq):
        g = h // G
        s = sc * (q[:, h, :] @ k[:, g, :].T)
        s = np.where(mask, s, -np.inf)
        mx = s.max(axis=1, keepdims=True)
        p = np.exp(s - mx)
        l = p.sum(axis=1, keepdims=True)
        p = p / l
        o[:, h, :] = p @ v[:, g, :]
        lse[:, h] = mx[:, 0] + np.log(l[:, 0])
    return o, lse


def attention_bwd_dense(q, k, v, do, meta, scale=None, mask=None):
    """dQ, dK, dV of L = <dO, O> by the analytic formulas, explicit mask.

    dp = dO V^T; delta = sum_j p dp; ds = p (dp - delta);
    dq = scale ds K; dk = scale ds^T Q (summed over the heads of a kv group);
    dv = p^T dO (same sum).
    """
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64); do = np.asarray(do, np.float64)
    sc = _scale(meta, scale)
    if mask is None:
        mask = dense_mask(meta)
    Tq, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    dq = np.zeros_like(q); dk = np.zeros_like(k); dv = np.zeros_like(v)
    for h in range(Hq):
        g = h // G
        s = np.where(mask, sc * (q[:, h, :] @ k[:, g, :].T), -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p = p / p.sum(axis=1, keepdims=True)
        dp = do[:, h, :] @ v[:, g, :].T
        delta = (p * dp).sum(axis=1, keepdims=True)
        ds = p * (dp - delta)
        dq[:, h, :] = sc * (ds @ k[:, g, :])
        dk[:, g, :] += sc * (ds.T @ q[:, h, :])
        dv[:, g, :] += p.T @ do[:, h, :]
    return dq, dk, dv


# --------------------------------------------------------------------------
# range form: visible key ranges derived from the per-segment metadata
# --------------------------------------------------------------------------

def _groups(meta, segments=None):
    """Groups of query tokens that see the same keys, with those keys.

    Yields (segment, query token indices, key token indices). The sets follow
    the same rule as ``visible``. With block-grid offset o, block j covers the
    context positions [jB - o, (j+1)B - o): the clean queries of block j see
    the clean keys [0, (j+1)B - o); with token-causal clean rows, the clean
    query at position p sees [0, p + 1); canvas c (block index b) sees the
    clean keys [0, bB - o) and its own B tokens.
    """
    B = int(meta.block_size)
    causal = bool(getattr(meta, "clean_causal", False))
    for s, (C, q0, cv, qo, ko) in enumerate(segment_layout(meta)):
        if segments is not None and s not in segments:
            continue
        o = _offset(meta, s)
        nq_clean = C - q0
        if causal:
            for p in range(q0, C):
                yield s, np.arange(qo + (p - q0), qo + (p - q0) + 1), np.arange(ko, ko + p + 1)
        else:
            for j in range((q0 + o) // B, (C + o + B - 1) // B):
                lo = max(q0, j * B - o)
                hi = min(C, (j + 1) * B - o)
                if hi <= lo:
                    continue
                qidx = np.arange(qo + (lo - q0), qo + (hi - q0))
                kidx = np.arange(ko, ko + hi)
                yield s, qidx, kidx
        for c, b in enumerate(cv):
            qstart = qo + nq_clean + c * B
            kstart = ko + C + c * B
            qidx = np.arange(qstart, qstart + B)
            kidx = np.concatenate([np.arange(ko, ko + max(0, b * B - o)), np.arange(kstart, kstart + B)])
            yield s, qidx, kidx


def _group_scores(q, k, qidx, kidx, G, sc):
    """Scaled scores for one group, shape [Hkv, G, nq, nk]."""
    nq = len(qidx)
    Hq, D = q.shape[1], q.shape[2]
    Hkv = Hq // G
    qg = q[qidx].reshape(nq, Hkv, G, D).transpose(1, 2, 0, 3)        # Hkv, G, nq, D
    kg = np.ascontiguousarray(k[kidx].transpose(1, 2, 0))             # Hkv, D, nk
    return sc * np.matmul(qg, kg[:, None, :, :])


def attention_fwd(q, k, v, meta, scale=None, segments=None):
    """O and LSE, evaluating each query only over its visible key ranges.

    Same result as ``attention_fwd_dense``. ``segments`` (optional iterable of
    segment indices) restricts the work; rows of other segments stay zero.
    """
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64); v = np.asarray(v, np.float64)
    sc = _scale(meta, scale)
    Tq, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    o = np.zeros((Tq, Hq, D))
    lse = np.zeros((Tq, Hq))
    seg = None if segments is None else set(segments)
    for _s, qidx, kidx in _groups(meta, seg):
        nq = len(qidx)
        s = _group_scores(q, k, qidx, kidx, G, sc)                      # Hkv, G, nq, nk
        mx = s.max(axis=-1, keepdims=True)
        p = np.exp(s - mx)
        l = p.sum(axis=-1, keepdims=True)
        vg = np.ascontiguousarray(v[kidx].transpose(1, 0, 2))[:, None]  # Hkv, 1, nk, D
        og = np.matmul(p / l, vg)                                       # Hkv, G, nq, D
        o[qidx] = og.transpose(2, 0, 1, 3).reshape(nq, Hq, D)
        lse[qidx] = (mx[..., 0] + np.log(l[..., 0])).transpose(2, 0, 1).reshape(nq, Hq)
    return o, lse


def attention_bwd(q, k, v, do, meta, scale=None, segments=None):
    """dQ, dK, dV of L = <dO, O>, each query over its visible key ranges.

    Same formulas as ``attention_bwd_dense``; keys receive the sum over every
    query group (and every head of their kv group) that sees them.
    """
    q = np.asarray(q, np.float64); k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64); do = np.asarray(do, np.float64)
    sc = _scale(meta, scale)
    Tq, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    dq = np.zeros_like(q); dk = np.zeros_like(k); dv = np.zeros_like(v)
    seg = None if segments is None else set(segments)
    for _s, qidx, kidx in _groups(meta, seg):
        nq = len(qidx)
        s = _group_scores(q, k, qidx, kidx, G, sc)                      # Hkv, G, nq, nk
        p = np.exp(s - s.max(axis=-1, keepdims=True))
        p = p / p.sum(axis=-1, keepdims=True)
        dog = do[qidx].reshape(nq, Hkv, G, D).transpose(1, 2, 0, 3)     # Hkv, G, nq, D
        vg = np.ascontiguousarray(v[kidx].transpose(1, 2, 0))[:, None]  # Hkv, 1, D, nk
        dp = np.matmul(dog, vg)                                         # Hkv, G, nq, nk
        delta = (p * dp).sum(axis=-1, keepdims=True)
        ds = p * (dp - delta)
        kg = np.ascontiguousarray(k[kidx].transpose(1, 0, 2))[:, None]  # Hkv, 1, nk, D
        dqg = sc * np.matmul(ds, kg)                                    # Hkv, G, nq, D
        dq[qidx] = dqg.transpose(2, 0, 1, 3).reshape(nq, Hq, D)
        qg = q[qidx].reshape(nq, Hkv, G, D).transpose(1, 2, 0, 3)
        dkg = sc * np.matmul(ds.transpose(0, 1, 3, 2), qg).sum(axis=1)  # Hkv, nk, D
        dvg = np.matmul(p.transpose(0, 1, 3, 2), dog).sum(axis=1)       # Hkv, nk, D
        dk[kidx] += dkg.transpose(1, 0, 2)
        dv[kidx] += dvg.transpose(1, 0, 2)
    return dq, dk, dv
