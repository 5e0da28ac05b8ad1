"""Decodes a serialized plan (host copy) into Python records, and rebuilds the
visibility those records encode, so tests can compare it with the oracle."""
from __future__ import annotations

import numpy as np

MAGIC = 0x62646174
SECTIONS = ["qtiles", "fwd", "split", "merge", "dq", "ktiles", "canvq", "bwd", "bmerge"]
WIDTH = {"qtiles": 8, "fwd": 4, "split": 16, "merge": 16, "dq": 4, "ktiles": 8, "canvq": 4, "bwd": 4, "bmerge": 4}


def decode(blob):
    b = np.asarray(blob, dtype=np.int64)
    assert b[0] == MAGIC and b[1] == 3
    out = {}
    for i, name in enumerate(SECTIONS):
        cnt, off = int(b[2 + 2 * i]), int(b[3 + 2 * i])
        assert off % 4 == 0
        w = WIDTH[name]
        out[name] = b[off:off + cnt * w].reshape(cnt, w) if w > 1 else b[off:off + cnt]
    return out


def _grain(meta):
    """Step of the clean row limits: the block size, or 1 for token-causal clean rows."""
    return 1 if getattr(meta, "clean_causal", False) else meta.block_size


def qtile_visibility(rec, meta, G):
    """Boolean [Tq, Tk] visibility encoded by the query tiles (each token once per tile).

    A clean tile's row limit is the first row's limit raised by the grain at
    every multiple of the grain its grid position (pos0 + t) crosses."""
    Bc = _grain(meta)
    vis = np.zeros((meta.tq, meta.tk), dtype=bool)
    cover = np.zeros(meta.tq, dtype=np.int64)
    for q_tok, n_tok, k_ctx, pos0, lim_max, lim_min, k_own, n_own in rec["qtiles"]:
        for t in range(n_tok):
            L = lim_min + ((pos0 + t) // Bc - pos0 // Bc) * Bc if pos0 >= 0 else lim_min
            assert L <= lim_max and L >= lim_min
            vis[q_tok + t, k_ctx:k_ctx + L] = True
            vis[q_tok + t, k_own:k_own + n_own] = True
            cover[q_tok + t] += 1
    return vis, cover


def ktile_visibility(rec, meta, G):
    """Boolean [Tq, Tk] visibility encoded by the key tiles and canvas-query entries
    (key-side positions are grid positions)."""
    Bc = _grain(meta)
    vis = np.zeros((meta.tq, meta.tk), dtype=bool)
    cover = np.zeros(meta.tk, dtype=np.int64)
    cv = rec["canvq"]
    for k_tok, n_keys, p0, cq_tok, cq_len, cq_pos, cv_begin, cv_count in rec["ktiles"]:
        cover[k_tok:k_tok + n_keys] += 1
        for kk in range(n_keys):
            key = k_tok + kk
            for t in range(cq_len):
                L = ((cq_pos + t) // Bc + 1) * Bc
                if p0 >= 0 and p0 + kk < L:
                    vis[cq_tok + t, key] = True
            for e in range(cv_begin, cv_begin + cv_count):
                q_tok, n_tok, lim, own = cv[e]
                if own or (p0 >= 0 and p0 + kk < lim):
                    vis[q_tok:q_tok + n_tok, key] = True
    return vis, cover
