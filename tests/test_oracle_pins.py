"""Pins of the CPU oracle to things other than itself (CPU only).

* the hand-worked visibility matrices under tests/golden/ (the base rule, a
  shifted block grid, the commit-folded step); a shifted grid equals the
  aligned grid without its first tokens;
* special cases that reduce to torch's scaled_dot_product_attention (CPU, fp64):
  one block -> bidirectional attention, block size 1 -> causal attention,
  canvas at the last block index in canvas-only mode -> unmasked attention,
  grouped-query attention -> multi-head attention with repeated K/V;
  token-causal clean rows -> causal attention; the commit-folded step -> causal
  rows plus an unmasked canvas; a lone partial first block -> bidirectional;
* torch SDPA with the oracle's explicit boolean mask (forward and autograd);
* central finite differences of the forward for the analytic gradients.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import bd_oracle as orc
from block_diffusion_attention_amd.workloads import Meta, random_meta, random_workload
from helpers import read_golden_matrix


def _sdpa(q, k, v, mask=None, causal=False, scale=None):
    """torch SDPA on [T, H, D] float64 arrays; kv heads repeated per group."""
    G = q.shape[1] // k.shape[1]
    tq = torch.tensor(q, dtype=torch.float64).permute(1, 0, 2)[None]
    tk = torch.tensor(k, dtype=torch.float64).repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    tv = torch.tensor(v, dtype=torch.float64).repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    am = None if mask is None else torch.tensor(mask)
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=am, is_causal=causal, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def _sdpa_grads(q, k, v, do, mask=None, causal=False, scale=None):
    G = q.shape[1] // k.shape[1]
    tq = torch.tensor(q, dtype=torch.float64, requires_grad=True)
    tk = torch.tensor(k, dtype=torch.float64, requires_grad=True)
    tv = torch.tensor(v, dtype=torch.float64, requires_grad=True)
    qq = tq.permute(1, 0, 2)[None]
    kk = tk.repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    vv = tv.repeat_interleave(G, dim=1).permute(1, 0, 2)[None]
    am = None if mask is None else torch.tensor(mask)
    o = F.scaled_dot_product_attention(qq, kk, vv, attn_mask=am, is_causal=causal, scale=scale)
    o = o[0].permute(1, 0, 2)
    (o * torch.tensor(do, dtype=torch.float64)).sum().backward()
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def _wl(meta, seed, sigma=1.0):
    return random_workload(np.random.default_rng(seed), meta, sigma=sigma, with_do=True)


# ---------------------------------------------------------------- golden mask

def test_golden_mask_replay():
    gold, m = read_golden_matrix("mask_b2_two_canvases.txt")
    meta = Meta([int(m["ctx_len"])], [int(m["ctx_q_begin"])],
                [[int(x) for x in m["canvases"].split(",")]], int(m["block_size"]), 1, 1, 4)
    mask = orc.dense_mask(meta)
    assert mask.shape == gold.shape
    assert (mask == gold.astype(bool)).all()


def test_golden_mask_canvas_only_rows():
    # Canvas-only mode (q0 = C) keeps exactly the canvas rows of the same matrix.
    gold, m = read_golden_matrix("mask_b2_two_canvases.txt")
    meta = Meta([4], [4], [[1, 2]], 2, 1, 1, 4)
    assert (orc.dense_mask(meta) == gold[4:].astype(bool)).all()


def test_two_documents_block_diagonal():
    # Packed documents are mutually invisible: the mask of a pack is block-diagonal
    # with the masks of its documents on the diagonal.
    a = Meta([4], [0], [[1, 2]], 2, 1, 1, 4)
    b = Meta([6], [2], [[0, 3]], 2, 1, 1, 4)
    ab = Meta([4, 6], [0, 2], [[1, 2], [0, 3]], 2, 1, 1, 4)
    ma, mb, mab = orc.dense_mask(a), orc.dense_mask(b), orc.dense_mask(ab)
    top = np.concatenate([ma, np.zeros((ma.shape[0], mb.shape[1]), bool)], 1)
    bot = np.concatenate([np.zeros((mb.shape[0], ma.shape[1]), bool), mb], 1)
    assert (mab == np.concatenate([top, bot], 0)).all()


def _golden_meta(m):
    off = [int(m["block_offset"])] if "block_offset" in m else None
    return Meta([int(m["ctx_len"])], [int(m["ctx_q_begin"])],
                [[int(x) for x in m["canvases"].split(",")]], int(m["block_size"]), 1, 1, 4,
                block_offset=off, clean_causal=m.get("clean_causal") == "1")


@pytest.mark.parametrize("name", ["mask_b2_offset1_three_canvases.txt",
                                  "mask_b2_commit_folded_token_causal.txt"])
def test_golden_masks_offset_and_commit(name):
    gold, m = read_golden_matrix(name)
    mask = orc.dense_mask(_golden_meta(m))
    assert mask.shape == gold.shape
    assert (mask == gold.astype(bool)).all()


def test_commit_folded_block_causal_rows():
    # Block-causal commit rows see their whole block: the same rows of the
    # two-canvas golden matrix (queries c2 c3 and canvas Y at block index 2).
    gold, _ = read_golden_matrix("mask_b2_two_canvases.txt")
    mask = orc.dense_mask(Meta([4], [2], [[2]], 2, 1, 1, 4))
    want = gold[[2, 3, 6, 7]][:, [0, 1, 2, 3, 6, 7]]
    assert (mask == want.astype(bool)).all()


@pytest.mark.parametrize("B,n,o", [(2, 3, 1), (4, 3, 3), (3, 4, 2), (5, 2, 4)])
def test_offset_grid_is_the_aligned_grid_without_its_first_tokens(B, n, o):
    # A grid offset o is the aligned grid of n whole blocks with its first o
    # context tokens removed: the mask of (C = nB - o, offset o) is the mask of
    # (C = nB, offset 0) without the rows and columns of those tokens.
    cv = [list(range(n + 1))]
    shifted = Meta([n * B - o], [0], cv, B, 1, 1, 4, block_offset=[o])
    aligned = Meta([n * B], [0], cv, B, 1, 1, 4)
    ma = orc.dense_mask(aligned)
    keep_q = [i for i in range(ma.shape[0]) if i >= o]
    keep_k = [j for j in range(ma.shape[1]) if j >= o]
    assert (orc.dense_mask(shifted) == ma[keep_q][:, keep_k]).all()
    assert orc.visible_pairs(shifted) == int(ma[keep_q][:, keep_k].sum())


# ------------------------------------------------------ SDPA special cases

@pytest.mark.parametrize("B,n,o", [(1, 6, 0), (4, 3, 0), (4, 3, 3), (8, 2, 5)])
def test_token_causal_clean_stream_is_causal(B, n, o):
    # Token-causal clean rows with no canvases: plain causal attention, whatever
    # the block size and the grid offset.
    meta = Meta([n * B - o], [0], [[]], B, 4, 2, 16, block_offset=[o], clean_causal=True)
    wl = _wl(meta, 40 + B + o)
    ref = _sdpa(wl.q, wl.k, wl.v, causal=True)
    o1, _ = orc.attention_fwd(wl.q, wl.k, wl.v, meta)
    np.testing.assert_allclose(o1, ref, rtol=0, atol=1e-12)
    od, _ = orc.attention_fwd_dense(wl.q, wl.k, wl.v, meta)
    np.testing.assert_allclose(od, ref, rtol=0, atol=1e-12)
    g = orc.attention_bwd(wl.q, wl.k, wl.v, wl.do, meta)
    r = _sdpa_grads(wl.q, wl.k, wl.v, wl.do, causal=True)
    for a, b in zip(g, r):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11)


@pytest.mark.parametrize("B,n", [(2, 3), (4, 4), (3, 2)])
def test_commit_folded_step_reduces_to_sdpa(B, n):
    # The commit-folded step with token-causal commit rows: the finished block's
    # rows are the last B rows of causal attention over the context, the canvas
    # at the next block index attends to the whole context and itself.
    C = n * B
    meta = Meta([C], [C - B], [[n]], B, 2, 1, 8, clean_causal=True)
    wl = _wl(meta, 70 + B)
    o, _ = orc.attention_fwd(wl.q, wl.k, wl.v, meta)
    full = _wl(Meta([C], [0], [[]], B, 2, 1, 8), 0)
    qc = np.concatenate([full.q[:C - B], wl.q[:B]], 0)     # any first rows: only the last B are compared
    ref_clean = _sdpa(qc, wl.k[:C], wl.v[:C], causal=True)[C - B:]
    np.testing.assert_allclose(o[:B], ref_clean, rtol=0, atol=1e-12)
    ref_canvas = _sdpa(wl.q[B:], wl.k, wl.v)
    np.testing.assert_allclose(o[B:], ref_canvas, rtol=0, atol=1e-12)


@pytest.mark.parametrize("B,o", [(4, 1), (8, 7)])
def test_partial_first_block_is_bidirectional(B, o):
    # A context that is only the partial first block (C = B - o) is one block:
    # every clean row sees every context key.
    meta = Meta([B - o], [0], [[]], B, 2, 2, 16, block_offset=[o])
    wl = _wl(meta, 90 + o)
    out, _ = orc.attention_fwd(wl.q, wl.k, wl.v, meta)
    np.testing.assert_allclose(out, _sdpa(wl.q, wl.k, wl.v), rtol=0, atol=1e-12)


@pytest.mark.parametrize("B", [1, 3, 8])
def test_single_block_is_bidirectional(B):
    # No context, one canvas at block index 0: the canvas sees only itself, all of it.
    meta = Meta([0], [0], [[0]], B, 4, 2, 16)
    wl = _wl(meta, 11 + B)
    o, _ = orc.attention_fwd_dense(wl.q, wl.k, wl.v, meta)
    np.testing.assert_allclose(o, _sdpa(wl.q, wl.k, wl.v), rtol=0, atol=1e-12)
    o2, _ = orc.attention_fwd(wl.q, wl.k, wl.v, meta)
    np.testing.assert_allclose(o2, _sdpa(wl.q, wl.k, wl.v), rtol=0, atol=1e-12)
    g = orc.attention_bwd(wl.q, wl.k, wl.v, wl.do, meta)
    r = _sdpa_grads(wl.q, wl.k, wl.v, wl.do)
    for a, b in zip(g, r):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11)


def test_single_clean_block_is_bidirectional():
    meta = Meta([8], [0], [[]], 8, 2, 2, 16)
    wl = _wl(meta, 5)
    o, _ = orc.attention_fwd(wl.q, wl.k, wl.v, meta)
    np.testing.assert_allclose(o, _sdpa(wl.q, wl.k, wl.v), rtol=0, atol=1e-12)


@pytest.mark.parametrize("n", [1, 5, 17])
def test_block_size_one_is_causal(n):
    meta = Meta([n], [0], [[]], 1, 4, 1, 16)
    wl = _wl(meta, 100 + n)
    o, _ = orc.attention_fwd(wl.q, wl.k, wl.v, meta)
    np.testing.assert_allclose(o, _sdpa(wl.q, wl.k, wl.v, causal=True), rtol=0, atol=1e-12)
    od, _ = orc.attention_fwd_dense(wl.q, wl.k, wl.v, meta)
    np.testing.assert_allclose(od, _sdpa(wl.q, wl.k, wl.v, causal=True), rtol=0, atol=1e-12)
    g = orc.attention_bwd(wl.q, wl.k, wl.v, wl.do, meta)
    r = _sdpa_grads(wl.q, wl.k, wl.v, wl.do, causal=True)
    for a, b in zip(g, r):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11)


@pytest.mark.parametrize("B,n", [(2, 3), (4, 4)])
def test_last_block_canvas_only_is_unmasked(B, n):
    # Canvas-only with b = n: the canvas sees the whole context and itself.
    meta = Meta([n * B], [n * B], [[n]], B, 2, 1, 8)
    wl = _wl(meta, 7)
    o, _ = orc.attention_fwd(wl.q, wl.k, wl.v, meta)
    np.testing.assert_allclose(o, _sdpa(wl.q, wl.k, wl.v), rtol=0, atol=1e-12)
    g = orc.attention_bwd(wl.q, wl.k, wl.v, wl.do, meta)
    r = _sdpa_grads(wl.q, wl.k, wl.v, wl.do)
    for a, b in zip(g, r):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11)


def test_gqa_equals_mha_with_repeated_kv():
    meta = Meta([6, 4], [0, 2], [[2, 0], [1]], 2, 6, 2, 8)
    mha = Meta([6, 4], [0, 2], [[2, 0], [1]], 2, 6, 6, 8)
    wl = _wl(meta, 3)
    k6 = np.repeat(wl.k, 3, axis=1); v6 = np.repeat(wl.v, 3, axis=1)
    o, lse = orc.attention_fwd(wl.q, wl.k, wl.v, meta)
    o6, lse6 = orc.attention_fwd(wl.q, k6, v6, mha)
    np.testing.assert_allclose(o, o6, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse, lse6, rtol=0, atol=1e-13)
    dq, dk, dv = orc.attention_bwd(wl.q, wl.k, wl.v, wl.do, meta)
    dq6, dk6, dv6 = orc.attention_bwd(wl.q, k6, v6, wl.do, mha)
    np.testing.assert_allclose(dq, dq6, rtol=0, atol=1e-12)
    # dK of the shared head is the sum over its group of the MHA gradients.
    np.testing.assert_allclose(dk, dk6.reshape(dk6.shape[0], 2, 3, -1).sum(2), rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv, dv6.reshape(dv6.shape[0], 2, 3, -1).sum(2), rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(6))
def test_sdpa_with_explicit_mask(seed):
    rng = np.random.default_rng(1000 + seed)
    meta = random_meta(rng, hq=4, hkv=2, d=8)
    wl = random_workload(rng, meta)
    mask = orc.dense_mask(meta)
    o, _ = orc.attention_fwd_dense(wl.q, wl.k, wl.v, meta, mask=mask)
    np.testing.assert_allclose(o, _sdpa(wl.q, wl.k, wl.v, mask=mask), rtol=0, atol=1e-12)
    g = orc.attention_bwd_dense(wl.q, wl.k, wl.v, wl.do, meta, mask=mask)
    r = _sdpa_grads(wl.q, wl.k, wl.v, wl.do, mask=mask)
    for a, b in zip(g, r):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-11)


def test_explicit_scale_matches_sdpa():
    meta = Meta([4], [0], [[2, 1]], 2, 2, 1, 8, softmax_scale=0.7)
    wl = _wl(meta, 9)
    mask = orc.dense_mask(meta)
    o, _ = orc.attention_fwd(wl.q, wl.k, wl.v, meta, scale=0.7)
    np.testing.assert_allclose(o, _sdpa(wl.q, wl.k, wl.v, mask=mask, scale=0.7), rtol=0, atol=1e-12)


# ------------------------------------------------------ finite differences

@pytest.mark.parametrize("seed", range(3))
def test_gradients_by_central_differences(seed):
    rng = np.random.default_rng(2000 + seed)
    meta = random_meta(rng, hq=2, hkv=1, d=4, max_blocks=3, block_sizes=(1, 2, 3))
    wl = random_workload(rng, meta)
    mask = orc.dense_mask(meta)
    q, k, v, do = (x.astype(np.float64) for x in (wl.q, wl.k, wl.v, wl.do))
    dq, dk, dv = orc.attention_bwd_dense(q, k, v, do, meta, mask=mask)

    def loss(qq, kk, vv):
        o, _ = orc.attention_fwd_dense(qq, kk, vv, meta, mask=mask)
        return float((o * do).sum())

    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(20):
            idx = tuple(int(rng.integers(0, s)) for s in x.shape)
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            fd = (loss(*args_p) - loss(*args_m)) / (2 * h)
            assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(g[idx])), (name, idx, fd, g[idx])
