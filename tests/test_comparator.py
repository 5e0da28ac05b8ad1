"""The parity comparator rejects what a broken kernel would return (CPU only).

With inputs ~ N(0,1)/sqrt(128) the softmax is nearly uniform, so |O| ~ 1e-3 and the
gradients are smaller still: a zero tensor would pass max-abs/mean-abs alone. The
relative Frobenius bound must reject zeros and results computed under a mutated
visibility rule, while accepting the oracle's own result rounded to bf16.
"""
import numpy as np
import pytest

from oracle import bd_oracle as orc
from block_diffusion_attention_amd.workloads import Meta, random_workload, round_bf16
from helpers import error_stats, within


def _wl():
    meta = Meta([256], [0], [[2, 5, 7]], 32, 4, 1, 128, "bf16")
    return random_workload(np.random.default_rng(5), meta, sigma=1 / np.sqrt(128))


def test_rounded_oracle_passes_and_zeros_fail():
    wl = _wl()
    o, _ = orc.attention_fwd(wl.q, wl.k, wl.v, wl.meta)
    dq, dk, dv = orc.attention_bwd(wl.q, wl.k, wl.v, wl.do, wl.meta)
    for i, x in enumerate((o, dq, dk, dv)):
        assert within(error_stats(round_bf16(x.astype(np.float32)), x), "bf16")
        zero = error_stats(np.zeros_like(x), x)
        if i in (1, 2):   # dQ and dK: the absolute bars alone would accept zeros
            assert zero["max_abs"] < 2e-2 and zero["mean_abs"] < 2e-3
        assert not within(zero, "bf16")


def _mutant_sees_own_block(qr, kr, B, *_):
    qs, qc, _, _, qb = qr
    ks, kc, kp, _, _ = kr
    if qs == ks and qc and not kc:
        return kp // B <= qb
    return ORIG(qr, kr, B)


def _mutant_token_causal(qr, kr, B, *_):
    qs, qc, qp, _, _ = qr
    ks, kc, kp, _, _ = kr
    if qs == ks and not qc and not kc:
        return kp <= qp
    return ORIG(qr, kr, B)


ORIG = orc.visible


@pytest.mark.parametrize("mutant", [_mutant_sees_own_block, _mutant_token_causal])
def test_mutated_mask_fails(monkeypatch, mutant):
    wl = _wl()
    o_ref, _ = orc.attention_fwd(wl.q, wl.k, wl.v, wl.meta)
    g_ref = orc.attention_bwd(wl.q, wl.k, wl.v, wl.do, wl.meta)
    monkeypatch.setattr(orc, "visible", mutant)
    mask = orc.dense_mask(wl.meta)
    o_bad, _ = orc.attention_fwd_dense(wl.q, wl.k, wl.v, wl.meta, mask=mask)
    g_bad = orc.attention_bwd_dense(wl.q, wl.k, wl.v, wl.do, wl.meta, mask=mask)
    assert not within(error_stats(o_bad, o_ref), "bf16")
    assert any(not within(error_stats(a, r), "bf16") for a, r in zip(g_bad, g_ref))
