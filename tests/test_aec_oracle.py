"""Pins of the normalized-entropy / AEC oracle to things other than itself (CPU).

* hand-worked closed forms under tests/golden/ (entropies, state means, losses);
* scipy: stats.entropy (natural log) divided by log|V|, special.logsumexp;
* uniform logits give Hbar = 1 for any vocabulary; one raised logit has a
  closed form; shifting a row's logits changes lse by the shift and Hbar not at all;
* hinge and gate edge cases; planted mistakes in the entropy are caught.
"""
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp
from scipy.stats import entropy

from oracle import bd_aec_oracle as ao

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "aec_four_rows.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split(":", 1)
            vals[k.strip()] = [float(x) for x in v.split()]
    return vals


def test_golden_closed_forms():
    g = _golden()
    logits = np.array([g[f"logits_row{i}"] for i in range(4)])
    unres = [int(x) for x in g["unresolved"]]
    rows = [int(x) for x in g["state_rows"]]
    nxt = [int(x) for x in g["pair_next"]]
    lse, hbar, hs, loss = ao.aec_forward(logits, unres, rows, nxt, g["pair_h_source"], g["pair_weight"],
                                         g["rho"][0], math.inf)
    np.testing.assert_allclose(lse, g["lse"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(hbar[:3], g["hbar_rows012"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(hs, g["state_mean"], rtol=0, atol=1e-14)
    assert abs(loss - g["loss_gate_inf"][0]) <= 1e-15
    loss2 = ao.aec_loss(hs, nxt, g["pair_h_source"], g["pair_weight"], g["rho"][0], 0.85)
    assert abs(loss2 - g["loss_gate_085"][0]) <= 1e-15


@pytest.mark.parametrize("V", [2, 7, 1000, 151936])
def test_matches_scipy(V):
    rng = np.random.default_rng(V)
    x = rng.standard_normal((3, V)) * np.array([[0.1], [2.0], [8.0]])
    lse, hbar = ao.lse_and_entropy(x)
    np.testing.assert_allclose(lse, logsumexp(x, axis=1), rtol=1e-13, atol=0)
    p = np.exp(x - logsumexp(x, axis=1, keepdims=True))
    want = entropy(p, axis=1) / np.log(V)
    np.testing.assert_allclose(hbar, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("V", [2, 3, 50257, 151936])
def test_uniform_is_one_and_shift_invariance(V):
    x = np.zeros((2, V))
    x[1] += 37.5
    lse, hbar = ao.lse_and_entropy(x)
    np.testing.assert_allclose(hbar, 1.0, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, [math.log(V), 37.5 + math.log(V)], rtol=1e-15)


@pytest.mark.parametrize("V,a", [(4, 3.0), (1000, 10.0), (151936, 20.0)])
def test_one_raised_logit_closed_form(V, a):
    # logits (a, 0, ..., 0): p_0 = e^a / (e^a + V - 1), the rest (1 - p_0) / (V - 1)
    x = np.zeros((1, V))
    x[0, 0] = a
    z = math.exp(a) + V - 1
    p0 = math.exp(a) / z
    q = 1.0 / z
    H = -(p0 * math.log(p0) + (V - 1) * q * math.log(q))
    lse, hbar = ao.lse_and_entropy(x)
    assert abs(lse[0] - math.log(z)) <= 1e-12
    assert abs(hbar[0] - H / math.log(V)) <= 1e-12


def test_hinge_gate_and_empty_cases():
    hs = np.array([0.5, np.nan, 0.9])
    # next state below (1 - rho) * source: hinge 0
    assert ao.aec_loss(hs, [0], [0.9], [1.0], 0.1, math.inf) == 0.0
    # a next state without unresolved positions or a NaN source: the pair is not valid
    assert ao.aec_loss(hs, [1, 0], [0.1, float("nan")], [1.0, 1.0], 0.0, math.inf) == 0.0
    # a next-state index outside [0, S) names no state: not a valid pair
    assert ao.aec_loss(hs, [-1, 3, 0], [0.1, 0.1, 0.9], [1.0, 1.0, 1.0], 0.1, math.inf) == 0.0
    # every pair gated off: D = 0, loss 0
    assert ao.aec_loss(hs, [2], [0.5], [1.0], 0.0, 0.2) == 0.0
    # rho = 1: the hinge is H_next^2
    assert abs(ao.aec_loss(hs, [2], [0.3], [2.0], 1.0, math.inf) - 0.81) <= 1e-15
    # weights normalize: two identical pairs with weights 1 and 3 give one pair's hinge
    assert abs(ao.aec_loss(hs, [2, 2], [0.5, 0.5], [1.0, 3.0], 0.0, math.inf) - 0.16) <= 1e-15
    assert np.isnan(ao.state_means(np.array([0.3, 0.4]), [0, 0], [0, 2])[0])


def test_planted_mistakes_are_caught(monkeypatch):
    g = _golden()
    logits = np.array([g[f"logits_row{i}"] for i in range(4)])
    orig = ao.lse_and_entropy

    def log2_normalizer(x):                  # entropy in nats divided by log2|V|
        lse, h = orig(x)
        return lse, h * math.log(x.shape[1]) / math.log2(x.shape[1])

    def unnormalized_p(x):                   # p = exp(x) without the normalizer
        x = np.asarray(x, np.float64)
        p = np.exp(x)
        return logsumexp(x, axis=1), -(p * x).sum(1) / math.log(x.shape[1])

    for bad in (log2_normalizer, unnormalized_p):
        monkeypatch.setattr(ao, "lse_and_entropy", bad)
        _, hbar = ao.lse_and_entropy(logits)
        assert np.abs(hbar[:3] - g["hbar_rows012"]).max() > 1e-3
    monkeypatch.setattr(ao, "lse_and_entropy", orig)
