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


# ------------------------------------------------------------- the gradient

def _tiny(seed, V=7):
    rng = np.random.default_rng(seed)
    N = 10
    x = rng.standard_normal((N, V)) * rng.uniform(0.5, 3.0, size=(N, 1))
    unres = [int(u) for u in rng.random(N) < 0.7]
    rows = [0, 3, 6, 8, 10]
    nxt = [1, 2, 3, 0, 7]                 # the last names no state
    hs = list(rng.uniform(0.0, 1.0, size=5))
    hs[3] = float("nan")                  # no captured source mean
    w = list(rng.uniform(0.2, 1.0, size=5))
    return x, unres, rows, nxt, hs, w


def _fd(x, args, eps=1e-6):
    g = np.zeros_like(x)
    for i in range(x.shape[0]):
        for v in range(x.shape[1]):
            xp, xm = x.copy(), x.copy()
            xp[i, v] += eps
            xm[i, v] -= eps
            g[i, v] = (ao.aec_forward(xp, *args)[3] - ao.aec_forward(xm, *args)[3]) / (2 * eps)
    return g


@pytest.mark.parametrize("seed,rho,gate", [(0, 0.1, math.inf), (1, 0.0, math.inf), (2, 0.3, 0.6), (3, 0.9, 0.8)])
def test_gradient_by_central_differences(seed, rho, gate):
    x, unres, rows, nxt, hs, w = _tiny(seed)
    args = (unres, rows, nxt, hs, w, rho, gate)
    g = ao.aec_backward(x, *args)
    fd = _fd(x, args)
    assert np.abs(g - fd).max() <= 1e-6 * max(1.0, np.abs(fd).max())
    assert ao.aec_backward(x, *args, grad_loss=2.5) == pytest.approx(2.5 * g, abs=1e-15)


def test_gradient_matches_torch_autograd():
    torch = pytest.importorskip("torch")
    x, unres, rows, nxt, hs, w = _tiny(5, V=11)
    rho = 0.2
    t = torch.tensor(x, dtype=torch.float64, requires_grad=True)
    logp = torch.log_softmax(t, dim=1)
    hbar = -(logp.exp() * logp).sum(1) / math.log(x.shape[1])
    means = []
    for s in range(len(rows) - 1):
        sel = [i for i in range(rows[s], rows[s + 1]) if unres[i]]
        means.append(hbar[sel].mean() if sel else None)
    num = torch.zeros((), dtype=torch.float64)
    den = 0.0
    for n, h_src, wt in zip(nxt, hs, w):
        if not (0 <= n < len(means)) or means[n] is None or not math.isfinite(h_src):
            continue
        num = num + wt * torch.clamp(means[n] - (1 - rho) * h_src, min=0.0) ** 2
        den += wt
    (num / den).backward()
    g = ao.aec_backward(x, unres, rows, nxt, hs, w, rho, math.inf)
    np.testing.assert_allclose(g, t.grad.numpy(), rtol=0, atol=1e-13)


def test_gradient_is_zero_without_kept_pairs():
    x, unres, rows, nxt, hs, w = _tiny(4)
    assert not ao.aec_backward(x, unres, rows, nxt, hs, w, 0.1, -1.0).any()      # every pair gated off
    # every hinge closed (H_next <= 1 = (1 - 0) * H_source): no gradient either
    assert not ao.aec_backward(x, unres, rows, nxt, [1.0] * 5, w, 0.0, math.inf).any()


def test_planted_gradient_mistake_is_caught():
    x, unres, rows, nxt, hs, w = _tiny(0)
    args = (unres, rows, nxt, hs, w, 0.1, math.inf)
    good = ao.aec_backward(x, *args)
    V = x.shape[1]
    lse = np.log(np.exp(x).sum(1, keepdims=True))
    p = np.exp(x - lse)
    # dropping the entropy term of dHbar/dx (only -p log p / log V)
    scale = np.divide(good, -p * ((x - lse) + (-(p * (x - lse)).sum(1, keepdims=True))) / math.log(V),
                      out=np.zeros_like(good), where=good != 0)
    bad = scale * (-p * (x - lse)) / math.log(V)
    fd = _fd(x, args)
    assert np.abs(good - fd).max() < 1e-6 < np.abs(bad - fd).max()
