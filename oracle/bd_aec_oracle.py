"""Plain fp64 CPU oracle of the normalized-entropy / adjacent-entropy-contraction
(AEC) reduction over vocabulary logits.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. It imports
nothing from the library.

What is computed (ORL paper, the paragraph "Learning how fast to refine", which
defines the normalized entropy, the unresolved-state mean and the AEC hinge, and
the appendix paragraph on valid AEC pairs, their weights w_R and the gate):
  * for every position i with logits x_i over a vocabulary V: the softmax p_i,
    its natural-log normalizer lse_i = log sum_v exp(x_iv) (the log-normalizer
    that a later softmax over the same logits can reuse, appendix F.1
    "Kernels"), and its normalized entropy Hbar_i = -sum_v p_iv log p_iv / log|V|;
  * for every state s (a block of positions): the mean of Hbar over its
    unresolved (still masked) positions;
  * for every pair (source state, next state): the hinge
    max(0, H_next - (1 - rho) H_source)^2, where H_next is the replayed next
    state's mean and H_source the captured mean of the source state;
  * the loss: sum over valid pairs of w * g * hinge / D with D = sum of w * g
    over valid pairs, and 0 when D = 0.

Readings of points the pages leave open:
  * the equation that combines the pairs was lost in extraction; the plainest
    reading of the surrounding text (weights w given before gating, D the
    weighted count of retained pairs, zero loss for D = 0) is the weighted mean
    above;
  * a pair is valid when its next state exists (index in [0, S)), has at least
    one unresolved position, and its source mean is a finite number (the caller
    marks a source without unresolved positions with NaN);
  * the gate keeps a pair when H_source <= gate_max (gate_max = +inf keeps
    every pair, the LLaDA setting; 0.20 is the QwenDLM setting);
  * a state with no unresolved position has mean NaN.

Parity pins (tests/test_aec_oracle.py): scipy's entropy and logsumexp, uniform
logits (Hbar = 1), a closed form for one raised logit, hand-worked state means
and losses under tests/golden/, and planted mistakes.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = ["lse_and_entropy", "state_means", "aec_loss", "aec_forward", "aec_backward"]


def lse_and_entropy(logits):
    """Per row: natural-log normalizer and entropy / log|V| (float64)."""
    x = np.asarray(logits, np.float64)
    V = x.shape[1]
    m = x.max(axis=1, keepdims=True)
    e = np.exp(x - m)
    s = e.sum(axis=1, keepdims=True)
    lse = m[:, 0] + np.log(s[:, 0])
    logp = x - lse[:, None]
    p = np.exp(logp)
    h = -(p * logp).sum(axis=1)
    return lse, h / math.log(V)


def state_means(hbar, unresolved, state_rows):
    """Mean normalized entropy over the unresolved rows of each state; NaN if none."""
    out = np.full(len(state_rows) - 1, np.nan)
    for s in range(len(state_rows) - 1):
        lo, hi = int(state_rows[s]), int(state_rows[s + 1])
        sel = [i for i in range(lo, hi) if unresolved[i]]
        if sel:
            out[s] = sum(hbar[i] for i in sel) / len(sel)
    return out


def aec_loss(h_state, pair_next, h_source, weight, rho, gate_max):
    """Weighted mean of the gated hinge over valid pairs (0 when nothing is kept)."""
    num = den = 0.0
    for n, hs, w in zip(pair_next, h_source, weight):
        if not 0 <= int(n) < len(h_state):      # no such state: not a valid pair
            continue
        hn = h_state[int(n)]
        if not (math.isfinite(hs) and math.isfinite(hn)):
            continue
        g = 1.0 if hs <= gate_max else 0.0
        hinge = max(0.0, hn - (1.0 - rho) * hs)
        num += w * g * hinge * hinge
        den += w * g
    return num / den if den > 0 else 0.0


def aec_forward(logits, unresolved, state_rows, pair_next, h_source, weight, rho, gate_max):
    """Everything at once: (lse, hbar, per-state means, loss)."""
    lse, hbar = lse_and_entropy(logits)
    hs = state_means(hbar, unresolved, state_rows)
    return lse, hbar, hs, aec_loss(hs, pair_next, h_source, weight, rho, gate_max)


def aec_backward(logits, unresolved, state_rows, pair_next, h_source, weight, rho, gate_max, grad_loss=1.0):
    """Gradient of grad_loss * loss with respect to the logits (float64, [N, V]).

    By the chain rule through the definitions above:
      dL/dH_next(n) = sum over kept valid pairs p with next n of 2 w_p hinge_p / D
                      (hinge_p taken before squaring; 0 where the hinge is 0);
      dH_state/dHbar_i = 1 / (unresolved rows of the state) for its unresolved rows;
      dHbar_i/dx_iv = -p_iv (log p_iv + H_i) / log|V|, H_i the entropy in nats.
    The captured source means are constants (detached).
    """
    x = np.asarray(logits, np.float64)
    N, V = x.shape
    lse, hbar = lse_and_entropy(x)
    hs = state_means(hbar, unresolved, state_rows)
    den = 0.0
    kept = []
    for n, h_src, w in zip(pair_next, h_source, weight):
        n = int(n)
        if not 0 <= n < len(hs):
            continue
        if not (math.isfinite(h_src) and math.isfinite(hs[n])):
            continue
        if not h_src <= gate_max:
            continue
        den += w
        kept.append((n, h_src, w))
    g_state = np.zeros(len(hs))
    if den > 0:
        for n, h_src, w in kept:
            hinge = max(0.0, hs[n] - (1.0 - rho) * h_src)
            g_state[n] += 2.0 * w * hinge / den
    g_row = np.zeros(N)
    for s in range(len(state_rows) - 1):
        rows = [i for i in range(int(state_rows[s]), int(state_rows[s + 1])) if unresolved[i]]
        for i in rows:
            g_row[i] += g_state[s] / len(rows)
    logp = x - lse[:, None]
    p = np.exp(logp)
    H = hbar * math.log(V)
    return grad_loss * g_row[:, None] * (-p * (logp + H[:, None])) / math.log(V)
