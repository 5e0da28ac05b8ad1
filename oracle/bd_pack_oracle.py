"""Plain CPU oracle of the replay-row packer and its group assignment.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. It imports
nothing from the library.

What is computed (ORL paper, section 3.2 "Packed and cost-balanced state
training" and appendix D.3):
  * one row per (response, step): the response's clean tokens stored a single
    time, followed by that step's captured block states, each placed as a
    canvas at its own block index so that it attends to the clean prefix in
    the row rather than to a private copy;
  * rows of different responses sit side by side as separate documents with no
    attention between them;
  * a weighted proxy of sequence tokens, supervised positions and resident pages
    is each row's estimated cost, and rows go to data-parallel groups largest
    cost first, deterministically;
  * each group returns numerators and denominators of the response-normalized
    losses; the global loss is sum(num) / sum(den), which does not depend on the
    packing or the assignment (up to rounding).

Readings of points the pages leave open:
  * a row keeps the clean tokens its states can see, i.e. the context below the
    clean copy of its furthest block: max over its states of (b*B - o), clamped
    to [0, C] (clean tokens no state of the row sees add cost and nothing else);
  * rows are numbered by (response, step); within a row the states keep their
    input order;
  * largest-cost-first is list scheduling in decreasing cost: ties between rows
    go to the lower row number, each row to the group with the least total cost
    so far, ties to the lowest group index;
  * integer weights, so that costs and loads are exact.

Parity pins (tests/test_packer.py): a hand-worked example under tests/golden/,
Graham's bound for largest-cost-first against brute-force optima on small
instances, structural invariants (every state in exactly one row, one response
and step per row, minimal clean length), and the num/den invariance.
"""
from __future__ import annotations

import itertools

__all__ = ["build_rows", "assign_largest_first", "pack", "group_loss_terms", "optimal_makespan"]


def build_rows(clean_len, block_offset, states, B, w_tokens=1, w_supervised=0, w_pages=0):
    """Rows from the captured states.

    ``states``: list of dicts with keys resp, block, step and optionally
    supervised (default B) and pages (default 0). Returns a list of rows, each a
    dict: resp, step, states (indices), ctx (clean tokens held), cost.
    """
    groups = {}
    for i, st in enumerate(states):
        groups.setdefault((st["resp"], st["step"]), []).append(i)
    rows = []
    for (resp, step) in sorted(groups):
        idx = groups[(resp, step)]
        o = block_offset[resp] if block_offset is not None else 0
        furthest = max(states[i]["block"] for i in idx)
        ctx = min(max(furthest * B - o, 0), clean_len[resp])
        tokens = ctx + len(idx) * B
        sup = sum(states[i].get("supervised", B) for i in idx)
        pages = sum(states[i].get("pages", 0) for i in idx)
        rows.append({"resp": resp, "step": step, "states": idx, "ctx": ctx,
                     "cost": w_tokens * tokens + w_supervised * sup + w_pages * pages})
    return rows


def assign_largest_first(costs, G):
    """Largest-cost-first list scheduling; returns (group of each item, rows per
    group in assignment order, load per group)."""
    order = sorted(range(len(costs)), key=lambda r: (-costs[r], r))
    load = [0] * G
    group = [None] * len(costs)
    members = [[] for _ in range(G)]
    for r in order:
        g = min(range(G), key=lambda x: (load[x], x))
        group[r] = g
        members[g].append(r)
        load[g] += costs[r]
    return group, members, load


def pack(clean_len, block_offset, states, B, G, w_tokens=1, w_supervised=0, w_pages=0):
    """Rows and their assignment: (rows, group of each row, rows per group, load per group)."""
    rows = build_rows(clean_len, block_offset, states, B, w_tokens, w_supervised, w_pages)
    group, members, load = assign_largest_first([r["cost"] for r in rows], G)
    return rows, group, members, load


def group_loss_terms(rows, members, states, label_losses):
    """Numerator and denominator of the response-normalized loss for each group.

    ``label_losses[i]`` holds the per-label losses of state i. A response's
    labels are weighted by 1 / (its label count), so each response counts once
    (responses without labels drop out); the global loss is sum(num) / sum(den).
    """
    per_resp = {}
    for i, st in enumerate(states):
        per_resp[st["resp"]] = per_resp.get(st["resp"], 0) + len(label_losses[i])
    out = []
    for mem in members:
        num = den = 0.0
        for r in mem:
            for i in rows[r]["states"]:
                if not label_losses[i]:          # no labels: nothing to weigh
                    continue
                w = 1.0 / per_resp[states[i]["resp"]]
                num += w * sum(label_losses[i])
                den += w * len(label_losses[i])
        out.append((num, den))
    return out


def optimal_makespan(costs, G):
    """Smallest possible largest group load, by trying every assignment (tiny inputs)."""
    best = None
    for assign in itertools.product(range(G), repeat=len(costs)):
        load = [0] * G
        for c, g in zip(costs, assign):
            load[g] += c
        m = max(load)
        best = m if best is None else min(best, m)
    return best if best is not None else 0
