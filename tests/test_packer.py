"""Replay-row packer and largest-cost-first assignment (CPU only).

* the oracle against a hand-worked example (tests/golden/), Graham's bound for
  largest-cost-first list scheduling against brute-force optima, and structural
  invariants; a planted ordering mistake breaks the bound;
* the library's bd_attn_pack against the oracle, bit for bit;
* the response-normalized loss summed as sum(num) / sum(den) over groups equals
  the unpacked objective for any assignment;
* a group's rows form a valid attention plan whose visibility is the oracle's.
"""
import os

import numpy as np
import pytest

from oracle import bd_oracle as orc
from oracle import bd_pack_oracle as po
from pack_common import group_meta

b = pytest.importorskip("block_diffusion_attention_amd.binding")
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "pack_three_responses.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, v = line.split(":", 1)
        vals[k.strip()] = [int(x) for x in v.split()]
    return vals


def _states(resp, block, step, sup=None, pages=None):
    out = []
    for i in range(len(resp)):
        st = {"resp": int(resp[i]), "block": int(block[i]), "step": int(step[i])}
        if sup is not None:
            st["supervised"] = int(sup[i])
        if pages is not None:
            st["pages"] = int(pages[i])
        out.append(st)
    return out


def test_golden_example_oracle_and_library():
    g = _golden()
    B, G = g["block_size"][0], g["groups"][0]
    states = _states(g["state_resp"], g["state_block"], g["state_step"])
    rows, group, members, load = po.pack(g["clean_len"], None, states, B, G)
    assert [r["resp"] for r in rows] == g["row_resp"]
    assert [r["step"] for r in rows] == g["row_step"]
    assert [r["ctx"] for r in rows] == g["row_ctx_len"]
    assert [r["cost"] for r in rows] == g["row_cost"]
    assert group == g["row_group"]
    assert members == [g["group0_rows"], g["group1_rows"]]
    assert load == g["group_cost"]
    p = b.pack(g["clean_len"], g["state_resp"], g["state_block"], g["state_step"], B, G)
    assert list(p["row_ctx_len"]) == g["row_ctx_len"] and list(p["row_cost"]) == g["row_cost"]
    assert list(p["row_group"]) == g["row_group"]
    assert list(p["group_rows"]) == g["group0_rows"] + g["group1_rows"]
    assert list(p["group_cost"]) == g["group_cost"]


def _graham_ok(costs, G, assign):
    _, _, load = assign(costs, G)
    opt = po.optimal_makespan(costs, G)
    return max(load) * 3 * G <= (4 * G - 1) * opt      # LPT <= (4/3 - 1/(3G)) OPT


def test_largest_first_meets_grahams_bound():
    rng = np.random.default_rng(5)
    for _ in range(150):
        G = int(rng.integers(2, 4))
        costs = [int(x) for x in rng.integers(1, 40, size=int(rng.integers(G + 1, 8)))]
        assert _graham_ok(costs, G, po.assign_largest_first), (costs, G)


def test_planted_smallest_first_breaks_the_bound():
    def smallest_first(costs, G):
        load = [0] * G
        for r in sorted(range(len(costs)), key=lambda r: (costs[r], r)):
            g = min(range(G), key=lambda x: (load[x], x))
            load[g] += costs[r]
        return None, None, load
    rng = np.random.default_rng(5)
    broken = 0
    for _ in range(150):
        G = int(rng.integers(2, 4))
        costs = [int(x) for x in rng.integers(1, 40, size=int(rng.integers(G + 1, 8)))]
        broken += not _graham_ok(costs, G, smallest_first)
    assert broken > 0


def _random_instance(rng, R=None, B=None):
    R = R or int(rng.integers(1, 9))
    B = B or int(rng.choice([1, 2, 4, 16, 32]))
    nb = rng.integers(0, 9, size=R)
    off = [int(rng.integers(0, B)) if n > 0 else 0 for n in nb]
    clean = [int(n) * B - o for n, o in zip(nb, off)]
    N = int(rng.integers(0, 40))
    resp = rng.integers(0, R, size=N)
    block = [int(rng.integers(0, nb[r] + 1)) for r in resp]
    step = rng.integers(0, 6, size=N)
    sup = rng.integers(0, B + 1, size=N)
    pages = rng.integers(0, 50, size=N)
    return clean, off, resp, block, step, sup, pages, B


@pytest.mark.parametrize("seed", range(20))
def test_library_matches_oracle(seed):
    rng = np.random.default_rng(1000 + seed)
    clean, off, resp, block, step, sup, pages, B = _random_instance(rng)
    G = int(rng.integers(1, 9))
    w = [int(x) for x in rng.integers(0, 5, size=3)]
    states = _states(resp, block, step, sup, pages)
    rows, group, members, load = po.pack(clean, off, states, B, G, *w)
    p = b.pack(clean, resp, block, step, B, G, block_offset=off, state_supervised=sup, state_pages=pages,
               w_tokens=w[0], w_supervised=w[1], w_pages=w[2])
    assert p["n_rows"] == len(rows)
    assert list(p["row_resp"]) == [r["resp"] for r in rows]
    assert list(p["row_step"]) == [r["step"] for r in rows]
    assert list(p["row_ctx_len"]) == [r["ctx"] for r in rows]
    assert list(p["row_cost"]) == [r["cost"] for r in rows]
    assert list(p["row_group"]) == group
    flat = [r for m in members for r in m]
    assert list(p["group_rows"]) == flat
    assert list(p["group_cost"]) == load
    for i, r in enumerate(rows):
        got = p["row_states"][p["row_state_offsets"][i]:p["row_state_offsets"][i + 1]]
        assert list(got) == r["states"]
        assert all(p["state_row"][s] == i for s in r["states"])


@pytest.mark.parametrize("seed", range(10))
def test_row_invariants(seed):
    rng = np.random.default_rng(2000 + seed)
    clean, off, resp, block, step, sup, pages, B = _random_instance(rng)
    states = _states(resp, block, step)
    rows = po.build_rows(clean, off, states, B)
    seen = sorted(i for r in rows for i in r["states"])
    assert seen == list(range(len(states))), "every state in exactly one row"
    for r in rows:
        assert {(states[i]["resp"], states[i]["step"]) for i in r["states"]} == {(r["resp"], r["step"])}
        # every state sees the clean context it needs, and no clean token is held
        # that none of the row's states sees
        needs = [min(max(states[i]["block"] * B - off[r["resp"]], 0), clean[r["resp"]]) for i in r["states"]]
        assert r["ctx"] == max(needs)
    assert len({(r["resp"], r["step"]) for r in rows}) == len(rows)


@pytest.mark.parametrize("G", [1, 2, 3, 8])
def test_num_den_reduction_is_assignment_invariant(G):
    rng = np.random.default_rng(30 + G)
    clean, off, resp, block, step, sup, pages, B = _random_instance(rng, R=6, B=4)
    while len(resp) < 10:                 # enough states to spread over the groups
        clean, off, resp, block, step, sup, pages, B = _random_instance(rng, R=6, B=4)
    states = _states(resp, block, step, sup)
    losses = [list(rng.random(int(s["supervised"]))) for s in states]
    # unpacked objective: mean over responses (that have labels) of the mean of their labels
    per = {}
    for s, l in zip(states, losses):
        per.setdefault(s["resp"], []).extend(l)
    per = {k: v for k, v in per.items() if v}
    if not per:
        pytest.skip("no labels drawn")
    want = np.mean([np.mean(v) for v in per.values()])
    rows, _g, members, _l = po.pack(clean, off, states, B, G)
    terms = po.group_loss_terms(rows, members, states, losses)
    got = sum(t[0] for t in terms) / sum(t[1] for t in terms)
    assert abs(got - want) <= 1e-12


@pytest.mark.parametrize("over,msg", [
    (dict(num_groups=0), "num_groups"),
    (dict(block_size=0), "block_size"),
    (dict(state_resp=[0, 3]), "state_resp"),
    (dict(state_block=[0, 9]), "state_block"),
    (dict(state_step=[0, -1]), "state_step"),
    (dict(clean_len=[65, 32]), "clean_len"),
    (dict(block_offset=[40, 0]), "block_offset"),
    (dict(w_tokens=-1), "weights"),
])
def test_pack_validation(over, msg):
    args = dict(clean_len=[64, 32], state_resp=[0, 1], state_block=[2, 1], state_step=[0, 0],
                block_size=32, num_groups=2)
    kw = {k: over.pop(k) for k in ("block_offset", "w_tokens") if k in over}
    args.update(over)
    with pytest.raises(b.BdAttnError) as e:
        b.pack(**args, **kw)
    assert e.value.status == b.EINVAL and msg in str(e.value)


def test_group_rows_form_a_valid_attention_plan():
    rng = np.random.default_rng(77)
    clean, off, resp, block, step, sup, pages, B = _random_instance(rng, R=8, B=4)
    G = 3
    p = b.pack(clean, resp, block, step, B, G, block_offset=off)
    for g in range(G):
        if p["group_row_offsets"][g + 1] == p["group_row_offsets"][g]:
            continue
        meta = group_meta(p, g, clean, off, block, B, 4, 2, 64, "bf16")
        plan = b.Plan(meta)
        assert plan.visible_pairs == orc.visible_pairs(meta)


def test_empty_batch_and_more_groups_than_rows():
    p = b.pack([64, 32], [], [], [], 32, 4)
    assert p["n_rows"] == 0 and list(p["group_row_offsets"]) == [0] * 5 and not p["group_cost"].any()
    # three rows over five groups: one row each in the first three groups, largest first
    p = b.pack([64, 96, 32], [0, 1, 2], [2, 3, 1], [0, 0, 0], 32, 5)
    assert p["n_rows"] == 3
    assert list(p["group_row_offsets"]) == [0, 1, 2, 3, 3, 3]
    assert list(p["group_rows"]) == [1, 0, 2]          # costs 128, 96, 64
    assert list(p["group_cost"]) == [128, 96, 64, 0, 0]


def test_row_with_only_block_zero_states_holds_no_clean_token():
    # states at block 0 see no clean token; with a grid offset the row still
    # needs none, and its attention plan takes offset 0
    p = b.pack([29], [0, 0], [0, 0], [3, 3], 32, 1, block_offset=[3])
    assert p["n_rows"] == 1 and p["row_ctx_len"][0] == 0 and p["row_cost"][0] == 64
    meta = group_meta(p, 0, [29], [3], [0, 0], 32, 4, 2, 64, "bf16")
    assert meta.block_offset == [0]
    assert b.Plan(meta).visible_pairs == orc.visible_pairs(meta)
