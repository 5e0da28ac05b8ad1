"""Workloads and planted records for the record-checking kernels (plans made
with BD_ATTN_FLAG_DEBUG_CHECKS), used by test_gpu_device_checks.py; the binding
module is passed in."""
from __future__ import annotations

import numpy as np
import torch

from block_diffusion_attention_amd import workloads as W
from plan_decode import SECTIONS, WIDTH

# (name, meta factory, plan flag names): every kernel and both record paths of
# the forward (direct / split + merge, with and without transposed V), the split
# dK/dV with its merge, token-causal clean rows, a ragged shape and fp32
CASES = [
    ("fp32", lambda: W.config_meta(1, np.random.default_rng(1)), ()),
    ("denoise, split forward", lambda: W.config_meta(2, np.random.default_rng(2)), ()),
    ("denoise, split forward, transposed V", lambda: W.config_meta(2, np.random.default_rng(2)), ("FLAG_FWD_VT",)),
    ("staircase, split dK/dV", lambda: W.config_meta(4, np.random.default_rng(4)), ()),
    ("staircase, transposed V", lambda: W.config_meta(4, np.random.default_rng(4)), ("FLAG_FWD_VT",)),
    ("staircase, forced split", lambda: W.config_meta(4, np.random.default_rng(4)), ("FLAG_FORCE_SPLIT",)),
    ("packed replay", lambda: W.config_meta(3, np.random.default_rng(3)), ()),
    ("ragged: B=3, G=3, D=64, token-causal", lambda: W.random_meta(
        np.random.default_rng(90), max_segments=3, max_blocks=12, block_sizes=(3,), max_canvases=4,
        hq=6, hkv=2, d=64, dtype="bf16", clean_causal=True), ("FLAG_FORCE_SPLIT",)),
    ("fp32 random pack: B in {4, 8}, G=2, D=64", lambda: W.random_meta(
        np.random.default_rng(7), max_segments=3, max_blocks=6, block_sizes=(4, 8), max_canvases=3,
        hq=4, hkv=2, d=64, dtype="fp32"), ()),
]


def flags_of(b, names) -> int:
    f = 0
    for n in names:
        f |= getattr(b, n)
    return f


def run_case(b, meta, flags, seed=5, plan=None):
    """Forward and backward on seeded device-generated inputs, into outputs that
    start at zero; returns the plan (a new one unless given) and the outputs (on
    the GPU)."""
    if plan is None:
        plan = b.Plan(meta, flags).upload("cuda")
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    hq, hkv, d = meta.num_q_heads, meta.num_kv_heads, meta.head_dim

    def rnd(n, h, s):
        return (torch.randn(n, h, d, generator=g, device="cuda") * s).to(plan.dtype).contiguous()

    q, k, v, do = rnd(plan.tq, hq, 0.5), rnd(plan.tk, hkv, 0.5), rnd(plan.tk, hkv, 1.0), rnd(plan.tq, hq, 1.0)
    out = {n: torch.zeros_like(t) for n, t in (("o", q), ("dq", q), ("dk", k), ("dv", v))}
    out["lse"] = torch.zeros(plan.tq, hq, device="cuda", dtype=torch.float32)
    b.fwd(plan, q, k, v, o=out["o"], lse=out["lse"])
    b.bwd(plan, q, k, v, out["o"], out["lse"], do, dq=out["dq"], dk=out["dk"], dv=out["dv"])
    torch.cuda.synchronize()
    return plan, out


def _sections(blob):
    return {n: (int(blob[2 + 2 * i]), int(blob[3 + 2 * i])) for i, n in enumerate(SECTIONS)}


def _rec(blob, secs, name, i):
    cnt, off = secs[name]
    w = WIDTH[name]
    return off + i * w


def plant(meta, plan, blob, sections):
    """Plants one record out of range per named section in a copy of the
    work-list image:
      fwd, dq        : kv head = Hkv (forward / dQ item; an fp32 plan's forward reads the
                       dQ items too, so there the record is rejected twice)
      split, merge   : kv head = Hkv (split-forward part / merge block)
      bwd            : chunk range with begin = end + 1 (dK/dV item)
      bmerge         : kv head = Hkv (dK/dV merge)
      bwd_kvh        : kv head = Hkv in a dK/dV item of an fp32 plan (never split there)
    Each record is picked so that following it unchecked would still stay inside
    every tensor and workspace (checked here with asserts): a kv head of Hkv
    addresses head 0 of the next token, so the tiles chosen end before the last
    query and key token; an inverted chunk range visits no chunk. Returns the
    modified image and the number of workgroups the checks must reject (one per
    record, and one per workgroup of a dK/dV merge record)."""
    hkv, d = meta.num_kv_heads, meta.head_dim
    tq, tk = plan.tq, plan.tk
    blob = list(blob)
    secs = _sections(blob)

    def clear_of_end(t):
        q_tok, n_tok, k_ctx, _, lim_max, _, k_own, n_own = t
        return q_tok + n_tok < tq and k_ctx + lim_max < tk and (n_own == 0 or k_own + n_own < tk)

    def qtile_at(i):
        o = _rec(blob, secs, "qtiles", i)
        return blob[o:o + 8]

    def ktile_clear_of_end(i):
        ko = _rec(blob, secs, "ktiles", i)
        k_tok, n_keys, _, cq_tok, cq_len, _, cv_begin, cv_count = blob[ko:ko + 8]
        if k_tok + n_keys >= tk or (cq_len > 0 and cq_tok + cq_len >= tq):
            return False
        for e in range(cv_begin, cv_begin + cv_count):
            co = _rec(blob, secs, "canvq", e)
            if blob[co] + blob[co + 1] >= tq:
                return False
        return True

    fp32 = meta.dtype != "bf16"

    def pick(sec, ok):
        cnt, _ = secs[sec]
        assert cnt > 0, f"the plan has no {sec} records"
        for i in list(range(cnt // 2, cnt)) + list(range(cnt // 2)):
            o = _rec(blob, secs, sec, i)
            if ok(o):
                return o
        raise AssertionError(f"no {sec} record to plant")

    expect = 0
    for sec in sections:
        if sec in ("fwd", "dq"):
            o = pick(sec, lambda o: blob[o] >= 0 and clear_of_end(qtile_at(blob[o])))
            blob[o + 1] = hkv
            expect += 2 if fp32 and sec == "dq" else 1
        elif sec in ("split", "merge"):
            o = pick(sec, lambda o: blob[o + 8] >= 0 and clear_of_end(blob[o:o + 8]))
            blob[o + 8] = hkv
            expect += 1
        elif sec == "bwd":
            o = pick(sec, lambda o: blob[o] >= 0 and blob[o + 3] < 2 ** 31 - 1)   # not an open end
            blob[o + 2] = blob[o + 3] + 1
            expect += 1
        elif sec == "bmerge":
            def kt_clear(o):
                ko = _rec(blob, secs, "ktiles", blob[o])
                return blob[ko] + blob[ko + 1] < tk
            o = pick(sec, kt_clear)
            blob[o + 1] = hkv
            expect += 128 * (d // 4) // 256      # workgroups per dK/dV merge record
        elif sec == "bwd_kvh":
            assert fp32, "bwd_kvh plants an fp32 plan's dK/dV item"
            o = pick("bwd", lambda o: blob[o] >= 0 and ktile_clear_of_end(blob[o]))
            blob[o + 1] = hkv
            expect += 1
        else:
            raise ValueError(sec)
    return blob, expect


# (case index, sections planted)
PLANTS = [(3, ("fwd", "dq", "bwd", "bmerge")), (5, ("split", "merge", "bmerge")), (8, ("dq", "bwd_kvh"))]
