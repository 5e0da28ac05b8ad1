"""Shared test helpers: golden-file reader and the parity comparator."""
from __future__ import annotations

import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

# Tolerances. bf16: max-abs 2e-2 and mean-abs 2e-3 (the stated parity bar) plus a
# relative Frobenius bound, because with near-uniform softmax the absolute values of
# O and of the gradients are ~1e-3..1e-4 and would let a zero tensor pass.
BF16_MAX_ABS = 2e-2
BF16_MEAN_ABS = 2e-3
BF16_REL_FRO = 1e-2
FP32_MAX_ABS = 1e-5
FP32_REL_FRO = 1e-5


def read_golden_matrix(name):
    rows, meta = [], {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line:
                continue
            if line.startswith("#"):
                if line.startswith("# meta:"):
                    for kv in line[len("# meta:"):].split():
                        k, v = kv.split("=")
                        meta[k] = v
                continue
            rows.append([float(x) for x in line.split()])
    return np.array(rows), meta


def error_stats(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    d = np.abs(got - ref)
    nref = float(np.linalg.norm(ref.ravel()))
    rel = float(np.linalg.norm((got - ref).ravel())) / max(nref, 1e-300)
    return {"max_abs": float(d.max()) if d.size else 0.0,
            "mean_abs": float(d.mean()) if d.size else 0.0,
            "rel_fro": rel if d.size else 0.0,
            "finite": bool(np.isfinite(got).all())}


def within(stats, dtype):
    if not stats["finite"]:
        return False
    if dtype == "fp32":
        return stats["max_abs"] <= FP32_MAX_ABS and stats["rel_fro"] <= FP32_REL_FRO
    return (stats["max_abs"] <= BF16_MAX_ABS and stats["mean_abs"] <= BF16_MEAN_ABS
            and stats["rel_fro"] <= BF16_REL_FRO)


def assert_close(name, got, ref, dtype):
    st = error_stats(got, ref)
    assert within(st, dtype), f"{name}: {st} ({dtype})"
    return st
