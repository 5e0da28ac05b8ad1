"""Host-side accounting of bench.py (no GPU): the useful FLOPs of a step, the
algorithmic work per kernel, the dominant kernel's roofline, the per-pass rates,
the gate on stored counter figures, and the refusal of more than one GPU.

The FLOP count of the headline workload is pinned to a closed form of its visible
pairs and to the oracle's own count; the serving step's bytes to its tensor shapes
worked out by hand.
"""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from block_diffusion_attention_amd import workloads as W
from oracle import bd_oracle as orc

b = pytest.importorskip("block_diffusion_attention_amd.binding")

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _plan(k):
    meta = W.config_meta(k, np.random.default_rng(k))
    return meta, b.Plan(meta)


def test_packed_replay_pairs_closed_form():
    # A replay segment of n clean blocks of 32 tokens with one canvas at block n:
    # clean block j sees 32 (j + 1) keys with its 32 queries, the canvas sees all
    # 32 n clean keys and its own 32, so 1024 (n (n + 1) / 2 + n + 1) pairs, which
    # is 512 (n + 1)(n + 2).
    n = np.random.default_rng(3).integers(8, 129, size=16)
    closed = int(sum(512 * (int(x) + 1) * (int(x) + 2) for x in n))
    meta, plan = _plan(3)
    assert plan.visible_pairs == orc.visible_pairs(meta) == closed
    # the step's useful FLOPs: 4 D (forward) + 10 D (backward) per pair and query head
    assert bench.useful_flop(128, 32, closed, True) == 14 * 128 * 32 * closed
    assert bench.useful_flop(128, 32, closed, False) == 4 * 128 * 32 * closed


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5, 6])
def test_useful_flop_counts_the_oracle_pairs(k):
    meta, plan = _plan(k)
    pairs = orc.visible_pairs(meta)
    assert plan.visible_pairs == pairs
    D, Hq = meta.head_dim, meta.num_q_heads
    assert bench.useful_flop(D, Hq, pairs, True) == 14.0 * D * Hq * pairs
    work = bench.kernel_work(k, meta.dtype, D, Hq, meta.num_kv_heads, plan.tq, plan.tk, pairs)
    # the two backward kernels execute 14 D per pair for the pass's useful 10 D
    assert work["dkdv"] == ("mfma", 8.0 * D * Hq * pairs)
    assert work["dq"] == ("mfma", 6.0 * D * Hq * pairs)
    assert work["dkdv_masked"] == work["dkdv"]


def test_denoising_step_forward_bytes():
    # 32 canvas tokens x 32 query heads x 128 dims of bf16 queries, and 2,048 clean +
    # 32 canvas keys x 8 kv heads x 128 dims for each of K and V
    meta, plan = _plan(2)
    assert (plan.tq, plan.tk) == (32, 2080)
    q_bytes = 32 * 32 * 128 * 2
    kv_bytes = 2080 * 8 * 128 * 2
    work = bench.kernel_work(2, "bf16", 128, 32, 8, plan.tq, plan.tk, plan.visible_pairs)
    assert work["fwd"] == ("hbm", float(q_bytes + 2 * kv_bytes)) == ("hbm", 8781824.0)
    # the merge writes O (bf16) and LSE (fp32) of every canvas row once
    assert work["merge"] == ("hbm", q_bytes + 32 * 32 * 4)
    # with O and LSE, the step's compulsory bytes
    assert q_bytes + 2 * kv_bytes + q_bytes + 32 * 32 * 4 == 9048064
    # the training workloads price their forward in FLOPs
    assert bench.kernel_work(3, "bf16", 128, 32, 8, 10, 10, 7)["fwd"] == ("mfma", 4.0 * 128 * 32 * 7)


def test_roofline_of_the_dominant_kernel(monkeypatch):
    monkeypatch.setattr(bench, "traffic_from_profiles", lambda kernel, k: None)
    pairs = 34146304
    work = bench.kernel_work(3, "bf16", 128, 32, 8, 28256, 28256, pairs)
    roof = bench.roofline({"fwd": 0.55, "dq": 0.77, "dkdv": 1.15}, work, bench.PEAK_BF16_TFLOPS, 3)
    flop = 8.0 * 128 * 32 * pairs
    assert roof["kernel"] == "dkdv" and roof["bound"] == "mfma" and roof["unit"] == "TFLOP/s"
    assert roof["work_per_launch"] == flop
    assert roof["achieved"] == pytest.approx(flop / 1.15e-3 / 1e12, abs=0.01)
    assert roof["frac"] == pytest.approx(roof["achieved"] / 2516.6, abs=1e-4)
    # 256 CUs x 2.4 GHz x 4096 bf16 FLOP per clock and CU, to one decimal
    assert roof["peak"] == 2516.6 == pytest.approx(256 * 2.4 * 4096 / 1000, abs=0.05)
    # a serving step: the forward kernel is the longer one and is priced in bytes
    work2 = bench.kernel_work(2, "bf16", 128, 32, 8, 32, 2080, 1)
    roof2 = bench.roofline({"fwd": 0.009, "merge": 0.007}, work2, bench.PEAK_BF16_TFLOPS, 2)
    assert roof2["kernel"] == "fwd" and roof2["bound"] == "hbm" and roof2["unit"] == "GB/s"
    assert roof2["achieved"] == pytest.approx(8781824 / 9e-6 / 1e9, abs=0.1)
    assert roof2["peak"] == 8000.0 and roof2["frac"] == pytest.approx(roof2["achieved"] / 8000.0, abs=1e-4)


def test_pass_rates():
    pairs = 1000
    p = bench.pass_rates({"fwd": 0.5, "dq": 0.75, "dkdv": 1.25}, ["fwd"], ["dq", "dkdv"], 128, 32, pairs, 2516.6)
    fwd = 4.0 * 128 * 32 * pairs / 0.5e-3 / 1e12
    bwd = 10.0 * 128 * 32 * pairs / 2.0e-3 / 1e12
    assert p["fwd"]["ms"] == 0.5 and p["bwd"]["ms"] == 2.0
    assert p["fwd"]["useful_tflops"] == pytest.approx(fwd, abs=0.01)
    assert p["bwd"]["useful_tflops"] == pytest.approx(bwd, abs=0.01)
    assert p["bwd"]["pct_of_peak"] == pytest.approx(100 * p["bwd"]["useful_tflops"] / 2516.6, abs=0.01)
    assert set(bench.pass_rates({"fwd": 0.5, "merge": 0.25}, ["fwd", "merge"], None, 128, 32, pairs,
                                2516.6)) == {"fwd"}


def test_stored_counter_figures_only_for_unchanged_sources(tmp_path, monkeypatch):
    h = bench.src_hash(bench.KERNEL_SOURCES["dkdv"])
    (tmp_path / "profiles").mkdir()
    rec = {"dkdv@3": {"src_sha256": h, "bytes_per_launch": 123.0, "mfma_busy": 0.5, "clock_ghz": 1.7,
                      "executed_tflops": 900.0, "profiled_us": 1200.0}}
    for name in ("traffic.json", "mfma.json"):
        (tmp_path / "profiles" / name).write_text(json.dumps(rec))
    # the stored records sit under the temporary root; the hash of the sources is
    # the one just taken from the real tree
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "src_hash", lambda files: h if files == bench.KERNEL_SOURCES["dkdv"] else "other")
    assert bench.traffic_from_profiles("dkdv", 3) == 123.0
    assert bench.mfma_from_profiles("dkdv", 3)["mfma_busy"] == 0.5
    assert bench.traffic_from_profiles("dkdv", 4) is None          # no record
    # a changed source (or compiler flag) makes the stored figures stale
    monkeypatch.setattr(bench, "src_hash", lambda files: "changed")
    assert bench.traffic_from_profiles("dkdv", 3) is None
    assert bench.mfma_from_profiles("dkdv", 3) is None


def test_src_hash_covers_the_compiler_flags(monkeypatch):
    from block_diffusion_attention_amd import build as bd
    before = bench.src_hash(["attn_bwd.hip"])
    monkeypatch.setitem(bd.HIP_FILE_FLAGS, "attn_bwd.hip", bd.HIP_FILE_FLAGS.get("attn_bwd.hip", []) + ["-O2"])
    assert bench.src_hash(["attn_bwd.hip"]) != before


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], stdout=subprocess.PIPE,
                       stderr=subprocess.PIPE, text=True, timeout=120)
    assert r.returncode == 2
    assert r.stdout == ""
    assert "exactly one GPU" in r.stderr


CC_HEADER = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
             "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
             "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
DKDV = "void bdattn::(anonymous namespace)::dkdv_bf16_kernel<128, false, false>(bdattn::BwdArgs)"
COPY = "void at::native::vectorized_elementwise_kernel<4, at::native::MulFunctor<float>, std::array<char*, 3ul> >(int)"


def _write_csv(path, header, rows):
    import csv
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def _cc_row(dispatch, kernel, counter, value, t0, t1):
    return [dispatch, dispatch, "Agent 1", 1, 1, 1, 256, 1, kernel, 256, 0, 0, 128, 0, 32, counter, value, t0, t1]


def test_summary_of_profiler_output(tmp_path, monkeypatch, capsys):
    """The profile summaries' arithmetic on synthetic rocprofv3 output: the copy
    probe's scale factor and the bytes per launch it gives, and the MFMA busy
    fraction, clock and executed FLOPs of a kernel."""
    import argparse
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "src_hash", lambda files: "h")
    monkeypatch.setattr(bench, "MFMA_STATS", {})
    (tmp_path / "profiles").mkdir()
    # kernel statistics
    _write_csv(tmp_path / "kt" / "run_kernel_stats.csv",
               ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"],
               [[DKDV, 3, 3600000, 1200000, 70.0, 1100000, 1300000]])
    # FETCH_SIZE (KiB per dispatch): the 256 MiB copy probe's largest dispatch counts
    # 2 x 256 MiB, so the scale factor is 0.5; dK/dV counts 1000 and 1200 KiB in its
    # two dispatches
    probe = 2 * 256 * 1024.0
    _write_csv(tmp_path / "fs" / "run_counter_collection.csv", CC_HEADER,
               [_cc_row(1, COPY, "FETCH_SIZE", 4.0, 0, 10),
                _cc_row(2, COPY, "FETCH_SIZE", probe, 0, 10),
                _cc_row(3, DKDV, "FETCH_SIZE", 1000.0, 0, 10),
                _cc_row(4, DKDV, "FETCH_SIZE", 1200.0, 0, 10)])
    args = argparse.Namespace(summarize=[str(tmp_path / "kt"), str(tmp_path / "fs")], command="cmd",
                              copy_probe_mb=256, summary_out=str(tmp_path / "s.md"), mfma_key=None,
                              traffic_key="dkdv@3")
    bench.summarize(args)
    text = (tmp_path / "s.md").read_text()
    assert "| bdattn::dkdv_bf16_kernel<128, false, false> | 3 | 1200.00 | 1100.00 | 1300.00 | 70.0 |" in text
    assert "FETCH_SIZE=0.5000" in text
    rec = json.loads((tmp_path / "profiles" / "traffic.json").read_text())["dkdv@3"]
    assert rec["bytes_per_launch"] == pytest.approx(1100.0 * 1024 * 0.5)
    assert rec["src_sha256"] == "h" and rec["command"] == "cmd"
    # MFMA counters of two dispatches of 1 ms: GRBM_GUI_ACTIVE summed over the 8 XCDs
    # is 8 x 1.7e6 cycles (1.7 GHz), the 1,024 SIMDs were MFMA-busy for half of them,
    # and 2e9 MFMA operations of 512 FLOPs each ran
    cyc = 1.7e6
    rows = []
    for d in (1, 2):
        for name, val in (("SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * cyc * 1024), ("GRBM_GUI_ACTIVE", 8 * cyc),
                          ("SQ_INSTS_VALU_MFMA_MOPS_BF16", 2e9)):
            rows.append(_cc_row(d, DKDV, name, val, 0, 1000000))
    _write_csv(tmp_path / "mf" / "run_counter_collection.csv", CC_HEADER, rows)
    args = argparse.Namespace(summarize=[str(tmp_path / "mf")], command="cmd2", copy_probe_mb=0,
                              summary_out=None, mfma_key=["dkdv@3"], traffic_key=None)
    bench.summarize(args)
    m = json.loads((tmp_path / "profiles" / "mfma.json").read_text())["dkdv@3"]
    assert m["mfma_busy"] == 0.5
    assert m["clock_ghz"] == 1.7
    assert m["executed_tflops"] == pytest.approx(2e9 * 512 / 1e-3 / 1e12, abs=0.1)
    assert m["profiled_us"] == 1000.0
    assert m["src_sha256"] == "h"


def test_denoising_step_compulsory_bytes():
    # Q (32 x 32 x 128 bf16) and O read/written once, K and V (2,080 x 8 x 128 bf16) read
    # once, LSE (32 x 32 fp32) written once: the step's GB/s is these bytes over its time
    meta, plan = _plan(2)
    assert bench.step_bytes("bf16", 128, 32, 8, plan.tq, plan.tk) == 9048064
    assert bench.step_bytes("fp32", 64, 2, 1, 80, 80) == 2 * 80 * 2 * 64 * 4 + 2 * 80 * 64 * 4 + 80 * 2 * 4


def test_cpu_model_is_named():
    name = bench.cpu_model()
    assert name is None or (isinstance(name, str) and name)
