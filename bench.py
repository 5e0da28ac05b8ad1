#!/usr/bin/env python3
"""Benchmark of the staircase block-diffusion attention on one MI355X.

A step is one forward and one backward pass (every kernel of the hot path) over
one packed batch of synthetic input already resident in HBM, with the plan
built once beforehand (as a model reuses one plan in every layer). The default
workload is the packed-replay pack: 16 segments, each a clean context of
256..4096 tokens (whole blocks of 32) followed by one 32-token canvas at the
next block index; 32 query / 8 kv heads, head_dim 128, bf16 inputs drawn from
N(0, 1/128) and dO from N(0, 1), seed 3.

Prints one JSON line: useful (visible-pair) TFLOP/s of the step, the roofline
of the dominant kernel (its algorithmic FLOPs or bytes per launch over its
average launch duration, timed with HIP events on the stream that runs it) and
the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA: 256 CUs x 2.4 GHz x 4096 FLOP/clk/CU
PEAK_FP32_TFLOPS = 157.3      # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E

METRIC = "useful TFLOP/s + % of bf16 MFMA peak, staircase block-diffusion attn fwd/bwd"
WORKLOAD_NAMES = {
    1: "tiny fp32: 64-token context (4 blocks of 16) + 1 canvas at block 4, 2q/1kv, D=64",
    2: "single-request denoising step: 2048-token context in KV + one 32-token canvas, 32q/8kv, D=128, bf16",
    3: "packed replay: 16 segments, contexts U[256,4096] in blocks of 32, one 32-token canvas each at the "
       "next block index, 32q/8kv, D=128, bf16, fwd+bwd",
    4: "staircase: 4096-token context + 24 canvases at distinct block indices in [1,128], 32q/8kv, D=128, "
       "bf16, fwd+bwd",
    5: "large pack: 4 x (8192-token context + 16 canvases), 32q/8kv, D=128, bf16, fwd+bwd",
    6: "commit-folded step: 2031-token context in KV (block grid offset 17), the finished 32-token block "
       "(token-causal) + the next canvas as queries, 32q/8kv, D=128, bf16, fwd",
}
FWD_ONLY = (2, 6)     # single-request serving steps: forward only, bandwidth-bound


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=3, choices=[1, 2, 3, 4, 5, 6])
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--flags", type=int, default=0, help="plan flags (BD_ATTN_FLAG_*)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="CPU oracle sample budget")
    ap.add_argument("--fwd-only", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step replayed from a captured HIP graph (no per-launch host cost); "
                         "value and ms_per_step then come from the replays")
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB (fp32 read + write), "
                         "the reference for scaling HBM byte counters")
    ap.add_argument("--summarize", metavar="DIR", nargs="+", default=None,
                    help="summarise rocprofv3 CSV output under the DIRs (no GPU work) and exit")
    ap.add_argument("--summary-out", default=None, help="with --summarize: write the text summary here")
    ap.add_argument("--command", default="", help="with --summarize: the command that produced DIR")
    ap.add_argument("--aec", action="store_true",
                    help="time the normalized-entropy / AEC reduction over vocabulary logits instead")
    ap.add_argument("--pack", action="store_true",
                    help="time the host packer (replay rows + largest-cost-first groups) instead; CPU only")
    ap.add_argument("--traffic-key", default=None,
                    help="with --summarize: record per-launch HBM bytes of KERNEL@WORKLOAD in "
                         "profiles/traffic.json, e.g. dkdv@3")
    ap.add_argument("--mfma-key", nargs="+", default=None,
                    help="with --summarize: record the MFMA busy fraction, clock and executed rate of "
                         "KERNEL@WORKLOAD in profiles/mfma.json, e.g. dkdv@3 fwd@3")
    return ap.parse_args()


def src_hash(files):
    """Hash of a kernel's source files and of the compiler flags they are built with
    (a flag can change the machine code as much as an edit)."""
    from block_diffusion_attention_amd import build as _build
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "block_diffusion_attention_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
        if f.endswith(".hip"):
            h.update(" ".join(_build.HIP_FLAGS + _build.HIP_FILE_FLAGS.get(f, [])).encode())
    return h.hexdigest()[:16]


KERNEL_SOURCES = {
    "fwd": ["attn_fwd.hip", "attn_fwd_vt.hip", "kcommon.h", "bd_records.h", "kernels.h"],
    "transpose_v": ["attn_fwd_vt.hip", "kcommon.h", "kernels.h"],
    "dkdv": ["attn_bwd.hip", "kcommon.h", "bd_records.h", "kernels.h"],
    "dkdv_masked": ["attn_bwd.hip", "kcommon.h", "bd_records.h", "kernels.h"],
    "dq": ["attn_dq.hip", "kcommon.h", "bd_records.h", "kernels.h"],
    "bwd_pre": ["attn_bwd.hip", "kcommon.h", "bd_records.h", "kernels.h"],
    "merge": ["attn_fwd.hip", "kcommon.h", "bd_records.h", "kernels.h"],
    "aec_entropy": ["aec.hip", "aec.h"],
    "aec_grad": ["aec.hip", "aec.h"],
}


def mfma_from_profiles(kernel, workload):
    """MFMA busy fraction, clock and executed rate of a kernel from rocprofv3 counters
    (profiles/mfma.json), only if its source has not changed since they were taken."""
    try:
        with open(os.path.join(ROOT, "profiles", "mfma.json")) as f:
            rec = json.load(f)[f"{kernel}@{workload}"]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("src_sha256") != src_hash(KERNEL_SOURCES[kernel]):
        return None
    return {k: rec[k] for k in ("mfma_busy", "clock_ghz", "executed_tflops", "profiled_us") if k in rec}


def traffic_from_profiles(kernel, workload):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/traffic.json),
    only if the kernel source has not changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)[f"{kernel}@{workload}"]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("src_sha256") != src_hash(KERNEL_SOURCES[kernel]):
        return None
    return rec.get("bytes_per_launch")


def useful_flop(D, Hq, pairs, backward):
    """Useful FLOPs of one step: 4*D per visible (query row, key) pair and query head
    for the forward (S = Q K^T, then P V), and 10*D more for the backward (S
    recomputed, dP = dO V^T, dV = P^T dO, dK = dS^T Q, dQ = dS K)."""
    return (4.0 + (10.0 if backward else 0.0)) * D * Hq * pairs


def pass_rates(avg_ms, fwd_names, bwd_names, D, Hq, pairs, peak):
    """Useful rate of each pass on its own: the forward's 4*D and the backward's 10*D
    FLOP per visible pair and query head, over the summed average durations of that
    pass's kernels (bwd_names None: forward only)."""
    fwd_ms = sum(avg_ms[n] for n in fwd_names)
    passes = {"fwd": {"ms": round(fwd_ms, 4),
                      "useful_tflops": round(4.0 * D * Hq * pairs / (fwd_ms * 1e-3) / 1e12, 2)}}
    if bwd_names is not None:
        bwd_ms = sum(avg_ms[n] for n in bwd_names)
        passes["bwd"] = {"ms": round(bwd_ms, 4),
                         "useful_tflops": round(10.0 * D * Hq * pairs / (bwd_ms * 1e-3) / 1e12, 2)}
    for p_ in passes.values():
        p_["pct_of_peak"] = round(100.0 * p_["useful_tflops"] / peak, 2)
    return passes


def kernel_work(k, dtype, D, Hq, Hkv, tq, tk, pairs):
    """Algorithmic work per launch of each kernel, as (bound, FLOPs or bytes).

    MFMA kernels count the products they execute per visible pair and query head
    (forward 4*D; dK/dV 8*D: S, dP, dV, dK; dQ 6*D: S, dP, dQ). The serving steps'
    forward is priced in the bytes it must read (Q, K, V once each); its O and LSE
    leave through the split partials and the merge."""
    esz = 2 if dtype == "bf16" else 4
    q_bytes = tq * Hq * D * esz
    kv_bytes = tk * Hkv * D * esz
    algo = {
        "fwd": ("mfma", 4.0 * D * Hq * pairs),
        "dkdv": ("mfma", 8.0 * D * Hq * pairs),
        "dq": ("mfma", 6.0 * D * Hq * pairs),
        "bwd_pre": ("hbm", 2.0 * q_bytes + 3.0 * tq * Hq * 4),
        "merge": ("hbm", q_bytes + tq * Hq * 4),
        "transpose_v": ("hbm", 2.0 * kv_bytes),
    }
    if k in FWD_ONLY:   # the serving steps are bandwidth-bound: their forward is priced in bytes
        algo["fwd"] = ("hbm", float(q_bytes + 2 * kv_bytes))
    algo["dkdv_masked"] = algo["dkdv"]
    return algo


def step_bytes(dtype, D, Hq, Hkv, tq, tk):
    """Compulsory HBM bytes of one forward call: Q, K and V read once, O and LSE
    written once (9,048,064 B for the single-request denoising step)."""
    esz = 2 if dtype == "bf16" else 4
    return 2 * tq * Hq * D * esz + 2 * tk * Hkv * D * esz + tq * Hq * 4


def roofline(avg_ms, algo, peak, k):
    """Roofline object of the dominant kernel (largest mean duration): its algorithmic
    work per launch over its mean launch duration, against the bf16 MFMA or HBM peak."""
    dom = max(avg_ms, key=lambda n: avg_ms[n])
    bound, work = algo[dom]
    dur_s = avg_ms[dom] * 1e-3
    if bound == "mfma":
        achieved = work / dur_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4),
                # the products the kernel itself executes, which for the two backward
                # kernels (8*D and 6*D per pair) sum to more than the pass's useful 10*D
                "work_kind": "executed MFMA FLOPs of this kernel"}
    else:
        achieved = work / dur_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4),
                "work_kind": "compulsory bytes of this kernel"}
    roof["kernel"] = dom
    roof["work_per_launch"] = work
    roof["avg_launch_ms"] = round(avg_ms[dom], 4)
    roof["traffic"] = traffic_from_profiles(dom, k)
    return roof


KERNEL_SYMBOLS = {"fwd": "fwd_", "merge": "merge_kernel", "bwd_pre": "bwd_pre_kernel",
                  "dkdv": "dkdv_bf16_kernel", "dq": "dq_bf16_kernel", "transpose_v": "transpose_v_kernel",
                  "aec_entropy": "aec_entropy_kernel", "aec_grad": "aec_grad_kernel"}
COPY_SYMBOL = "MulFunctor"


def _read_csvs(roots, suffix):
    import csv
    rows = []
    for root in roots:
        for dp, _dn, fn in os.walk(root):
            for f in fn:
                if f.endswith(suffix):
                    with open(os.path.join(dp, f), newline="") as fh:
                        rows.extend(csv.DictReader(fh))
    return rows


def _short(name):
    """Kernel name without namespaces, return type and argument list."""
    name = name.replace("(anonymous namespace)::", "").replace("void ", "")
    depth, out = 0, []
    for ch in name:          # drop the argument list (the first top-level parenthesis)
        if ch == "(" and depth == 0:
            break
        depth += ch == "<"
        depth -= ch == ">"
        out.append(ch)
    return "".join(out)[:90]


def summarize(args):
    """Text summary of rocprofv3 CSV output: kernel stats and, when present, the
    per-dispatch FETCH_SIZE / WRITE_SIZE counters scaled by a plain copy kernel."""
    import collections
    roots = args.summarize
    lines = ["# rocprofv3 summary of " + ", ".join(os.path.basename(os.path.normpath(r)) for r in roots), "",
             f"command: {args.command}" if args.command else "command: (not given)", ""]
    stats = _read_csvs(roots, "kernel_stats.csv")
    if stats:
        lines += ["## kernel stats (rocprofv3 --kernel-trace --stats)", "",
                  "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
        for r in sorted(stats, key=lambda r: -float(r.get("TotalDurationNs", 0))):
            short = _short(r["Name"])
            lines.append(f"| {short} | {r['Calls']} | {float(r['AverageNs'])/1e3:.2f} | "
                         f"{float(r['MinNs'])/1e3:.2f} | {float(r['MaxNs'])/1e3:.2f} | "
                         f"{float(r['Percentage']):.1f} |")
        lines.append("")
    pmc = _read_csvs(roots, "counter_collection.csv")
    lines += _summarize_sq(pmc)
    pmc = [r for r in pmc if r["Counter_Name"] in ("FETCH_SIZE", "WRITE_SIZE")]
    traffic = {}
    if pmc:
        per = collections.defaultdict(list)     # (kernel, counter) -> values per dispatch
        for r in pmc:
            per[(r["Kernel_Name"], r["Counter_Name"])].append(float(r["Counter_Value"]))
        copy_bytes = args.copy_probe_mb * 2**20 if args.copy_probe_mb else None
        scale = {}
        for (kn, cn), vals in per.items():
            if COPY_SYMBOL in kn and copy_bytes:
                # the largest elementwise dispatch is the copy probe (fp32 in, fp32 out)
                scale[cn] = copy_bytes / (max(vals) * 1024.0)
        lines += ["## HBM counters per dispatch (KiB as read; bytes after scaling)", "",
                  f"copy probe: {args.copy_probe_mb} MiB read + written; scale factors "
                  + ", ".join(f"{k}={v:.4f}" for k, v in sorted(scale.items())), "",
                  "| kernel | counter | dispatches | mean KiB | scaled MB |", "|---|---|---|---|---|"]
        for (kn, cn), vals in sorted(per.items()):
            mean = sum(vals) / len(vals)
            sc = scale.get(cn)
            mb = f"{mean * 1024.0 * sc / 1e6:.2f}" if sc else "-"
            short = _short(kn)
            lines.append(f"| {short} | {cn} | {len(vals)} | {mean:.1f} | {mb} |")
            for key, sym in KERNEL_SYMBOLS.items():
                if sym in kn and sc:
                    traffic.setdefault(key, 0.0)
                    traffic[key] += mean * 1024.0 * sc
        lines.append("")
    text = "\n".join(lines)
    if args.summary_out:
        with open(args.summary_out, "w") as f:
            f.write(text + "\n")
    print(text)
    if args.mfma_key and MFMA_STATS:
        path = os.path.join(ROOT, "profiles", "mfma.json")
        try:
            with open(path) as f:
                rec = json.load(f)
        except (OSError, ValueError):
            rec = {}
        for key in args.mfma_key:
            kern, _wl = key.split("@")
            hits = [v for kn, v in MFMA_STATS.items() if KERNEL_SYMBOLS[kern] in kn]
            if hits:
                rec[key] = dict(hits[0], src_sha256=src_hash(KERNEL_SOURCES[kern]), command=args.command)
                print(f"mfma {key}: {rec[key]}")
        with open(path, "w") as f:
            json.dump(rec, f, indent=1, sort_keys=True)
    if args.traffic_key and traffic:
        kern, wl = args.traffic_key.split("@")
        path = os.path.join(ROOT, "profiles", "traffic.json")
        try:
            with open(path) as f:
                rec = json.load(f)
        except (OSError, ValueError):
            rec = {}
        rec[args.traffic_key] = {"bytes_per_launch": traffic[kern], "src_sha256": src_hash(KERNEL_SOURCES[kern]),
                                 "command": args.command}
        with open(path, "w") as f:
            json.dump(rec, f, indent=1, sort_keys=True)
        print(f"traffic {args.traffic_key}: {traffic[kern] / 1e6:.2f} MB per launch -> {path}")


SIMDS = 256 * 4                # MI355X: 256 compute units x 4 SIMDs
MFMA_STATS = {}                # short kernel name -> MFMA counters of the last summary
XCDS = 8


def _summarize_sq(rows):
    """MFMA utilisation and LDS counters per kernel from rocprofv3 --pmc rows.

    MFMA busy fraction = sum over SIMDs of SQ_VALU_MFMA_BUSY_CYCLES / (GPU cycles x SIMDs),
    with the GPU cycles of one XCD (GRBM_GUI_ACTIVE summed over the 8 XCDs / 8); executed
    MFMA FLOPs = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512; the clock is those cycles over the
    dispatch's own start/end timestamps."""
    import collections
    per = collections.defaultdict(dict)          # (kernel, dispatch) -> counter -> value
    for r in rows:
        if r["Counter_Name"] in ("FETCH_SIZE", "WRITE_SIZE") or "bdattn" not in r["Kernel_Name"]:
            continue
        d = per[(_short(r["Kernel_Name"]), r["Dispatch_Id"])]
        d[r["Counter_Name"]] = float(r["Counter_Value"])
        d["dur_s"] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
    if not per:
        return []
    by_kernel = collections.defaultdict(list)
    for (kn, _), d in per.items():
        by_kernel[kn].append(d)
    out = []
    mfma = {"SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_INSTS_VALU_MFMA_MOPS_BF16"}
    if any(mfma <= set(d) for ds in by_kernel.values() for d in ds):
        out += ["## MFMA utilisation (SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE, SQ_INSTS_VALU_MFMA_MOPS_BF16)", "",
                "| kernel | dispatches | mean us | clock GHz | MFMA busy % | executed TFLOP | executed TFLOP/s | % of 2516.6 TFLOP/s |",
                "|---|---|---|---|---|---|---|---|"]
        for kn, ds in sorted(by_kernel.items()):
            ds = [d for d in ds if mfma <= set(d) and d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] > 0]
            if not ds:
                continue
            dur = sum(d["dur_s"] for d in ds) / len(ds)
            cyc = sum(d["GRBM_GUI_ACTIVE"] for d in ds) / len(ds) / XCDS
            busy = sum(d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in ds) / len(ds)
            flop = sum(d["SQ_INSTS_VALU_MFMA_MOPS_BF16"] for d in ds) / len(ds) * 512.0
            MFMA_STATS[kn] = {"mfma_busy": round(busy / (cyc * SIMDS), 4), "clock_ghz": round(cyc / dur / 1e9, 3),
                              "executed_tflops": round(flop / dur / 1e12, 1), "profiled_us": round(dur * 1e6, 1)}
            out.append(f"| {kn} | {len(ds)} | {dur * 1e6:.1f} | {cyc / dur / 1e9:.2f} | {100 * busy / (cyc * SIMDS):.1f} | "
                       f"{flop / 1e12:.4f} | {flop / dur / 1e12:.0f} | {100 * flop / dur / 1e12 / PEAK_BF16_TFLOPS:.1f} |")
        out.append("")
    stall = ["SQ_WAVE_CYCLES", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VALU",
             "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_SCA", "SQ_ACTIVE_INST_VMEM"]
    if any(set(stall) <= set(d) for ds in by_kernel.values() for d in ds):
        out += ["## Where the waves' time goes (% of SQ_WAVE_CYCLES; quad-cycle counters, per wave)", "",
                "| kernel | waiting for anything | waiting to issue | active (any) | active VALU/MFMA | active LDS | "
                "active scalar | active vector memory |", "|---|---|---|---|---|---|---|---|"]
        for kn, ds in sorted(by_kernel.items()):
            ds = [d for d in ds if set(stall) <= set(d)]
            if not ds:
                continue
            m = {c: sum(d[c] for d in ds) / len(ds) for c in stall}
            wc = max(m["SQ_WAVE_CYCLES"], 1.0)
            out.append(f"| {kn} | " + " | ".join(f"{100 * m[c] / wc:.1f}" for c in stall[1:]) + " |")
        out.append("")
    lds = ["SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_INSTS_LDS", "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_VALU",
           "SQ_INSTS_VALU", "SQ_WAVE_CYCLES"]
    if any(set(lds) <= set(d) for ds in by_kernel.values() for d in ds):
        out += ["## LDS and VALU counters (SQ_WAVE_CYCLES, SQ_WAIT_INST_LDS, SQ_ACTIVE_INST_VALU in quad-cycles)", "",
                "| kernel | LDS bank-conflict cycles | LDS instructions | waiting for LDS issue, % of wave time | "
                "VALU active, % of wave time | VALU instructions |", "|---|---|---|---|---|---|"]
        for kn, ds in sorted(by_kernel.items()):
            ds = [d for d in ds if set(lds) <= set(d)]
            if not ds:
                continue
            m = {c: sum(d[c] for d in ds) / len(ds) for c in lds}
            wc = max(m["SQ_WAVE_CYCLES"], 1.0)
            out.append(f"| {kn} | {m['SQ_LDS_BANK_CONFLICT']:.0f} | {m['SQ_INSTS_LDS']:.3e} | "
                       f"{100 * m['SQ_WAIT_INST_LDS'] / wc:.1f} | {100 * m['SQ_ACTIVE_INST_VALU'] / wc:.1f} | "
                       f"{m['SQ_INSTS_VALU']:.3e} |")
        out.append("")
    return out


COLD_SETS = 48      # distinct input sets a cold serving-step run rotates over


def cold_serving(plan, q, k, v, o, lse, fwd_names, algo, steps, step_b):
    """The serving step with its inputs out of cache: the forward rotates over
    COLD_SETS distinct copies of Q, K, V (and outputs), several hundred MB in all,
    more than the last-level cache holds, so every call reads its Q/K/V from HBM.
    Timed like the hot loop: events around the whole run and around each kernel."""
    import numpy as np
    import torch

    from block_diffusion_attention_amd import binding as b
    sets = [(q.clone(), k.clone(), v.clone(), torch.empty_like(o), torch.empty_like(lse)) for _ in range(COLD_SETS)]
    n = max(steps, 2 * COLD_SETS)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fwd_names) + 1)] for _ in range(n)]
    for e in [x for row in ev for x in row]:
        e.record()
    for st in sets:                       # one untimed pass: every set written and resident in HBM
        b.fwd(plan, *st[:3], o=st[3], lse=st[4])
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for i in range(n):
        st = sets[i % COLD_SETS]
        b.fwd(plan, *st[:3], o=st[3], lse=st[4], events=ev[i])
    c1.record()
    torch.cuda.synchronize()
    ms_step = c0.elapsed_time(c1) / n
    kern = {name: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(n)]))
            for j, name in enumerate(fwd_names)}
    per_set = sum(t.numel() * t.element_size() for t in sets[0])
    fwd_bytes = algo["fwd"][1]
    return {"buffer_sets": COLD_SETS, "bytes_rotated": per_set * COLD_SETS, "steps": n,
            "ms_per_step": round(ms_step, 4), "kernels_ms": {name: round(t, 4) for name, t in kern.items()},
            "fwd_GBps": round(fwd_bytes / (kern["fwd"] * 1e-3) / 1e9, 1),
            "step_GBps": round(step_b / (ms_step * 1e-3) / 1e9, 1)}


def cpu_model():
    """The host CPU's model name (first processor in /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl, budget_s):
    """The oracle (fp64 numpy) on a bounded sample of the workload: whole
    (segment, kv head) slices, forward + backward, until the budget is spent."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from block_diffusion_attention_amd import workloads as W
    from oracle import bd_oracle as orc

    m = wl.meta
    G = m.num_q_heads // m.num_kv_heads
    order = [(s, g) for s in range(m.num_segments) for g in range(m.num_kv_heads)]
    rng = np.random.default_rng(0)
    rng.shuffle(order)
    done, flops, t_total = [], 0.0, 0.0
    backward = wl.do is not None and wl.passes != "fwd"
    for s, g in order:
        sub = W.kv_group_slice(W.segment_slice(wl, s), g)
        t0 = time.perf_counter()
        orc.attention_fwd(sub.q, sub.k, sub.v, sub.meta)
        if backward:
            orc.attention_bwd(sub.q, sub.k, sub.v, sub.do, sub.meta)
        t_total += time.perf_counter() - t0
        pairs = orc.visible_pairs(sub.meta)
        flops += (14.0 if backward else 4.0) * m.head_dim * G * pairs
        done.append((s, g))
        if t_total >= budget_s:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info() if p.get("internal_api") in
                   ("openblas", "mkl", "blis")] or [1])
    frac = len(done) / len(order)
    return {
        "value": flops / t_total / 1e12,
        "unit": "TFLOP/s",
        "cores": int(threads),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{len(done)} of {len(order)} (segment, kv head) slices ({frac:.1%} of the work), "
                  f"{'fwd+bwd' if backward else 'fwd'}, fp64 numpy, {t_total:.1f} s",
        "seconds": t_total,
    }


def pack_bench(args):
    """Host packer on a synthetic replay batch: 256 responses, contexts of 8..128
    blocks of 32 behind a prompt that ends U[0, 32) tokens into a block, 4..16
    captured denoising steps per block, 1..32 supervised positions and 0..7
    resident pages per state, cost weights (1, 1, 4), 8 data-parallel groups."""
    import numpy as np

    from block_diffusion_attention_amd import binding as b

    rng = np.random.default_rng(args.seed if args.seed is not None else 11)
    B, R, G = 32, 256, 8
    nb = rng.integers(8, 129, size=R)
    off = rng.integers(0, B, size=R)
    clean = nb * B - off
    steps = rng.integers(4, 17, size=int(nb.sum()))
    resp = np.repeat(np.repeat(np.arange(R), nb), steps)
    block = np.repeat(np.concatenate([np.arange(1, n + 1) for n in nb]), steps)
    step = np.concatenate([np.arange(k) for k in steps])
    N = len(resp)
    sup = rng.integers(1, B + 1, size=N)
    pages = rng.integers(0, 8, size=N)
    args_ = (clean, resp, block, step, B, G)
    kw = dict(block_offset=off, state_supervised=sup, state_pages=pages, w_tokens=1, w_supervised=1, w_pages=4)
    times = []
    for _ in range(args.warmup + args.steps):
        t0 = time.perf_counter()
        p = b.pack(*args_, **kw)
        times.append(time.perf_counter() - t0)
    t = float(np.median(times[args.warmup:]))
    loads = p["group_cost"].astype(np.float64)
    out = {
        "metric": "host packer: captured states packed into replay rows and assigned per second",
        "value": round(N / t, 1), "unit": "states/s", "higher_is_better": True,
        "steps": args.steps, "warmup": args.warmup, "ms_per_call": round(t * 1e3, 3),
        "data": "synthetic",
        "config": {"workload": " ".join(pack_bench.__doc__.split(":", 1)[1].split()),
                   "states": N, "rows": int(p["n_rows"]), "groups": G,
                   "note": "wall time includes the Python argument marshalling of the binding"},
        "balance": {"max_over_mean_group_cost": round(float(loads.max() / loads.mean()), 5)},
    }
    if not args.no_cpu:
        from oracle import bd_pack_oracle as po
        states = [{"resp": int(r), "block": int(bl), "step": int(k), "supervised": int(su), "pages": int(pg)}
                  for r, bl, k, su, pg in zip(resp, block, step, sup, pages)]
        t0 = time.perf_counter()
        po.pack(clean.tolist(), off.tolist(), states, B, G, 1, 1, 4)
        to = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(N / to, 1), "unit": "states/s", "cores": 1,
                               "cpu_model": cpu_model(), "kind": "oracle",
                               "sample": f"the whole batch ({N} states), pure Python, {to:.2f} s"}
    print(json.dumps(out), flush=True)


def aec_bench(args):
    """Normalized entropy + AEC loss over the logits of the canvas positions of a
    replay batch: 16 states of 32 positions, a 151,936-entry vocabulary, bf16
    logits N(0, tau^2) with tau ~ U[0.5, 6] per row, seed 7; forward and the
    gradient with respect to the logits."""
    import ctypes

    import numpy as np
    import torch

    from block_diffusion_attention_amd import binding as b
    from block_diffusion_attention_amd import workloads as W

    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = W.aec_workload(7 if args.seed is None else args.seed)
    N, V = wl.logits.shape[0], wl.vocab
    logits = torch.from_numpy(wl.logits).to(dev).to(torch.bfloat16).contiguous()
    t = lambda x, ty: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(ty)
    kw = dict(unresolved=t(wl.unresolved, torch.uint8), state_rows=t(wl.state_rows, torch.int32),
              pair_next=t(wl.pair_next, torch.int32), pair_h_source=t(wl.pair_h_source, torch.float32),
              pair_weight=t(wl.pair_weight, torch.float32), rho=wl.rho, gate_max=wl.gate_max)
    d = b.aec_desc(N, V, logits.shape[1], "bf16", len(wl.state_rows) - 1, len(wl.pair_next), wl.rho, wl.gate_max)
    nk = b.aec_kernels(d)
    names = ["aec_entropy", "aec_reduce"][:nk]
    ws = torch.empty(max(16, b.aec_workspace_bytes(d)), dtype=torch.uint8, device=dev)
    backward = not args.fwd_only
    grad = torch.ones(1, dtype=torch.float32, device=dev)
    dlogits = torch.empty_like(logits)

    def step(evf=None, evb=None):
        lse, hbar, hs, _loss = b.aec_fwd(logits, V, events=evf, ws=ws, **kw)
        if backward:
            args_b = [ctypes.byref(d), b._ptr(logits), b._ptr(kw["unresolved"]), b._ptr(kw["state_rows"]),
                      b._ptr(kw["pair_next"]), b._ptr(kw["pair_h_source"]), b._ptr(kw["pair_weight"]),
                      b._ptr(lse), b._ptr(hbar), b._ptr(hs), b._ptr(grad), b._ptr(dlogits), b._ptr(ws),
                      b._stream(dev)]
            if evb is None:
                b._check(b._lib.bd_aec_bwd(*args_b))
            else:
                arr, n = b._events_arg(evb)
                b._check(b._lib.bd_aec_bwd_timed(*args_b, arr, n))

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nk + 1)] for _ in range(K)]
    evb = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)] if backward else [None] * K
    for e in [x for row in ev for x in row] + [x for row in evb if row for x in row]:
        e.record()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(K):
        step(ev[i], evb[i])
    end.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(end) / K
    avg = {n: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(K)])) for j, n in enumerate(names)}
    if backward:
        for j, n in enumerate(["aec_grad_coef", "aec_grad"]):
            avg[n] = float(np.mean([evb[i][j].elapsed_time(evb[i][j + 1]) for i in range(K)]))
    logit_bytes = float(N) * V * 2
    # rows the gradient reaches (it reads their logits; it writes every row): the
    # unresolved rows of states named by a kept pair with an open hinge
    hs = b.aec_fwd(logits, V, ws=ws, **kw)[2].cpu().numpy()
    reached = np.zeros(N, bool)
    for n, h_src in zip(wl.pair_next, wl.pair_h_source):
        if 0 <= n < len(hs) and np.isfinite(hs[n]) and np.isfinite(h_src) and h_src <= wl.gate_max \
                and hs[n] > (1.0 - wl.rho) * h_src:
            lo, hi = wl.state_rows[n], wl.state_rows[n + 1]
            reached[lo:hi] |= wl.unresolved[lo:hi] != 0
    algo = {"aec_entropy": logit_bytes + 8.0 * N + N,     # logits, flags in; lse, hbar out
            "aec_grad": logit_bytes * (1.0 + reached.mean()) + 12.0 * N}   # reached rows in, all rows out
    dom = max((n for n in avg if n in algo), key=lambda n: avg[n])
    work = algo[dom]
    achieved = work / (avg[dom] * 1e-3) / 1e9
    out = {
        "metric": "normalized-entropy + AEC loss (forward and gradient) over vocabulary logits: logit bytes "
                  "per second",
        "value": round(logit_bytes / (ms_step * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1, "steps": K,
        "passes": "fwd+bwd" if backward else "fwd",
        "warmup": args.warmup, "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": " ".join(aec_bench.__doc__.split()), "rows": N, "vocab": V,
                   "states": len(wl.state_rows) - 1, "pairs": len(wl.pair_next),
                   "rows_reached_by_the_gradient": int(reached.sum())},
        "kernels_ms": {n: round(x, 4) for n, x in avg.items()},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBS, 4), "kernel": dom, "work_per_launch": work,
                     "avg_launch_ms": round(avg[dom], 4), "traffic": traffic_from_profiles(dom, "aec")},
    }
    if args.copy_probe_mb:
        n = args.copy_probe_mb * 2**20 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu:
        from oracle import bd_aec_oracle as ao
        rows = 64
        t0 = time.perf_counter()
        ao.lse_and_entropy(wl.logits[:rows, :V])
        if backward:      # the gradient's per-row work: softmax, log-probabilities, one product
            ao.aec_backward(wl.logits[:rows, :V], wl.unresolved[:rows], wl.state_rows[:rows // 32 + 1],
                            [], [], [], wl.rho, wl.gate_max)
        to = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(rows * V * 2 / to / 1e9, 3), "unit": "GB/s", "cores": 1,
                               "cpu_model": cpu_model(), "kind": "oracle", "sample": f"{rows} of {N} rows (normalizer and entropy"
                                                           f"{', then the gradient' if backward else ''}), "
                                                           f"fp64 numpy, {to:.2f} s"}
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.summarize:
        summarize(args)
        return
    if args.pack:
        pack_bench(args)
        return
    if args.aec:
        aec_bench(args)
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from block_diffusion_attention_amd import binding as b
    from block_diffusion_attention_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    k = args.workload
    wl = W.make_config(k, seed=args.seed)
    m = wl.meta
    backward = wl.do is not None and not args.fwd_only and k not in FWD_ONLY
    t_plan0 = time.perf_counter()
    plan = b.Plan(m, args.flags)
    t_plan = time.perf_counter() - t_plan0
    plan.upload(dev)
    dt = plan.dtype
    to = lambda x: torch.from_numpy(x).to(dev).to(dt).contiguous()
    q, kk, v = to(wl.q), to(wl.k), to(wl.v)
    do = to(wl.do) if backward else None
    o = torch.empty_like(q)
    lse = torch.empty((plan.tq, m.num_q_heads), dtype=torch.float32, device=dev)
    dq, dk, dv = (torch.empty_like(q), torch.empty_like(kk), torch.empty_like(v)) if backward else (None,) * 3

    nf = plan.kernels(False)
    fwd_names = plan.kernel_names(False)
    bwd_names = plan.kernel_names(True)

    def step(evf=None, evb=None):
        b.fwd(plan, q, kk, v, o, lse, events=evf)
        if backward:
            b.bwd(plan, q, kk, v, o, lse, do, dq, dk, dv, events=evb)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    evf = [[torch.cuda.Event(enable_timing=True) for _ in range(nf + 1)] for _ in range(K)]
    evb = ([[torch.cuda.Event(enable_timing=True) for _ in range(len(bwd_names) + 1)] for _ in range(K)]
           if backward else [None] * K)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for e in [x for row in evf for x in row] + [x for row in evb if row for x in row]:
        e.record()          # creates the HIP events before the timed region
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record()
    for i in range(K):
        step(evf[i], evb[i])
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = start.elapsed_time(end)
    ms_step = ms_total / K
    ms_eager = ms_step
    if args.graph:
        # the same step captured once and replayed (stream-ordered, no host launches)
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()                          # warm the side stream before capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(K):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        ms_step = g0.elapsed_time(g1) / K

    per_kernel = {}
    for i in range(K):
        for j, n in enumerate(fwd_names):
            per_kernel.setdefault(n, []).append(evf[i][j].elapsed_time(evf[i][j + 1]))
        if backward:
            for j, n in enumerate(bwd_names):
                per_kernel.setdefault(n, []).append(evb[i][j].elapsed_time(evb[i][j + 1]))
    avg_ms = {n: float(np.mean(v_)) for n, v_ in per_kernel.items()}
    # spread over the timed steps: p10 / median / p90 of each kernel and of the
    # step's kernels from the first launch to the last
    pct = lambda v_: [round(float(x), 4) for x in np.percentile(v_, [10, 50, 90])]
    spread = {n: pct(v_) for n, v_ in per_kernel.items()}
    step_span = [evf[i][0].elapsed_time(evb[i][-1] if backward else evf[i][-1]) for i in range(K)]
    spread["step (first to last kernel)"] = pct(step_span)

    D, Hq = m.head_dim, m.num_q_heads
    pairs = plan.visible_pairs
    useful = useful_flop(D, Hq, pairs, backward)
    value = useful / (ms_step * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if m.dtype == "bf16" else PEAK_FP32_TFLOPS
    passes = pass_rates(avg_ms, fwd_names, bwd_names if backward else None, D, Hq, pairs, peak)
    algo = kernel_work(k, m.dtype, D, Hq, m.num_kv_heads, plan.tq, plan.tk, pairs)
    roof = roofline(avg_ms, algo, peak, k)
    # rocprofv3 counters of the kernels (profiles/mfma.json; null when stale or absent)
    counters = {n: mfma_from_profiles(n, k) for n in avg_ms if algo.get(n, ("",))[0] == "mfma"}

    serving = None
    if k in FWD_ONLY:   # the step's compulsory bytes over its time, hot and cold
        sb = step_bytes(m.dtype, D, Hq, m.num_kv_heads, plan.tq, plan.tk)
        serving = {"compulsory_bytes": sb, "GBps": round(sb / (ms_step * 1e-3) / 1e9, 1),
                   "pct_of_hbm": round(100.0 * sb / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)}
    cold = cold_serving(plan, q, kk, v, o, lse, fwd_names, algo, K, serving["compulsory_bytes"]) \
        if k in FWD_ONLY else None

    if args.copy_probe_mb:
        n = args.copy_probe_mb * 2**20 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.mul(src, 1.0, out=dst)        # one elementwise kernel: n*4 bytes read, n*4 written
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(wl, args.cpu_seconds)
        cpu.pop("seconds", None)

    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "pct_of_peak": round(100.0 * value / peak, 2),
        "per_pass": passes,
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": m.dtype,
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD_NAMES[k],
            "seed": k if args.seed is None else args.seed,
            "tq": plan.tq, "tk": plan.tk, "visible_pairs_per_head": pairs,
            "passes": "fwd+bwd" if backward else "fwd",
            "useful_flop_per_step": useful,
            "parallelism": "single GPU",
            "launch": "hip graph replay" if args.graph else "eager stream launches",
        },
        "eager_ms_per_step": round(ms_eager, 4),
        "kernels_ms": {n: round(t, 4) for n, t in avg_ms.items()},
        "kernels_ms_p10_p50_p90": spread,
        "plan_ms": round(t_plan * 1e3, 3),
        "wall_s": round(wall, 3),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if any(v is not None for v in counters.values()):
        out["mfma_counters"] = counters
    if serving is not None:
        out["step_bytes"] = serving
    if cold is not None:
        out["cold"] = cold
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
