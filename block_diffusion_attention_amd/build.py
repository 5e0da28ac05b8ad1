"""Builds libbdattn.so (gfx950) in-tree with hipcc; the planner is plain C++ (g++)."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libbdattn.so")
BUILD_DIR = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

HIP_SOURCES = ["attn_fwd.hip", "attn_fwd_vt.hip", "attn_bwd.hip", "attn_f32.hip", "aec.hip", "bd_attn_abi.hip"]
CXX_SOURCES = ["planner.cpp", "packer.cpp"]
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             # packed fp32 VALU instructions stay disabled for all device code
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Extra flags per source. attn_bwd.hip: MFMA results go to vector registers even
# in kernels that keep operands in accumulation registers (the dK/dV kernel holds
# its K/V fragments there); otherwise the scores come out in accumulation
# registers and every element costs an extra copy before the vector ALU sees it.
HIP_FILE_FLAGS = {"attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed: {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    """Compiles every source and links libbdattn.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = []
    for s in HIP_SOURCES:
        obj = os.path.join(BUILD_DIR, s.replace(".hip", ".o"))
        jobs.append(([HIPCC, *HIP_FLAGS, *HIP_FILE_FLAGS.get(s, []), "-c", os.path.join(CSRC, s), "-o", obj], obj))
    for s in CXX_SOURCES:
        obj = os.path.join(BUILD_DIR, s.replace(".cpp", ".o"))
        jobs.append((["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, s), "-o", obj], obj))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(lambda j: _run(j[0]), jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[j[1] for j in jobs], "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
