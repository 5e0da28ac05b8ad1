"""Builds libbdattn.so (gfx950) in-tree with hipcc; the planner is plain C++ (g++).
A debug build of the same sources with the host code sanitized: --sanitize."""
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

HIP_SOURCES = ["attn_fwd.hip", "attn_fwd_vt.hip", "attn_bwd.hip", "attn_dq.hip", "attn_f32.hip", "aec.hip",
               "bd_attn_abi.hip"]
CXX_SOURCES = ["planner.cpp", "packer.cpp"]
HIP_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
             # packed fp32 VALU instructions stay disabled for all device code
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# Extra flags per source. attn_bwd.hip and attn_dq.hip: MFMA results go to vector
# registers even in kernels that keep operands in accumulation registers (the
# dK/dV kernel holds its K/V fragments there); otherwise the scores come out in
# accumulation registers and every element costs an extra copy before the vector
# ALU sees it. Machine-scheduler strategies, each measured against the default on
# the packed replay: dK/dV 1.3 % faster with max-ilp, dQ 1.3 % faster with
# iterative-ilp (which slows dK/dV by 2.8 %, hence the separate files); the
# forward is within noise under every strategy and keeps the default.
HIP_FILE_FLAGS = {
    "attn_bwd.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-sched-strategy=max-ilp"],
    "attn_dq.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form", "-mllvm", "-amdgpu-sched-strategy=iterative-ilp"],
}
CXX_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra"]
# Sanitizer build of the host code (address + undefined behaviour), for the CPU
# test suite: every source goes through hipcc so one runtime (clang's) serves the
# whole library; the options apply to the host compilation only (GPU code is
# never built with a sanitizer). Load the result with the clang ASan runtime
# preloaded (see sanitizer_env()).
SAN_DIR = os.path.join(BUILD_DIR, "san")
SAN_LIB = os.path.join(SAN_DIR, "libbdattn.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


# A plain C99 program that uses the library through include/bd_attn.h alone (the
# C-ABI consumer test): strict C, ROCm headers as system headers, the in-tree
# library found next to the package at run time.
CONSUMER_SRC = os.path.join(ROOT, "tests", "c_consumer", "bd_attn_consumer.c")
CONSUMER_BIN = os.path.join(ROOT, "tests", "c_consumer", "bd_attn_consumer")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_consumer(cc: str = "gcc") -> str:
    """Compiles the C consumer against the in-tree libbdattn.so; returns its path
    (None for a copy of the package without the tests)."""
    if not os.path.exists(CONSUMER_SRC):
        return None
    tmp = CONSUMER_BIN + ".tmp"
    _run([cc, "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
          "-isystem", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), CONSUMER_SRC,
          "-o", tmp, "-L", HERE, "-lbdattn", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
          "-Wl,-rpath,$ORIGIN/../../block_diffusion_attention_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    os.replace(tmp, CONSUMER_BIN)
    return CONSUMER_BIN


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build step failed: {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, sanitize: bool = False) -> str:
    """Compiles every source and links libbdattn.so; returns its path.
    sanitize=True builds the host-sanitized copy under _build/san instead."""
    out_dir = SAN_DIR if sanitize else BUILD_DIR
    lib = SAN_LIB if sanitize else LIB
    os.makedirs(out_dir, exist_ok=True)
    san = SAN_FLAGS if sanitize else []
    jobs = []
    for s in HIP_SOURCES:
        obj = os.path.join(out_dir, s.replace(".hip", ".o"))
        jobs.append(([HIPCC, *HIP_FLAGS, *HIP_FILE_FLAGS.get(s, []), *san, "-c", os.path.join(CSRC, s),
                      "-o", obj], obj))
    for s in CXX_SOURCES:
        obj = os.path.join(out_dir, s.replace(".cpp", ".o"))
        if sanitize:
            cmd = [HIPCC, "-x", "c++", *CXX_FLAGS, *san, "-c", os.path.join(CSRC, s), "-o", obj]
        else:
            cmd = ["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, s), "-o", obj]
        jobs.append((cmd, obj))
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        outs = list(ex.map(lambda j: _run(j[0]), jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = lib + ".tmp"
    link_san = [*san, "-shared-libsan"] if sanitize else []
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *link_san, *[j[1] for j in jobs], "-o", tmp])
    os.replace(tmp, lib)
    if not sanitize:
        build_consumer()
    return lib


def sanitizer_env() -> dict:
    """Environment for a process that loads the sanitized library: the clang
    ASan runtime preloaded (the interpreter itself is not instrumented), leak
    checking off (the interpreter's own allocations), BDATTN_LIBRARY pointing at
    the sanitized build."""
    import glob
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        raise RuntimeError("clang ASan runtime not found under /opt/rocm/llvm")
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt[-1], ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", BDATTN_LIBRARY=SAN_LIB)
    return env


if __name__ == "__main__":
    # python build.py [-v] [--sanitize [pytest args...]]: --sanitize builds the
    # host-sanitized library and, given pytest arguments, runs them against it
    if "--sanitize" in sys.argv:
        rest = sys.argv[sys.argv.index("--sanitize") + 1:]
        print(build(verbose="-v" in sys.argv, sanitize=True))
        if rest:
            sys.exit(subprocess.call([sys.executable, "-m", "pytest", *rest], env=sanitizer_env(), cwd=ROOT))
    else:
        print(build(verbose="-v" in sys.argv))
