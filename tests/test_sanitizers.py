"""The host code (planner, packer, C ABI) built with AddressSanitizer and
UndefinedBehaviorSanitizer (build.py --sanitize) runs the named workloads' plans
and the packer cleanly, and the sanitizer is live: a planted overflow (a caller
buffer smaller than the size it claims) is reported.

The full host suite runs against the same build with
  python block_diffusion_attention_amd/build.py --sanitize tests -m "not gpu"
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CLEAN = r'''
import ctypes, os, sys
sys.path.insert(0, ROOT)
import numpy as np
from block_diffusion_attention_amd import binding as b, workloads as W
assert b.LIB_PATH.endswith("_build/san/libbdattn.so"), b.LIB_PATH
maps = open("/proc/self/maps").read()
assert "libclang_rt.asan" in maps and "_build/san/libbdattn.so" in maps
rng = np.random.default_rng(5)
for k in (1, 2, 3, 4, 5, 6):
    p = b.Plan(W.config_meta(k, rng))
    blob = p.host_blob()
    assert blob[0] == 0x62646174
for _ in range(20):
    m = W.random_meta(rng, max_segments=4, max_blocks=9, block_sizes=(1, 3, 16, 32), max_canvases=4,
                      hq=8, hkv=2, d=128, dtype="bf16", offsets=True)
    b.Plan(m, int(rng.integers(0, 64)) & ~16)
res = b.pack([64, 96], [0, 0, 1, 1], [1, 2, 3, 1], [0, 0, 1, 1], 32, 2)
assert res["n_rows"] == 2
print("clean", flush=True)
os._exit(0)      # skip interpreter finalization (not instrumented, and not under test)
'''

PLANTED = r'''
import ctypes, sys
sys.path.insert(0, ROOT)
from block_diffusion_attention_amd import binding as b, workloads as W
p = b.Plan(W.config_meta(4, __import__("numpy").random.default_rng(4)))
buf = ctypes.create_string_buffer(1024)        # claims meta_bytes, holds 1 KiB (from malloc)
b._lib.bd_attn_plan_serialize(p.handle, ctypes.cast(buf, ctypes.c_void_p), p.meta_bytes)
print("not caught")
'''


def _san_build():
    if not os.path.exists("/opt/rocm/bin/hipcc") or shutil.which("g++") is None:
        pytest.skip("no hipcc")
    sys.path.insert(0, ROOT)
    from block_diffusion_attention_amd import build as bd
    bd.build(sanitize=True)
    return bd


def _run(bd, code):
    return subprocess.run([sys.executable, "-c", f"ROOT = {ROOT!r}\n" + code], env=bd.sanitizer_env(),
                          stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=300)


def test_host_code_under_sanitizers():
    bd = _san_build()
    r = _run(bd, CLEAN)
    assert r.returncode == 0 and "clean" in r.stdout, r.stderr[-3000:]
    r = _run(bd, PLANTED)
    assert r.returncode != 0 and "not caught" not in r.stdout
    assert "AddressSanitizer" in r.stderr and "overflow" in r.stderr, r.stderr[-3000:]
