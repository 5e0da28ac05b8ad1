"""The device-checked build (libbdattn_checked.so, from build.py --device-checks),
on the GPU.

* On clean plans its kernels reject no record and give outputs bit-identical to
  the normal build's (forward direct and split with its merge, with and without
  the transposed V copy; dQ; dK/dV, split with its merge and masked; fp32).
* Records planted out of range in the device copy of the work lists are counted
  and their workgroups skipped: a kv head equal to Hkv in a forward, dQ, split-part,
  merge and dK/dV merge record and in an fp32 dK/dV record, and an inverted chunk
  range in a dK/dV record. Each planted
  record is chosen (and asserted on the host) so that even a build without the
  checks would stay inside every tensor and workspace while following it.

The binding binds one library per process, so the checked library runs in a child
process; the parent computes the normal build's outputs and hands them over in a
temporary file.
"""
import os
import subprocess
import sys
import tempfile

import pytest
import torch

import device_check_cases as C

b = pytest.importorskip("block_diffusion_attention_amd.binding")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

pytestmark = pytest.mark.gpu

CHILD = r'''
import os, sys
sys.path.insert(0, ROOT); sys.path.insert(0, os.path.join(ROOT, "tests"))
import torch
from block_diffusion_attention_amd import binding as b
import device_check_cases as C
assert b.LIB_PATH == b.CHECKED_LIB_PATH, b.LIB_PATH
torch.cuda.set_device(0)
b.device_check_errors(reset=True)
for i, (name, make, flags) in enumerate(C.CASES):
    print(f"checked build: case {name}", flush=True)
    meta = make()
    plan, out = C.run_case(b, meta, C.flags_of(b, flags))
    ref = torch.load(os.path.join(TMP, f"case{i}.pt"), weights_only=True)
    for k, t in out.items():
        r = ref[k].to("cuda")
        assert t.shape == r.shape and t.dtype == r.dtype, (name, k)
        assert torch.equal(t.view(torch.uint8), r.view(torch.uint8)), f"{name}: {k} differs from the normal build"
    n = b.device_check_errors(reset=True)
    assert n == 0, f"{name}: {n} workgroups rejected a record of a clean plan"
    del plan, out, ref

for ci, secs in C.PLANTS:
    name, make, flags = C.CASES[ci]
    print(f"checked build: planted records {secs} in {name}", flush=True)
    meta = make()
    plan, _ = C.run_case(b, meta, C.flags_of(b, flags))
    blob, expect = C.plant(meta, plan, plan.host_blob(), secs)
    img = torch.tensor(blob, dtype=torch.int32).view(torch.uint8)
    plan.meta_dev[:img.numel()].copy_(img.to("cuda"))
    torch.cuda.synchronize()
    assert b.device_check_errors(reset=True) == 0
    C.run_case(b, meta, 0, plan=plan)
    n = b.device_check_errors(reset=True)
    assert n == expect, f"{name}: {n} workgroups rejected a record, expected {expect}"
    assert b.device_check_errors() == 0
    print(f"planted: ok ({n} workgroups rejected)", flush=True)
print("all planted: ok", flush=True)
'''


def _normal_outputs(tmp):
    for i, (name, make, flags) in enumerate(C.CASES):
        print(f"normal build: case {name}", flush=True)
        _, out = C.run_case(b, make(), C.flags_of(b, flags))
        torch.save({k: t.cpu() for k, t in out.items()}, os.path.join(tmp, f"case{i}.pt"))
        del out
    torch.cuda.empty_cache()


def test_checked_build_matches_normal_build_and_counts_planted_records():
    if not os.path.exists(b.CHECKED_LIB_PATH):
        pytest.fail("libbdattn_checked.so is missing: run build.py --device-checks (build() does)")
    with tempfile.TemporaryDirectory() as tmp:
        _normal_outputs(tmp)
        env = dict(os.environ, BDATTN_LIBRARY=b.CHECKED_LIB_PATH)
        r = subprocess.run([sys.executable, "-u", "-c", f"ROOT = {ROOT!r}\nTMP = {tmp!r}\n" + CHILD], env=env,
                           stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600)
    print(r.stdout[-4000:])
    assert r.returncode == 0, r.stdout[-4000:]
    assert "all planted: ok" in r.stdout
