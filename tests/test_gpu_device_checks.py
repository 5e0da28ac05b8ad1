"""Record-checking kernels (plans made with BD_ATTN_FLAG_DEBUG_CHECKS), on the GPU.

* On clean plans the checking kernels reject no record and give outputs bit-identical
  to the kernels without checks (forward direct and split with its merge, with and
  without the transposed V copy; dQ; dK/dV, split with its merge and masked; fp32).
* Records planted out of range in the device copy of the work lists are counted
  and their workgroups skipped: a kv head equal to Hkv in a forward, dQ, split-part,
  merge and dK/dV merge record and in an fp32 dK/dV record, and an inverted chunk
  range in a dK/dV record. Each planted record is chosen (and asserted on the host)
  so that even kernels without the checks would stay inside every tensor and
  workspace while following it.
"""
import pytest
import torch

import device_check_cases as C

b = pytest.importorskip("block_diffusion_attention_amd.binding")

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("case", range(len(C.CASES)))
def test_checking_kernels_match_and_reject_nothing_on_clean_plans(case):
    name, make, flags = C.CASES[case]
    _say(f"case device checks, clean: {name}")
    meta = make()
    f = C.flags_of(b, flags)
    b.device_check_errors(reset=True)
    _, ref = C.run_case(b, meta, f)
    assert b.device_check_errors() == 0
    _, out = C.run_case(b, meta, f | b.FLAG_DEBUG_CHECKS)
    for k, t in out.items():
        assert torch.equal(t.view(torch.uint8), ref[k].view(torch.uint8)), f"{name}: {k} differs"
    n = b.device_check_errors(reset=True)
    assert n == 0, f"{name}: {n} workgroups rejected a record of a clean plan"


@pytest.mark.parametrize("plant", range(len(C.PLANTS)))
def test_checking_kernels_count_and_skip_planted_records(plant):
    ci, secs = C.PLANTS[plant]
    name, make, flags = C.CASES[ci]
    _say(f"case device checks, planted {secs}: {name}")
    meta = make()
    plan, _ = C.run_case(b, meta, C.flags_of(b, flags) | b.FLAG_DEBUG_CHECKS)
    blob, expect = C.plant(meta, plan, plan.host_blob(), secs)
    img = torch.tensor(blob, dtype=torch.int32).view(torch.uint8)
    plan.meta_dev[:img.numel()].copy_(img.to(plan.meta_dev.device))
    torch.cuda.synchronize()
    assert b.device_check_errors(reset=True) == 0
    C.run_case(b, meta, 0, plan=plan)
    n = b.device_check_errors(reset=True)
    assert n == expect, f"{name}: {n} workgroups rejected a record, expected {expect}"
    assert b.device_check_errors() == 0
