"""GPU parity on inputs that drive the forward kernels through their
running-maximum rescale (alpha != 0): a late context tile, and separately each
canvas's own block, score >= 12 log2 units above the first visited tile.

Before the GPU runs, the same CPU replay as tests/test_rescale_inputs.py asserts
that the inputs do reach the rescale in the launch configuration under test.
Checked through the default forward, the transposed-V forward and a forced split
of 4 key tiles; O, LSE and the gradients against the oracle.
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


if not _gpu_available():
    pytest.skip("no GPU", allow_module_level=True)

from block_diffusion_attention_amd import binding as b  # noqa: E402
from gpu_common import run_gpu, run_oracle  # noqa: E402
from helpers import assert_close  # noqa: E402
from test_rescale_inputs import SPLIT_TILES, reached  # noqa: E402

LAUNCHES = {
    "default": (0, None),
    "fwd_vt": (b.FLAG_FWD_VT, None),
    "split4": (b.FLAG_FORCE_SPLIT | b.flag_split_tiles(SPLIT_TILES), SPLIT_TILES),
}


@pytest.mark.parametrize("launch", sorted(LAUNCHES))
@pytest.mark.parametrize("kind", ["context", "canvas"])
def test_rescale_parity(kind, launch):
    from rescale_common import stress_workload
    flags, tps = LAUNCHES[launch]
    frac, _, _ = reached(kind, tps)
    assert frac >= 0.6, f"the inputs no longer reach the rescale ({frac:.2f})"
    wl = stress_workload(kind)
    print(f"case rescale {kind} {launch} (rows reaching +12: {frac:.2f})", flush=True)
    sys.stdout.flush()
    gpu, plan = run_gpu(wl, flags=flags)
    if tps:
        assert "merge" in plan.kernel_names(False)
    ref = run_oracle(wl)
    for n in ("o", "dq", "dk", "dv"):
        assert_close(f"{wl.name}/{launch}:{n}", gpu[n], ref[n], "bf16")
    err = np.abs(gpu["lse"] - ref["lse"]).max()
    assert err <= 2e-3, f"lse max err {err}"
