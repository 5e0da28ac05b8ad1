"""The AEC entry points on the CPU: argument validation and launch geometry
(no kernel is launched here)."""
import math

import pytest

b = pytest.importorskip("block_diffusion_attention_amd.binding")


def _d(**over):
    args = dict(num_rows=512, vocab=151936, row_stride=151936, dtype="bf16", num_states=16, num_pairs=12,
                rho=0.1, gate_max=math.inf)
    args.update(over)
    return b.aec_desc(**args)


@pytest.mark.parametrize("over,msg", [
    (dict(num_rows=0), "num_rows"),
    (dict(vocab=1), "vocab"),
    (dict(row_stride=151935), "row_stride"),
    (dict(vocab=50257, row_stride=50260), "row_stride"),      # bf16 rows need a multiple of 8
    (dict(num_states=-1), "num_states"),
    (dict(rho=1.5), "rho"),
    (dict(rho=float("nan")), "rho"),
    (dict(gate_max=float("nan")), "gate_max"),
])
def test_validation(over, msg):
    with pytest.raises(b.BdAttnError) as e:
        b.aec_workspace_bytes(_d(**over))
    assert e.value.status == b.EINVAL and msg in str(e.value)
    assert b.aec_kernels(_d(**over)) == 0


def test_geometry_and_workspace():
    # a long batch: the backward's state gradients (256-byte aligned) and row coefficients
    assert b.aec_workspace_bytes(_d(num_rows=4096)) == 256 + 4096 * 4 and b.aec_kernels(_d(num_rows=4096)) == 2
    # a short batch splits each row over several workgroups of >= 8192 logits:
    # the forward's partial triples dominate the workspace
    d = _d(num_rows=8)
    assert b.aec_kernels(d) == 2
    nsplit = b.aec_workspace_bytes(d) // (8 * 3 * 4)
    assert 2 <= nsplit <= 151936 // 8192
    # fp32 rows may have a stride that is a multiple of 4
    assert b.aec_workspace_bytes(_d(vocab=1002, row_stride=1004, dtype="fp32", num_rows=2)) > 0


def test_split_forward_requires_workspace_and_backward_always():
    import ctypes
    vp = ctypes.c_void_p
    d = _d(num_rows=8)
    st = b._lib.bd_aec_fwd(ctypes.byref(d), vp(16), vp(16), vp(16), vp(16), vp(16), vp(16),
                           vp(16), vp(16), vp(16), vp(16), vp(0), vp(0))
    assert st == b.EWORKSPACE
    d = _d(num_rows=4096)
    st = b._lib.bd_aec_bwd(ctypes.byref(d), vp(16), vp(16), vp(16), vp(16), vp(16), vp(16),
                           vp(16), vp(16), vp(16), vp(16), vp(16), vp(0), vp(0))
    assert st == b.EWORKSPACE
