"""bd_attn_fwd_noalloc: the forward whose workspace is the library's fixed
per-GPU array (for callers that cannot allocate device memory).

* CPU: a plan whose forward workspace exceeds the array is rejected with
  EWORKSPACE before any device call;
* GPU: through the C ABI, two calls in a row (the second with a smaller input)
  match bd_attn_fwd on the same inputs bit for bit, and both the parity bar
  against the oracle; a transposed-V plan (its V copy in the array) likewise.
"""
import ctypes

import numpy as np
import pytest

from block_diffusion_attention_amd import workloads as W

b = pytest.importorskip("block_diffusion_attention_amd.binding")


def test_noalloc_rejects_a_workspace_beyond_the_array():
    # a transposed-V plan over ~20k keys x 8 kv heads needs a 41 MB copy of V
    meta = W.Meta([20000], [19968], [[625]], 32, 32, 8, 128, "bf16")
    plan = b.Plan(meta, b.FLAG_FWD_VT)
    assert plan.ws_fwd_bytes > b.NOALLOC_WS_BYTES
    fake = ctypes.c_void_p(1 << 20)             # never dereferenced: the size check comes first
    st = b._lib.bd_attn_fwd_noalloc(plan.handle, fake, fake, fake, fake, fake, fake, None)
    assert st == b.EWORKSPACE
    assert "exceeds" in b._lib.bd_attn_last_error().decode()


def _gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.gpu
@pytest.mark.skipif(not _gpu(), reason="no GPU")
@pytest.mark.parametrize("flags", [0, b.FLAG_FWD_VT])
def test_noalloc_matches_fwd_on_two_calls(flags):
    import torch
    from gpu_common import nan_like, run_oracle, to_dev
    from helpers import assert_close

    big = W.make_config(2, with_do=False)                    # denoising step: split path, partials in ws
    rng = np.random.default_rng(77)
    small_meta = W.Meta([512], [512], [[9]], 32, 8, 2, 128, "bf16")
    small = W.random_workload(rng, small_meta, sigma=0.3, with_do=False)
    sizes = []
    for wl in (big, small):
        plan = b.Plan(wl.meta, flags).upload("cuda")
        assert plan.ws_fwd_bytes > 0, "the case must use the workspace"
        assert plan.ws_fwd_bytes <= b.NOALLOC_WS_BYTES
        sizes.append(plan.ws_fwd_bytes)
        q, k, v = (to_dev(x, plan.dtype) for x in (wl.q, wl.k, wl.v))
        print(f"case noalloc {wl.name} flags {flags} ws {plan.ws_fwd_bytes} B", flush=True)
        o_ref, lse_ref = b.fwd(plan, q, k, v, nan_like(q.shape, plan.dtype),
                               nan_like((plan.tq, wl.meta.num_q_heads), torch.float32))
        o, lse = b.fwd_noalloc(plan, q, k, v, nan_like(q.shape, plan.dtype),
                               nan_like((plan.tq, wl.meta.num_q_heads), torch.float32))
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
        ref = run_oracle(wl, backward=False)
        got = o.float().cpu().numpy().astype(np.float64)
        assert_close(f"noalloc {wl.name}:o", got, ref["o"], "bf16")
        assert np.abs(lse.cpu().numpy() - ref["lse"]).max() <= 2e-3
    assert sizes[1] < sizes[0], "the second call must be the smaller one"
