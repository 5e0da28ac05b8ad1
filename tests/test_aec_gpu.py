"""GPU parity of the normalized-entropy / AEC reduction against the fp64 oracle,
through the C ABI.

Tolerance (the fp32 bar, 1e-5): the kernel reads bf16 or fp32 logits and works
in fp32 throughout; per-thread running sums over ~V/2048 entries and fixed-order
merges keep the relative error of the partition sum near 1e-6, so the
normalized entropy (in [0, 1]) and the state means stay within 1e-5; the
log-normalizer is checked to 1e-5 relative to max(1, |lse|).
"""
import math
import sys

import numpy as np
import pytest

from block_diffusion_attention_amd import workloads as W

pytestmark = pytest.mark.gpu


def _gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


if not _gpu():
    pytest.skip("no GPU", allow_module_level=True)

import torch  # noqa: E402

from block_diffusion_attention_amd import binding as b  # noqa: E402
from oracle import bd_aec_oracle as ao  # noqa: E402

TOL = 1e-5


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(wl, **over):
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    dev = "cuda"
    logits = torch.from_numpy(wl.logits).to(dev).to(dt).contiguous()
    t = lambda x, ty: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(ty)
    args = dict(unresolved=t(wl.unresolved, torch.uint8), state_rows=t(wl.state_rows, torch.int32),
                pair_next=t(wl.pair_next, torch.int32), pair_h_source=t(wl.pair_h_source, torch.float32),
                pair_weight=t(wl.pair_weight, torch.float32), rho=wl.rho, gate_max=wl.gate_max)
    args.update(over)
    out = b.aec_fwd(logits, wl.vocab, **args)
    torch.cuda.synchronize()
    return [x.cpu().numpy().astype(np.float64) for x in out]


def _ref(wl, pair_next=None, h_source=None, gate_max=None):
    return ao.aec_forward(wl.logits[:, :wl.vocab], wl.unresolved, wl.state_rows,
                          wl.pair_next if pair_next is None else pair_next,
                          (wl.pair_h_source if h_source is None else h_source).astype(np.float64),
                          wl.pair_weight.astype(np.float64), wl.rho,
                          wl.gate_max if gate_max is None else gate_max)


def _check(wl, got, ref):
    lse, hbar, hs, loss = got
    rlse, rhbar, rhs, rloss = ref
    assert np.all(np.abs(lse - rlse) <= TOL * np.maximum(1.0, np.abs(rlse))), np.abs(lse - rlse).max()
    assert np.abs(hbar - rhbar).max() <= TOL, np.abs(hbar - rhbar).max()
    assert np.array_equal(np.isnan(hs), np.isnan(rhs))
    ok = ~np.isnan(rhs)
    assert np.abs(hs[ok] - rhs[ok]).max() <= TOL
    assert abs(loss[0] - rloss) <= TOL, (loss[0], rloss)


def test_replay_batch_logits():
    wl = W.aec_workload(7)
    _say(f"case {wl.name}")
    got = _run(wl)
    _check(wl, got, _ref(wl))
    assert np.isnan(got[2][3]), "a state without unresolved rows has no mean"


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_short_batch_splits_rows(dtype):
    wl = W.aec_workload(8, n_states=2, block=4, dtype=dtype, states_per_response=2)
    _say(f"case {wl.name}")
    dt = b.aec_desc(len(wl.unresolved), wl.vocab, wl.logits.shape[1], dtype, 2, len(wl.pair_next), 0.1, math.inf)
    assert b.aec_workspace_bytes(dt) >= len(wl.unresolved) * 2 * 12, "rows split over several workgroups"
    _check(wl, _run(wl), _ref(wl))


@pytest.mark.parametrize("vocab,stride,dtype", [(50257, 50264, "bf16"), (7, 8, "bf16"), (1000, 1000, "fp32"),
                                                (32003, 32016, "bf16"), (3, 4, "fp32")])
def test_ragged_vocabularies(vocab, stride, dtype):
    wl = W.aec_workload(9, n_states=6, block=8, vocab=vocab, row_stride=stride, dtype=dtype, states_per_response=3)
    _say(f"case {wl.name} stride {stride}")
    _check(wl, _run(wl), _ref(wl))


def test_gate_invalid_pairs_and_zero_denominator():
    wl = W.aec_workload(10, n_states=8, block=8, vocab=4096)
    nxt = wl.pair_next.copy()
    hs = wl.pair_h_source.copy()
    nxt[0] = -1                 # out of range: not a valid pair
    nxt[1] = 99
    hs[2] = np.nan              # no captured source mean: not valid
    got = _run(wl, pair_next=torch.from_numpy(nxt).cuda(), pair_h_source=torch.from_numpy(hs).cuda(),
               gate_max=0.5)
    _check(wl, got, _ref(wl, pair_next=nxt, h_source=hs, gate_max=0.5))
    # every pair gated off: D = 0 and the loss is 0
    got = _run(wl, gate_max=0.0)
    assert got[3][0] == 0.0


def test_deterministic():
    wl = W.aec_workload(11, n_states=4, block=16)
    a, c = _run(wl), _run(wl)
    for x, y in zip(a, c):
        assert np.array_equal(x, y, equal_nan=True)


# ------------------------------------------------------------------ backward

from helpers import assert_close  # noqa: E402


def _run_bwd(wl, grad_loss):
    dt = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
    dev = "cuda"
    logits = torch.from_numpy(wl.logits).to(dev).to(dt).contiguous()
    t = lambda x, ty: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(ty)
    kw = dict(unresolved=t(wl.unresolved, torch.uint8), state_rows=t(wl.state_rows, torch.int32),
              pair_next=t(wl.pair_next, torch.int32), pair_h_source=t(wl.pair_h_source, torch.float32),
              pair_weight=t(wl.pair_weight, torch.float32), rho=wl.rho, gate_max=wl.gate_max)
    lse, hbar, hs, _loss = b.aec_fwd(logits, wl.vocab, **kw)
    g = torch.tensor([grad_loss], dtype=torch.float32, device=dev)
    dx = b.aec_bwd(logits, wl.vocab, lse=lse, hbar=hbar, h_state=hs, grad_loss=g, **kw)
    torch.cuda.synchronize()
    return dx.float().cpu().numpy().astype(np.float64)


def _ref_bwd(wl, grad_loss):
    return ao.aec_backward(wl.logits[:, :wl.vocab], wl.unresolved, wl.state_rows, wl.pair_next,
                           wl.pair_h_source.astype(np.float64), wl.pair_weight.astype(np.float64), wl.rho,
                           wl.gate_max, grad_loss)


def _grad_scale(wl):
    # source means low enough that the hinges are open, and an upstream gradient
    # that brings the largest logit gradient to about 1, so that the absolute
    # bars are not met by small numbers alone
    wl.pair_h_source[:] = np.float32(0.05)
    g = _ref_bwd(wl, 1.0)
    assert np.abs(g).max() > 0, "some pair must pass a gradient"
    return 1.0 / np.abs(g).max(), g


def test_backward_replay_batch():
    wl = W.aec_workload(7)
    _say(f"case backward {wl.name}")
    scale, g1 = _grad_scale(wl)
    got = _run_bwd(wl, scale)
    assert np.all(got[:, wl.vocab:] == 0)
    assert_close("aec:dlogits", got[:, :wl.vocab], scale * g1, "bf16")
    # rows that no kept pair reaches get exactly zero
    assert np.all(got[np.abs(g1).max(axis=1) == 0] == 0)


@pytest.mark.parametrize("vocab,stride,dtype,n_states,block", [
    (151936, 151936, "fp32", 2, 4),        # rows split over several workgroups
    (50257, 50264, "bf16", 6, 8),
    (1000, 1000, "fp32", 6, 8),
    (7, 8, "bf16", 6, 4),
])
def test_backward_shapes(vocab, stride, dtype, n_states, block):
    wl = W.aec_workload(12, n_states=n_states, block=block, vocab=vocab, row_stride=stride, dtype=dtype,
                        states_per_response=2)
    if dtype == "fp32":
        # The gradient uses log p = x - lse with lse stored in fp32: its rounding,
        # ~2^-23 |lse|, enters every log-probability, so the absolute error of the
        # gradient grows with |lse| (1.6e-5 at |lse| ~ 60, for a gradient scaled to
        # 1). The fp32 bar of 1e-5 is checked on logits of moderate range
        # (|x| <= 8, |lse| <= ~20); the bf16 cases keep the full range.
        x = wl.logits[:, :vocab]
        wl.logits[:, :vocab] = x * np.float32(8.0 / np.abs(x).max())
    _say(f"case backward {wl.name} stride {stride}")
    scale, g1 = _grad_scale(wl)
    got = _run_bwd(wl, scale)
    assert_close("aec:dlogits", got[:, :vocab], scale * g1, dtype)


def test_backward_deterministic():
    wl = W.aec_workload(13, n_states=4, block=16)
    a, c = _run_bwd(wl, 3.0), _run_bwd(wl, 3.0)
    assert np.array_equal(a, c)


@pytest.mark.parametrize("vocab,stride", [(151936, 151936), (50257, 50264)])
def test_backward_in_place(vocab, stride):
    """dlogits may be the logits buffer itself: every element is read and written by
    the same thread, all of a thread's loads of a batch before its stores. The
    in-place result equals the out-of-place one bit for bit (columns past the
    vocabulary keep the logits in place)."""
    import ctypes
    wl = W.aec_workload(14, n_states=4, block=16, vocab=vocab, row_stride=stride, dtype="bf16")
    _say(f"case backward in place {wl.name} stride {stride}")
    dev = "cuda"
    logits = torch.from_numpy(wl.logits).to(dev).to(torch.bfloat16).contiguous()
    t = lambda x, ty: torch.from_numpy(np.ascontiguousarray(x)).to(dev).to(ty)
    kw = dict(unresolved=t(wl.unresolved, torch.uint8), state_rows=t(wl.state_rows, torch.int32),
              pair_next=t(wl.pair_next, torch.int32), pair_h_source=t(wl.pair_h_source, torch.float32),
              pair_weight=t(wl.pair_weight, torch.float32), rho=wl.rho, gate_max=wl.gate_max)
    lse, hbar, hs, _loss = b.aec_fwd(logits, vocab, **kw)
    g = torch.tensor([2.5], dtype=torch.float32, device=dev)
    ref = b.aec_bwd(logits, vocab, lse=lse, hbar=hbar, h_state=hs, grad_loss=g, **kw)
    inplace = logits.clone()
    n, s = inplace.shape
    d = b.aec_desc(n, vocab, s, inplace.dtype, hs.numel(), kw["pair_next"].numel(), wl.rho, wl.gate_max)
    ws = torch.empty(max(16, b.aec_workspace_bytes(d)), dtype=torch.uint8, device=dev)
    st = b._lib.bd_aec_bwd(ctypes.byref(d), b._ptr(inplace), b._ptr(kw["unresolved"]), b._ptr(kw["state_rows"]),
                           b._ptr(kw["pair_next"]), b._ptr(kw["pair_h_source"]), b._ptr(kw["pair_weight"]),
                           b._ptr(lse), b._ptr(hbar), b._ptr(hs), b._ptr(g), b._ptr(inplace), b._ptr(ws),
                           b._stream(inplace.device))
    assert st == b.OK, b._lib.bd_attn_last_error().decode()
    torch.cuda.synchronize()
    assert torch.equal(inplace[:, :vocab].view(torch.int16), ref[:, :vocab].view(torch.int16))
    assert torch.equal(inplace[:, vocab:].view(torch.int16), logits[:, vocab:].view(torch.int16))


@pytest.mark.parametrize("n_states,block", [(1100, 8), (100, 90)])
def test_batches_past_the_lds_forms(n_states, block):
    """Batches with more than 1024 states or more than 8192 rows take the global-memory
    forms of the two single-workgroup kernels (the LDS-resident forms cover smaller
    ones): forward and gradient against the oracle, with more than 256 pairs so that
    the pair loops run past their first batch."""
    wl = W.aec_workload(15, n_states=n_states, block=block, vocab=64, states_per_response=4)
    assert len(wl.unresolved) > 8192 or n_states > 1024
    assert len(wl.pair_next) > 256 or n_states <= 256
    _say(f"case {wl.name}: {n_states} states x {block} rows")
    _check(wl, _run(wl), _ref(wl))
    scale, g1 = _grad_scale(wl)
    got = _run_bwd(wl, scale)
    assert_close("aec:dlogits", got[:, :wl.vocab], scale * g1, "bf16")


def test_lds_forms_with_many_pairs():
    """The LDS-resident forms with more than 256 pairs (pairs past each thread's
    first one are read in the loop) and more than one 2048-pair tile of the
    gradient's state sums (the pair list repeated four times): forward and gradient
    against the oracle."""
    wl = W.aec_workload(16, n_states=1000, block=8, vocab=64, states_per_response=1000)
    wl.pair_next = np.tile(wl.pair_next, 4)
    wl.pair_h_source = np.tile(wl.pair_h_source, 4)
    wl.pair_weight = np.tile(wl.pair_weight, 4) * np.float32(0.25)
    assert len(wl.unresolved) <= 8192 and len(wl.pair_next) > 2048
    _say(f"case {wl.name}: {len(wl.pair_next)} pairs")
    _check(wl, _run(wl), _ref(wl))
    scale, g1 = _grad_scale(wl)
    got = _run_bwd(wl, scale)
    assert_close("aec:dlogits", got[:, :wl.vocab], scale * g1, "bf16")
