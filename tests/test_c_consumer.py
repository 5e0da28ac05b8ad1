"""The C ABI from a plain C99 program (tests/c_consumer/bd_attn_consumer.c, built by
build.py with -std=c99 -pedantic -Werror against include/bd_attn.h): no Python and no
torch in the process that calls the library.

* host part (CPU): the program plans a two-segment batch, gets the documented statuses
  for invalid calls, self-checks the serialized work lists and prints the plan's
  sizes, which must equal the binding's for the same metadata and the oracle's count
  of visible pairs;
* GPU part: the program runs the forward and the backward on seeded bf16 inputs with
  device memory from the HIP runtime, and its outputs must match the oracle on the
  inputs it wrote.
"""
import json
import os
import subprocess

import numpy as np
import pytest

from block_diffusion_attention_amd import workloads as W
from helpers import assert_close
from oracle import bd_oracle as orc

b = pytest.importorskip("block_diffusion_attention_amd.binding")
from block_diffusion_attention_amd import build as bd  # noqa: E402

# the batch the program plans (see the program's header comment)
META = W.Meta([48, 32], [0, 32], [[1, 3], [2]], 16, 4, 2, 64, "bf16")


def _consumer():
    if not os.path.exists(bd.CONSUMER_BIN):
        if not os.path.exists(b.LIB_PATH):
            pytest.skip("libbdattn.so not built")
        bd.build_consumer()
    return bd.CONSUMER_BIN


def _run(*args):
    r = subprocess.run([_consumer(), *args], stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-3000:]
    return r.stdout


def test_c_program_plans_and_checks_on_the_host():
    info = json.loads(_run().splitlines()[0])
    p = b.Plan(META, b.FLAG_CHECK_PLAN)
    assert info["version"] == b.version()
    assert (info["tq"], info["tk"]) == (p.tq, p.tk) == (META.tq, META.tk)
    assert (info["meta_bytes"], info["ws_fwd"], info["ws_bwd"]) == (p.meta_bytes, p.ws_fwd_bytes, p.ws_bwd_bytes)
    assert info["pairs"] == p.visible_pairs == orc.visible_pairs(META)
    assert (info["fwd_kernels"], info["bwd_kernels"]) == (p.kernels(False), p.kernels(True))
    pi = p.info()
    assert {k: info[k] for k in ("split", "dkdv_masked", "fwd_workgroups", "dkdv_workgroups")} == {
        k: pi[k] for k in ("split", "dkdv_masked", "fwd_workgroups", "dkdv_workgroups")}


def _read_bf16(raw, n, shape):
    u = np.frombuffer(raw, dtype=np.uint16, count=n).astype(np.uint32) << 16
    return u.view(np.float32).reshape(shape)


@pytest.mark.gpu
def test_c_program_forward_and_backward_match_the_oracle(tmp_path):
    out = tmp_path / "consumer.bin"
    print("case C consumer: fwd + bwd", flush=True)
    _run("--gpu", str(out))
    raw = out.read_bytes()
    tq, tk, hq, hkv, d = np.frombuffer(raw, dtype=np.int32, count=5)
    assert (tq, tk, hq, hkv, d) == (META.tq, META.tk, 4, 2, 64)
    nq, nk, nl = tq * hq * d, tk * hkv * d, tq * hq
    pos = 20
    arrays = {}
    for name, n, shape, dt in (("q", nq, (tq, hq, d), "bf16"), ("k", nk, (tk, hkv, d), "bf16"),
                               ("v", nk, (tk, hkv, d), "bf16"), ("do", nq, (tq, hq, d), "bf16"),
                               ("o", nq, (tq, hq, d), "bf16"), ("lse", nl, (tq, hq), "f32"),
                               ("dq", nq, (tq, hq, d), "bf16"), ("dk", nk, (tk, hkv, d), "bf16"),
                               ("dv", nk, (tk, hkv, d), "bf16")):
        size = n * (2 if dt == "bf16" else 4)
        chunk = raw[pos:pos + size]
        arrays[name] = (_read_bf16(chunk, n, shape) if dt == "bf16"
                        else np.frombuffer(chunk, dtype=np.float32).reshape(shape))
        pos += size
    assert pos == len(raw)
    wl = W.Workload("c-consumer", META, arrays["q"], arrays["k"], arrays["v"], arrays["do"], "fwd+bwd")
    o, lse = orc.attention_fwd(wl.q, wl.k, wl.v, META, scale=META.softmax_scale)
    dq, dk, dv = orc.attention_bwd(wl.q, wl.k, wl.v, wl.do, META, scale=META.softmax_scale)
    for name, ref in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv)):
        assert_close(f"c-consumer:{name}", arrays[name].astype(np.float64), ref, "bf16")
    assert np.abs(arrays["lse"] - lse).max() <= 2e-3
