"""Host planner and C ABI, on the CPU (no kernel is launched here).

* the library loads and exports every function include/bd_attn.h declares;
* metadata validation returns the documented status codes with a message;
* the work lists encode exactly the oracle's visibility (every query token in
  one query tile, every key token in one key tile, ranges == dense mask);
* plans are deterministic and their size grows with tiles, not with N^2.
"""
import ctypes
import itertools
import os
import re

import numpy as np
import pytest

from oracle import bd_oracle as orc
from block_diffusion_attention_amd.workloads import Meta, config_meta, random_meta
from plan_decode import decode, ktile_visibility, qtile_visibility

b = pytest.importorskip("block_diffusion_attention_amd.binding")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_exports_every_declared_function():
    hdr = open(os.path.join(ROOT, "include", "bd_attn.h")).read()
    names = set(re.findall(r"^\s*(?:bd_attn_status|const char\*|int32_t)\s+(bd_\w+)\s*\(", hdr, re.M))
    assert {"bd_attn_plan", "bd_attn_fwd", "bd_attn_bwd"} <= names
    lib = ctypes.CDLL(b.LIB_PATH)
    for n in sorted(names):
        assert hasattr(lib, n), n
    assert set(b.EXPORTED) == names


def test_plan_info_reports_the_plans_choices():
    """bd_attn_plan_info against the decoded work lists and the documented rules."""
    def info_and_lists(k, flags=0):
        p = b.Plan(config_meta(k, np.random.default_rng(k)), flags)
        return p.info(), decode(p.host_blob())

    i2, r2 = info_and_lists(2)                                 # one request's denoising step
    assert (i2["split"], i2["split_grid"], i2["split_tiles"]) == (1, 1, 2)
    assert i2["fwd_workgroups"] == len(r2["split"]) and i2["query_tiles"] == len(r2["qtiles"]) == 1
    assert b.Plan(config_meta(2, np.random.default_rng(2)), b.FLAG_NO_XCD).info()["split_grid"] == 0
    i6, _ = info_and_lists(6)                                  # two query tiles: records
    assert (i6["split"], i6["split_grid"]) == (1, 0)
    i3, r3 = info_and_lists(3)                                 # packed replay
    assert (i3["split"], i3["split_tiles"], i3["dkdv_masked"], i3["dkdv_split_tiles"]) == (0, 0, 0, 0)
    assert (i3["fwd_workgroups"], i3["dq_workgroups"], i3["dkdv_workgroups"]) == (
        len(r3["fwd"]), len(r3["dq"]), len(r3["bwd"]))
    assert i3["key_tiles"] == len(r3["ktiles"])
    i4, r4 = info_and_lists(4)                                 # staircase: split key tiles
    assert i4["dkdv_split_tiles"] == len(r4["bmerge"]) > 0
    assert info_and_lists(4, b.FLAG_FWD_VT)[0]["fwd_vt"] == 1 and i4["fwd_vt"] == 0
    assert info_and_lists(4, b.FLAG_DEBUG_CHECKS)[0]["debug_checks"] == 1 and i4["debug_checks"] == 0
    i1, r1 = info_and_lists(1)                                 # fp32: the forward runs the dQ items
    assert i1["fwd_workgroups"] == i1["dq_workgroups"] == len(r1["dq"])
    assert b._lib.bd_attn_plan_info(None, None) == b.EINVAL


def test_device_check_query_rejects_null_and_flag_is_accepted():
    # no HIP call is made for a NULL count
    assert b._lib.bd_attn_device_check_errors(None, 0) == b.EINVAL
    assert "count is NULL" in b._lib.bd_attn_last_error().decode()
    # the debug flag also runs the host self-check, and changes no work list
    meta = config_meta(4, np.random.default_rng(4))
    assert b.Plan(meta, b.FLAG_DEBUG_CHECKS).host_blob() == b.Plan(meta).host_blob()


def _status(meta, **over):
    d = dict(ctx=meta.ctx_len, q0=meta.ctx_q_begin, off=meta.canvas_offsets, cb=meta.flat_canvas_block_idx,
             B=meta.block_size, hq=meta.num_q_heads, hkv=meta.num_kv_heads, D=meta.head_dim,
             dtype=0 if meta.dtype == "bf16" else 1, scale=0.0, S=len(meta.ctx_len))
    d.update(over)
    keep = [b._arr(d["ctx"]), b._arr(d["q0"]), b._arr(d["off"]), b._arr(d["cb"])]
    desc = b.Desc()
    desc.num_segments = d["S"]
    desc.ctx_len, desc.ctx_q_begin, desc.canvas_offsets, desc.canvas_block_idx = (
        ctypes.cast(x, b._i32p) for x in keep)
    if "bo" in d:
        keep.append(b._arr(d["bo"]))
        desc.block_offset = ctypes.cast(keep[-1], b._i32p)
    desc.block_size, desc.num_q_heads, desc.num_kv_heads, desc.head_dim = d["B"], d["hq"], d["hkv"], d["D"]
    desc.dtype, desc.softmax_scale, desc.flags = d["dtype"], d["scale"], 0
    h = ctypes.c_void_p()
    st = b._lib.bd_attn_plan(ctypes.byref(desc), ctypes.byref(h))
    msg = b._lib.bd_attn_last_error().decode()
    if st == 0:
        b._lib.bd_attn_plan_destroy(h)
    return st, msg


GOOD = Meta([64, 32], [0, 32], [[1, 2], [1]], 16, 4, 2, 128, "bf16")


def test_planning_from_many_threads():
    # plans are built on the caller's thread with no shared state: concurrent
    # planning gives the same work lists as planning alone, and each thread's
    # last error message is its own (ctypes releases the interpreter lock)
    import threading
    metas = [config_meta(k, np.random.default_rng(k)) for k in (1, 2, 4, 6)]
    metas += [random_meta(np.random.default_rng(s), hq=4, hkv=2, d=64, dtype="bf16", offsets=True)
              for s in range(4)]
    ref = [b.Plan(m).host_blob() for m in metas]
    bad = [(dict(D=96), "head_dim must be 64 or 128"), (dict(hq=3), "multiple of num_kv_heads"),
           (dict(B=0), "block_size must be >= 1")]
    failures = []

    def work(tid):
        try:
            for rep in range(6):
                over, needle = bad[(tid + rep) % len(bad)]
                st, msg = _status(GOOD, **over)
                assert st != 0 and needle in msg, (tid, rep, st, msg)
                i = (tid + rep) % len(metas)
                assert b.Plan(metas[i]).host_blob() == ref[i], (tid, rep, i)
        except Exception as e:  # collected and reported by the main thread
            failures.append(repr(e))

    threads = [threading.Thread(target=work, args=(t,)) for t in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert not failures, failures[:3]


@pytest.mark.parametrize("over,code", [
    (dict(S=0), b.EINVAL),
    (dict(B=0), b.EINVAL),
    (dict(ctx=[65, 32]), b.EINVAL),          # not a multiple of B
    (dict(ctx=[-16, 32]), b.EINVAL),
    (dict(q0=[70, 32]), b.EINVAL),           # beyond ctx_len
    (dict(q0=[-1, 32]), b.EINVAL),
    (dict(cb=[1, 5, 1]), b.EINVAL),          # block index beyond ctx_len/B
    (dict(cb=[1, -1, 1]), b.EINVAL),
    (dict(off=[1, 2, 3]), b.EINVAL),         # offsets must start at 0
    (dict(off=[0, 2, 1]), b.EINVAL),         # non-decreasing
    (dict(hq=6, hkv=4), b.EINVAL),           # Hq % Hkv
    (dict(hkv=0), b.EINVAL),
    (dict(D=96), b.EUNSUPPORTED),
    (dict(hq=64, hkv=1), b.EUNSUPPORTED),    # group size above 32
    (dict(dtype=7), b.EINVAL),
    (dict(scale=float("inf")), b.EINVAL),
    (dict(ctx=[0, 0], q0=[0, 0], off=[0, 0, 0], cb=[]), b.EINVAL),   # no query at all
    (dict(bo=[16, 0]), b.EINVAL),            # grid offset must be below the block size
    (dict(bo=[-1, 0]), b.EINVAL),
    (dict(bo=[3, 0]), b.EINVAL),             # ctx_len + offset not a multiple of B
    (dict(ctx=[61, 32], bo=[3, 0], cb=[1, 5, 1]), b.EINVAL),   # b beyond (ctx_len + o) / B
    (dict(ctx=[0, 32], q0=[0, 32], bo=[4, 0]), b.EINVAL),      # empty context: offset 0 only
])
def test_validation_errors(over, code):
    st, msg = _status(GOOD, **over)
    assert st == code and msg
    st_ok, _ = _status(GOOD)
    assert st_ok == b.OK


@pytest.mark.parametrize("over,needle", [
    # 2^30 packed query tokens: beyond the planner's token limit (INT32_MAX / 2)
    (dict(S=1, ctx=[1 << 30], q0=[0], off=[0, 0], cb=[], B=1 << 20, hq=4, hkv=2), "token count"),
    # 2^26 tokens x 32 query heads = 2^31 rows: beyond int32 rows per tensor
    (dict(S=1, ctx=[1 << 26], q0=[0], off=[0, 0], cb=[], B=1 << 16, hq=32, hkv=1), "fit in int32"),
])
def test_size_limits(over, needle):
    st, msg = _status(GOOD, **over)
    assert st == b.EINVAL and needle in msg, msg


def test_shifted_grid_and_causal_metadata_accepted():
    st, msg = _status(GOOD, ctx=[61, 32], bo=[3, 0], cb=[1, 4, 1])
    assert st == b.OK, msg
    st, msg = _status(GOOD, ctx=[61, 29], q0=[0, 29], bo=[3, 3])
    assert st == b.OK, msg


def test_null_and_alignment_checks():
    p = b.Plan(GOOD)
    vp = ctypes.c_void_p
    st = b._lib.bd_attn_fwd(p.handle, vp(0), vp(16), vp(16), vp(16), vp(16), vp(16), vp(0), vp(0))
    assert st == b.EINVAL and "meta_dev" in b._lib.bd_attn_last_error().decode()
    st = b._lib.bd_attn_fwd(p.handle, vp(16), vp(18), vp(16), vp(16), vp(16), vp(16), vp(0), vp(0))
    assert st == b.EINVAL and "aligned" in b._lib.bd_attn_last_error().decode()
    st = b._lib.bd_attn_bwd(p.handle, *([vp(16)] * 10), vp(0), vp(0))
    assert st == b.EWORKSPACE
    assert b._lib.bd_attn_fwd(None, *([vp(16)] * 8)) == b.EINVAL
    assert b._lib.bd_attn_plan_destroy(None) == b.OK


def _check_plan(meta, flags=0):
    p = b.Plan(meta, flags)
    rec = decode(p.host_blob())
    G = meta.num_q_heads // meta.num_kv_heads
    mask = orc.dense_mask(meta)
    assert p.visible_pairs == int(mask.sum()) == orc.visible_pairs(meta)
    assert (p.tq, p.tk) == mask.shape
    vis, cover = qtile_visibility(rec, meta, G)
    assert (cover == 1).all(), "every query token in exactly one query tile"
    assert (vis == mask).all()
    kvis, kcover = ktile_visibility(rec, meta, G)
    assert (kcover == 1).all(), "every key token in exactly one key tile"
    assert (kvis == mask).all()
    hkv = meta.num_kv_heads
    nq, nk = len(rec["qtiles"]), len(rec["ktiles"])
    # launch lists: every (tile, kv head) exactly once, empty slots marked -1
    dq = [tuple(x[:2]) for x in rec["dq"] if x[0] >= 0]
    assert sorted(dq) == sorted(itertools.product(range(nq), range(hkv)))
    # dK/dV items: every (key tile, kv head) once, either whole or split into
    # parts whose chunk ranges tile [0, chunks) in slot order, listed by one
    # merge record
    qct = 64 // G
    cpc = -(-meta.block_size // qct)

    def chunks(i):
        t = rec["ktiles"][i]
        return -(-t[4] // qct) + t[7] * cpc

    whole, parts = [], {}
    for ktile, ys, c0, c1 in rec["bwd"]:
        if ktile < 0:
            continue
        h, slot = ys % hkv, ys // hkv - 1
        if slot < 0:
            assert c0 == 0 and c1 >= chunks(ktile)
            whole.append((int(ktile), int(h)))
        else:
            assert slot not in parts
            parts[int(slot)] = (int(ktile), int(h), int(c0), int(c1))
    merged = []
    for ktile, h, first, count in rec["bmerge"]:
        spans = [parts[s] for s in range(first, first + count)]
        assert all(sp[:2] == (ktile, h) for sp in spans)
        assert spans[0][2] == 0 and spans[-1][3] == chunks(ktile)
        assert all(a_[3] == b_[2] and a_[3] > a_[2] for a_, b_ in zip(spans, spans[1:]))
        merged.append((int(ktile), int(h)))
    assert len(parts) == sum(int(c) for *_, c in rec["bmerge"])
    assert sorted(whole + merged) == sorted(itertools.product(range(nk), range(hkv)))
    if meta.dtype != "bf16" or flags & b.FLAG_NO_SPLIT:
        assert len(rec["bmerge"]) == 0
    if len(rec["split"]) == 0:
        fw = [tuple(x[:2]) for x in rec["fwd"] if x[0] >= 0]
        assert sorted(fw) == sorted(dq)
        assert len(rec["merge"]) == 0
    else:
        _check_split(rec, meta, G)
    return p, rec


def _check_split(rec, meta, G):
    """Split path: every partial slot is written by exactly one launched part;
    the parts of a (query tile, kv head) cover its key tiles once, in slot
    order; each part and merge record carries a copy of its query tile; the merge
    workgroups of a tile cover its rows and run on the XCD of its first part."""
    assert len(rec["fwd"]) == 0
    hkv, D = meta.num_kv_heads, meta.head_dim
    qt_index = {tuple(int(x) for x in q): i for i, q in enumerate(rec["qtiles"])}
    sp = rec["split"]
    live = [(i, r) for i, r in enumerate(sp) if r[8] >= 0]
    slots = sorted(int(r[11]) for _, r in live)
    assert slots == list(range(len(live)))
    by_slot = {int(r[11]): r for _, r in live}
    launch_pos = {int(r[11]): i for i, r in live}
    bpw = 2 * (D // 32)          # merge blocks (32 rows x 16 columns) per 32-row wave of a part
    seen = {}
    for i, m in enumerate(rec["merge"]):
        if m[8] < 0:
            continue
        qt = qt_index[tuple(int(x) for x in m[:8])]
        kvh, first, count, blk = (int(x) for x in m[8:12])
        seen.setdefault((qt, kvh, first, count), []).append(blk)
        assert i % 8 == launch_pos[first] % 8, "merge workgroup off its parts' XCD"
    assert sorted((q, h) for q, h, _, _ in seen) == sorted(itertools.product(range(len(rec["qtiles"])), range(hkv)))
    covered = []
    for (qt, kvh, first, count), rows in seen.items():
        t = rec["qtiles"][qt]
        assert sorted(rows) == list(range(-(-int(t[1]) * G // 32) * bpw))
        spans = [by_slot[s] for s in range(first, first + count)]
        assert all(qt_index[tuple(int(x) for x in r[:8])] == qt and r[8] == kvh for r in spans)
        assert spans[0][9] == 0 and all(a_[10] == b_[9] and a_[10] > a_[9] for a_, b_ in zip(spans, spans[1:]))
        ntiles = -(-t[4] // 64) + -(-t[7] // 64)
        assert spans[-1][10] == ntiles
        covered += range(first, first + count)
    assert sorted(covered) == slots


def test_plan_encodes_oracle_visibility_exhaustive():
    n = 0
    for B in (1, 2, 3):
        for nb in range(0, 4):
            C = nb * B
            for q0 in sorted({0, C, min(C, B)}):
                for cv in [[]] + [[x] for x in range(nb + 1)] + [list(p) for p in itertools.permutations(range(nb + 1), 2)]:
                    if (C - q0) + len(cv) * B == 0:
                        continue
                    _check_plan(Meta([C], [q0], [cv], B, 2, 1, 64, "bf16"))
                    n += 1
    assert n > 100


def test_plan_encodes_shifted_grid_and_causal_exhaustive():
    n = 0
    for B in (2, 3, 5):
        for nb in range(1, 4):
            for o in range(B):
                C = nb * B - o
                for causal in (False, True):
                    for q0 in sorted({0, C, min(C, B - o), max(0, C - B)}):
                        for cv in [[]] + [[x] for x in range(nb + 1)] + [[nb, 0]]:
                            if (C - q0) + len(cv) * B == 0:
                                continue
                            _check_plan(Meta([C], [q0], [cv], B, 2, 1, 64, "bf16", block_offset=[o],
                                             clean_causal=causal))
                            n += 1
    assert n > 150


@pytest.mark.parametrize("seed", range(8))
def test_plan_encodes_shifted_and_causal_random(seed):
    rng = np.random.default_rng(900 + seed)
    meta = random_meta(rng, hq=8, hkv=2, d=64, max_segments=4, max_blocks=8,
                       block_sizes=(2, 4, 16, 32, 48, 64, 160), max_canvases=4, dtype="bf16",
                       offsets=True, clean_causal=bool(seed % 2))
    _check_plan(meta)
    _check_plan(meta, b.FLAG_FORCE_SPLIT)


def test_commit_folded_step_plan():
    # the finished block (queries from C - B, token-causal) and the next canvas
    # over a 2048-token context, grid offset 17 (a 2031-token prompt + blocks)
    meta = Meta([2048 - 17], [2048 - 17 - 32], [[64]], 32, 32, 8, 128, "bf16",
                block_offset=[17], clean_causal=True)
    p, _rec = _check_plan(meta)
    assert p.kernel_names(True)[1] == "dkdv_masked"
    # pairs: the canvas sees the whole context and itself; the block is causal
    C = 2048 - 17
    want = 32 * (C + 32) + sum(t + 1 for t in range(C - 32, C))
    assert p.visible_pairs == want


@pytest.mark.parametrize("seed", range(12))
def test_plan_encodes_oracle_visibility_random(seed):
    rng = np.random.default_rng(500 + seed)
    meta = random_meta(rng, hq=4, hkv=2, d=64, max_segments=4, max_blocks=8,
                       block_sizes=(1, 2, 4, 8, 16, 32, 48), max_canvases=4, dtype="bf16")
    _check_plan(meta)
    _check_plan(meta, b.FLAG_FORCE_SPLIT)
    _check_plan(meta, b.FLAG_NO_XCD)


@pytest.mark.parametrize("G", [1, 2, 3, 4, 8, 32])
def test_plan_group_sizes(G):
    meta = Meta([96, 64], [0, 64], [[2, 0, 3], [4]], 16, 2 * G, 2, 64, "bf16")
    _check_plan(meta)


def test_plan_large_blocks():
    # blocks larger than a query tile / key tile (B=256 as in the 256-token block models)
    meta = Meta([512], [0], [[1, 2, 0]], 256, 8, 2, 128, "bf16")
    _check_plan(meta)


@pytest.mark.parametrize("k", [2, 4])
def test_named_workload_plans(k):
    meta = config_meta(k, np.random.default_rng(k))
    p = b.Plan(meta)
    assert p.visible_pairs == orc.visible_pairs(meta)
    rec = decode(p.host_blob())
    if k == 2:
        # 2048 context keys + 32 own keys = 33 key tiles of 64 per kv head, cut
        # into parts of 2 tiles (264 tiles over 256 compute units): 17 parts per
        # kv head, merged by 4 x 8 one-wave workgroups (32 rows x 16 columns) each
        live = rec["split"][rec["split"][:, 8] >= 0]
        assert len(live) == 8 * 17
        assert (live[:, 10] - live[:, 9] <= 2).all()
        assert len(rec["merge"][rec["merge"][:, 8] >= 0]) == 8 * 32
        _check_split(rec, meta, meta.num_q_heads // meta.num_kv_heads)


def test_plan_is_deterministic():
    meta = config_meta(5, np.random.default_rng(5))
    a = b.Plan(meta).host_blob()
    c = b.Plan(meta).host_blob()
    assert a == c


def test_metadata_grows_with_tiles_not_n_squared():
    sizes = []
    for n in (64, 128, 256, 512):
        meta = Meta([32 * n], [0], [[n // 2, n]], 32, 32, 8, 128, "bf16")
        sizes.append(b.Plan(meta).meta_bytes)
    # doubling the context about doubles the work lists (linear), never quadruples them
    for s0, s1 in zip(sizes, sizes[1:]):
        assert s1 < 2.3 * s0


@pytest.mark.parametrize("ctx,q0,B,hq,hkv,dt,want", [
    # block a multiple of 32, 64 / G tokens dividing it, ranges at block starts
    ([256, 128], [0, 128], 32, 32, 8, "bf16", "dkdv"),
    ([256, 128], [0, 64], 64, 8, 8, "bf16", "dkdv"),          # G = 1: 64 tokens per chunk
    ([256, 128], [0, 40], 32, 32, 8, "bf16", "dkdv_masked"),  # query range inside a block
    ([256, 128], [0, 128], 16, 32, 8, "bf16", "dkdv_masked"),  # block below 32 keys
    ([288, 192], [0, 96], 96, 12, 4, "bf16", "dkdv_masked"),   # G = 3 does not divide 64
    ([256, 128], [0, 96], 32, 8, 8, "bf16", "dkdv_masked"),    # 64 tokens per chunk > block
    ([256, 128], [0, 40], 32, 32, 8, "fp32", "dkdv"),          # fp32 has one dK/dV kernel
    # grid offsets: a multiple of 32 with ranges at (shifted) block starts keeps
    # the unmasked program; any other offset or token-causal rows need limits
    ([224, 96], [32, 96], (64, [32, 32]), 32, 8, "bf16", "dkdv"),
    ([240, 112], [0, 112], (32, [16, 16]), 32, 8, "bf16", "dkdv_masked"),
    ([256, 128], [0, 128], (32, None, "causal"), 32, 8, "bf16", "dkdv_masked"),
])
def test_dkdv_variant_selection(ctx, q0, B, hq, hkv, dt, want):
    """The unmasked dK/dV program is only chosen when every (64-row query chunk,
    32-key group) pair is either wholly visible or wholly hidden."""
    offs, causal = None, False
    if isinstance(B, tuple):
        B, offs, causal = B[0], B[1], len(B) > 2
    meta = Meta(ctx, q0, [[1], [0, 2]], B, hq, hkv, 64, dt, block_offset=offs, clean_causal=causal)
    names = b.Plan(meta).kernel_names(True)
    # bf16: dQ (with the row terms) first, then dK/dV; fp32: row terms, dK/dV, dQ
    assert names[1] == want
    assert names[0] == ("dq" if dt == "bf16" else "bwd_pre")


def test_transposed_v_copy_only_on_request():
    """The V transpose pre-pass runs only with FWD_VT (block size a multiple of
    8, bf16); FWD_DIRECT wins over it."""
    step = config_meta(2, np.random.default_rng(2))
    replay = config_meta(3, np.random.default_rng(3))
    assert "transpose_v" not in b.Plan(step).kernel_names(False)
    assert "transpose_v" not in b.Plan(replay).kernel_names(False)
    assert "transpose_v" in b.Plan(step, b.FLAG_FWD_VT).kernel_names(False)
    assert "transpose_v" in b.Plan(replay, b.FLAG_FWD_VT).kernel_names(False)
    assert "transpose_v" not in b.Plan(replay, b.FLAG_FWD_DIRECT | b.FLAG_FWD_VT).kernel_names(False)
    # block sizes that are not a multiple of 8 never take it
    odd = Meta([96, 60], [0, 60], [[1], [0, 2]], 12, 8, 2, 64, "bf16")
    assert "transpose_v" not in b.Plan(odd, b.FLAG_FWD_VT).kernel_names(False)


def test_dkdv_split_of_long_key_tiles():
    """One long context (the staircase shape): its first key tiles see far more
    query chunks than the average workgroup, so their ranges are split and
    merged; the packed replay is balanced without splitting. FORCE_SPLIT splits
    every multi-chunk item, NO_SPLIT none."""
    stair = config_meta(4, np.random.default_rng(4))
    p = b.Plan(stair)
    assert p.kernel_names(True)[2] == "dkdv_merge"
    rec = decode(p.host_blob())
    assert len(rec["bmerge"]) > 0
    assert "dkdv_merge" not in b.Plan(stair, b.FLAG_NO_SPLIT).kernel_names(True)
    replay = config_meta(3, np.random.default_rng(3))
    assert "dkdv_merge" not in b.Plan(replay).kernel_names(True)
    small = Meta([96, 64], [0, 64], [[2, 0, 3], [4]], 16, 8, 2, 64, "bf16")
    _check_plan(small, b.FLAG_FORCE_SPLIT)
    _check_plan(small, b.FLAG_NO_SPLIT)
    f32 = Meta([96, 64], [0, 64], [[2, 0, 3], [4]], 16, 8, 2, 64, "fp32")
    _check_plan(f32, b.FLAG_FORCE_SPLIT)


# Nine segments over two kv heads with a short query stream: the forward takes
# the split path and its XCD-grouped launch order has empty slots (-1), which
# the forward kernels must skip.
SPLIT_WITH_EMPTY_SLOTS = Meta(
    [352, 264, 312, 264, 262, 223, 155, 102, 155], [0] * 9,
    [[1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11], [1, 2, 3, 4, 5, 6, 7, 8, 9], [1, 3, 4, 5, 8, 10],
     [1, 2, 3, 4, 7, 9], [1, 4, 5, 8, 9], [2, 4, 7], [3, 4, 5], [1, 2, 3, 4], [3, 5]],
    32, 8, 2, 128, "bf16", block_offset=[0, 24, 8, 24, 26, 1, 5, 26, 5])


def test_split_launch_order_has_empty_slots():
    p, rec = _check_plan(SPLIT_WITH_EMPTY_SLOTS)
    assert len(rec["merge"]) > 0 and (rec["split"][:, 8] < 0).any()


# ---------------------------------------------------------------- work-list self-check

def _sections(blob):
    return {name: (blob[2 + 2 * i], blob[3 + 2 * i]) for i, name in enumerate(
        ["qtiles", "fwd", "split", "merge", "dq", "ktiles", "canvq", "bwd", "bmerge"])}


@pytest.mark.parametrize("k", [1, 2, 3, 4, 6])
@pytest.mark.parametrize("flags", [0, b.FLAG_NO_XCD, b.FLAG_FORCE_SPLIT, b.FLAG_NO_SPLIT, b.FLAG_DKDV_RUNS])
def test_plan_self_check_accepts_every_plan(k, flags):
    meta = config_meta(k, np.random.default_rng(k))
    p = b.Plan(meta, flags | b.FLAG_CHECK_PLAN)   # bd_attn_plan runs the check itself
    p.check()
    assert b.Plan(meta, flags).host_blob() == p.host_blob()   # the flag changes nothing else


@pytest.mark.parametrize("seed", range(12))
def test_plan_self_check_accepts_random_plans(seed):
    rng = np.random.default_rng(seed)
    meta = random_meta(rng, hq=4, hkv=2, d=64, max_segments=4, max_blocks=8,
                       block_sizes=(1, 2, 4, 8, 16, 32, 48), max_canvases=4, dtype="bf16",
                       offsets=seed % 2 == 1, clean_causal=seed % 3 == 2)
    for flags in (0, b.FLAG_FORCE_SPLIT):
        b.Plan(meta, flags | b.FLAG_CHECK_PLAN).check()


# (section, record, field, value as a function of the plan's section sizes, expected message)
CORRUPTIONS = [
    ("dq", 0, 0, lambda n: n["qtiles"], "query tile index"),
    ("dq", 0, 1, lambda n: 8, "kv head"),
    ("dq", 0, 3, lambda n: 10 ** 6, "key tile range"),
    ("split", 0, 11, lambda n: 10 ** 6, "partial slot"),
    ("split", 0, 1, lambda n: 10 ** 6, "query rows"),
    ("merge", 0, 10, lambda n: 10 ** 6, "partial slots"),
    ("ktiles", 0, 7, lambda n: n["canvq"] + 1, "canvas-query entries"),
    ("ktiles", 0, 1, lambda n: 129, "keys outside"),
    ("canvq", 0, 0, lambda n: -1, "whole canvas"),
    ("canvq", 0, 1, lambda n: 1, "whole canvas"),
    ("bwd", 0, 0, lambda n: n["ktiles"], "key tile index"),
    ("qtiles", 0, 4, lambda n: 10 ** 7, "clean key range"),
]


@pytest.mark.parametrize("sec,rec,field,val,needle", CORRUPTIONS)
def test_plan_check_rejects_bad_records(sec, rec, field, val, needle):
    # the single-request serving workload uses every forward record kind (split
    # parts and merge blocks) as well as the backward lists
    meta = config_meta(2, np.random.default_rng(2))
    p = b.Plan(meta)
    blob = p.host_blob()
    secs = _sections(blob)
    counts = {n: c for n, (c, _) in secs.items()}
    width = {"qtiles": 8, "fwd": 4, "split": 16, "merge": 16, "dq": 4, "ktiles": 8, "canvq": 4, "bwd": 4,
             "bmerge": 4}[sec]
    cnt, off = secs[sec]
    assert cnt > rec
    # first live record of the launch lists (empty slots carry -1 and are skipped)
    live_field = {"dq": 0, "bwd": 0, "split": 8, "merge": 8}.get(sec)
    if live_field is not None:
        while blob[off + rec * width + live_field] < 0:
            rec += 1
    blob[off + rec * width + field] = val(counts)
    with pytest.raises(b.BdAttnError, match=needle) as e:
        p.check(blob)
    assert f"{sec} record {rec}" in str(e.value)


def test_plan_check_rejects_bad_header_and_size():
    p = b.Plan(config_meta(4, np.random.default_rng(4)))
    blob = p.host_blob()
    bad = list(blob)
    bad[2] += 1                       # query tile count
    with pytest.raises(b.BdAttnError, match="record count"):
        p.check(bad)
    bad = list(blob)
    bad[1] = 99                       # version
    with pytest.raises(b.BdAttnError, match="magic or version"):
        p.check(bad)
    with pytest.raises(b.BdAttnError) as e:
        p.check(blob[:-4])
    assert e.value.status == 3        # BD_ATTN_EWORKSPACE
    p.check(blob)


def test_transposed_v_copy_only_below_its_offset_range():
    # the transposed-V kernel addresses V^T rows with 32-bit byte offsets: a key
    # stream past 2^30 / head_dim keys falls back to the direct kernel
    small = Meta([4096], [0], [[1]], 32, 4, 1, 128, "bf16")
    assert "transpose_v" in b.Plan(small, b.FLAG_FWD_VT).kernel_names(False)
    n = (1 << 30) // 128                         # keys at which D * tk_pad * 2 reaches 2^31
    big = Meta([n], [n], [[n // 32]], 32, 4, 1, 128, "bf16")   # canvas-only: few query tiles
    assert "transpose_v" not in b.Plan(big, b.FLAG_FWD_VT).kernel_names(False)


def _bwd_launch(meta, flags):
    """dK/dV items in launch order as (XCD, class, cost, record); None for empty slots."""
    import bisect
    rec = decode(b.Plan(meta, flags).host_blob())
    G = meta.num_q_heads // meta.num_kv_heads
    qct = 64 // G
    cpc = -(-meta.block_size // qct)
    koff = meta.k_offsets()
    out = []
    for i, it in enumerate(rec["bwd"]):
        if it[0] < 0:
            out.append(None)
            continue
        kt = rec["ktiles"][it[0]]
        nall = -(-int(kt[4]) // qct) + int(kt[7]) * cpc
        cost = min(int(it[3]), nall) - min(int(it[2]), nall)
        seg = bisect.bisect_right(koff, int(kt[0])) - 1
        out.append((i % 8, (seg, int(it[1]) % meta.num_kv_heads), cost, tuple(int(x) for x in it)))
    return rec, out


def test_dkdv_runs_flag_reorders_the_dkdv_items_only():
    """BD_ATTN_FLAG_DKDV_RUNS: the same dK/dV items on the same XCDs, only launched
    in runs of one (segment, kv head) class; every other record is unchanged."""
    meta = config_meta(3, np.random.default_rng(3))
    rec0, d0 = _bwd_launch(meta, 0)
    rec1, d1 = _bwd_launch(meta, b.FLAG_DKDV_RUNS)
    for name in ("qtiles", "fwd", "split", "merge", "dq", "ktiles", "canvq", "bmerge"):
        assert np.array_equal(rec0[name], rec1[name]), name
    live0 = [x for x in d0 if x is not None]
    live1 = [x for x in d1 if x is not None]
    assert sorted(x[3] for x in live0) == sorted(x[3] for x in live1)
    assert [x[3] for x in live0] != [x[3] for x in live1]
    switches = []
    for x in range(8):
        s0 = [e for e in d0 if e is not None and e[0] == x]
        s1 = [e for e in d1 if e is not None and e[0] == x]
        assert sorted(e[3] for e in s0) == sorted(e[3] for e in s1)      # same XCD
        assert s1[0][2] == max(e[2] for e in s1)                          # opens with the largest
        for cls in {e[1] for e in s1}:                                    # a class largest first
            costs = [e[2] for e in s1 if e[1] == cls]
            assert costs == sorted(costs, reverse=True)
        switches.append((sum(a[1] != c[1] for a, c in zip(s0, s0[1:])),
                         sum(a[1] != c[1] for a, c in zip(s1, s1[1:]))))
    # runs of up to 8 tiles of a class: far fewer class switches on each XCD
    assert all(n1 * 2 < n0 for n0, n1 in switches), switches


def test_dkdv_runs_flag_keeps_single_segment_order():
    # one segment: each XCD holds one class, whose items are already in launch order
    meta = config_meta(4, np.random.default_rng(4))
    assert b.Plan(meta, b.FLAG_DKDV_RUNS).host_blob() == b.Plan(meta).host_blob()


@pytest.mark.parametrize("k", [3, 5])
def test_dkdv_runs_flag_has_no_effect_without_xcd_grouping(k):
    # the runs are formed inside each XCD's list; with NO_XCD there is one global order
    meta = config_meta(k, np.random.default_rng(k))
    assert (b.Plan(meta, b.FLAG_NO_XCD | b.FLAG_DKDV_RUNS).host_blob() ==
            b.Plan(meta, b.FLAG_NO_XCD).host_blob())
