"""Host check of the swizzled row-major LDS tile layout used by the bf16 kernels
(the formulas of SwLane / SwFetch / swz in csrc/kcommon.h, restated here).

A tile holds 64 rows of D bf16 in 16-byte chunks; chunk c of row r sits in slot
r * CH + (c ^ sw(r)). Checked for both head sizes:
  * a copy instruction m (lane l -> slot 64 m + l) places every (row, chunk) once;
  * the per-lane natural and transposed operand offsets address the intended
    (row, chunk);
  * no bank conflicts under the LDS pass model (16 lanes per pass for 16-byte
    reads, 32 lanes per pass for the 8-byte transposing reads; 64 banks x 4 B).
"""
import pytest


def sw(r, d):
    if d == 128:
        return ((r & 3) << 2) | ((r >> 2) & 3)
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3)


@pytest.mark.parametrize("d", [64, 128])
def test_swizzled_tile_layout(d):
    ch = d // 8
    held = {}
    for m in range(ch):
        for lane in range(64):
            slot = 64 * m + lane
            r, p = slot // ch, slot % ch
            held[slot] = (r, p ^ sw(r, d))
    assert sorted(held.values()) == sorted((r, c) for r in range(64) for c in range(ch))
    where = {v: k for k, v in held.items()}

    # natural operand: lane -> row rbase + lane%32, chunk 2 kk + lane/32
    for rbase in (0, 32):
        for kk in range(d // 16):
            slots = []
            for lane in range(64):
                j, h = lane & 31, lane >> 5
                a = 16 * (j * ch + ((2 * kk + h) ^ sw(j, d)))
                assert 16 * rbase * ch + a == 16 * where[(rbase + j, 2 * kk + h)]
                slots.append((16 * rbase * ch + a) // 16)
            for p0 in range(0, 64, 16):
                assert len({s % 16 for s in slots[p0:p0 + 16]}) == 16

    # transposed operand: lane -> row row0 + rl + 8 jj, chunk 4 db + cl, 8-byte half s & 1
    for row0 in (0, 16, 32, 48):
        for db in range(d // 32):
            for jj in (0, 1):
                offs = []
                for lane in range(64):
                    g, s = lane >> 4, lane & 15
                    cl = 2 * (g & 1) + ((s & 3) >> 1)
                    rl = 4 * (g >> 1) + (s >> 2)
                    w = sw(rl + 8 * jj, d)
                    t = 16 * ((rl + 8 * jj) * ch + 4 * (db ^ (w >> 2)) + (cl ^ (w & 3))) + 8 * (s & 1)
                    assert 16 * row0 * ch + t == 16 * where[(row0 + rl + 8 * jj, 4 * db + cl)] + 8 * (s & 1)
                    offs.append(16 * row0 * ch + t)
                for p0 in (0, 32):
                    banks = {((o // 4) + b) % 64 for o in offs[p0:p0 + 32] for b in range(2)}
                    assert len(banks) == 64
