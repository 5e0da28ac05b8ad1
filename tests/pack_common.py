"""From a packer result to the attention metadata of one data-parallel group."""
from __future__ import annotations

from block_diffusion_attention_amd.workloads import Meta


def group_meta(p, g, clean_len, block_offset, state_block, B, hq, hkv, d, dtype):
    """The attention metadata of group g: its rows, in assignment order, as
    replay segments (every clean token a query), each row's states as canvases."""
    rows = p["group_rows"][p["group_row_offsets"][g]:p["group_row_offsets"][g + 1]]
    ctx, cvs, offs = [], [], []
    for r in rows:
        ctx.append(int(p["row_ctx_len"][r]))
        sts = p["row_states"][p["row_state_offsets"][r]:p["row_state_offsets"][r + 1]]
        cvs.append([int(state_block[s]) for s in sts])
        resp = int(p["row_resp"][r])
        o = block_offset[resp] if block_offset is not None else 0
        offs.append(int(o) if p["row_ctx_len"][r] > 0 else 0)   # no clean token: no grid to shift
    return Meta(ctx, [0] * len(ctx), cvs, B, hq, hkv, d, dtype, block_offset=offs)
