// Host-side plan: validated metadata plus the serialized work lists.
#pragma once
#include <stdint.h>

#include <string>
#include <vector>

#include "../../include/bd_attn.h"
#include "bd_records.h"

namespace bdattn {

struct Plan {
  bd_attn_desc desc{};          // scalar fields only (pointers cleared)
  int G = 1;                    // query heads per kv head
  int qt_tokens = 1;            // tokens per query tile
  float scale = 1.f;
  std::vector<int32_t> ctx, q0, coff, cb, off;   // off: block-grid offset per segment
  int grain = 1;                // step of the clean row limits: B, or 1 (token-causal)
  int64_t tq = 0, tk = 0, pairs = 0;

  std::vector<QTile> qtiles;
  bool split = false;
  std::vector<FwdItem> fwd_items;    // direct path: launch order (empty on the split path)
  std::vector<SplitItem> split_items;  // split path: launch order
  std::vector<MergeItem> merge_items;  // split path: launch order
  int64_t n_split_slots = 0;         // partial slots of the split path
  // Regular split grid (0 parts: none): one query tile whose key range of grid_tiles
  // key tiles every kv head cuts into grid_parts parts of grid_tps tiles; split item
  // i is (kv head i % Hkv, part i / Hkv) writing slot kv head * parts + part. Its
  // split workgroups compute their work from their index instead of loading their
  // record (one dependent memory round trip less before the first K/V request).
  int grid_parts = 0, grid_tps = 0, grid_tiles = 0;
  std::vector<FwdItem> dq_items;     // launch order
  std::vector<KTile> ktiles;
  std::vector<CanvasQ> canvq;
  std::vector<BwdItem> bwd_items;    // launch order
  std::vector<BwdMerge> bwd_merge;   // split key tiles
  int64_t n_dkv_slots = 0;           // partial dK/dV slots of the split key tiles

  std::vector<int32_t> blob;         // device metadata image
  int64_t off_qtiles = 0, off_fwd = 0, off_split = 0, off_merge = 0, off_dq = 0,
          off_ktiles = 0, off_canvq = 0, off_bwd = 0, off_bmerge = 0;   // int32 offsets into blob
  size_t ws_fwd = 0, ws_bwd = 0;
  bool checks = false;               // launch the record-checking kernel instantiations
  bool use_vt = false;               // bf16 forward through the transposed V copy (B % 8 == 0)
  bool dkdv_masked = true;           // dK/dV needs per-score row limits (see build_plan)
  int64_t tk_pad = 0;                // row length of the transposed V copy
  int64_t off_ws_vt = 0;             // byte offsets in the forward workspace: V transposed,
  int64_t off_ws_part = 0;           // partial O (bf16 or fp32, the plan's dtype),
  int64_t off_ws_lse = 0;            // partial LSE (fp32)
  int64_t off_ws_lse2 = 0;           // byte offset of LSE*log2(e) in the backward workspace
  int64_t off_ws_dkv = 0;            // byte offset of the partial dK/dV slots (fp32)
};

// Validates desc and fills *plan. On error returns a non-OK status and sets *err.
bd_attn_status build_plan(const bd_attn_desc* desc, Plan* plan, std::string* err);

// Checks a serialized work-list image against the plan it claims to belong to:
// header, section counts and bounds, and that every index a kernel follows
// (query / key tile, canvas-query entry, kv head, key tile range, partial slot)
// and every token range lies inside its section or tensor. EINVAL + *why on the
// first violation.
bd_attn_status check_blob(const Plan& plan, const int32_t* blob, size_t n_ints, std::string* why);

}  // namespace bdattn

struct bd_attn_plan_s {
  bdattn::Plan p;
};
