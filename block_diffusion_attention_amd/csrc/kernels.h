// Kernel argument blocks and host-side launchers (one per kernel family).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bd_records.h"

namespace bdattn {

struct FwdArgs {
  const int32_t* qtiles;
  const FwdItem* items;      // direct path: one item per workgroup
  const SplitItem* splits;   // split path: one item per workgroup (else NULL)
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  void* part_o;              // split path: partial O [slot][kQRows][D] bf16
  float* part_lse;           // split path: partial LSE [slot][kQRows] fp32
  const void* vt;            // V transposed, [Hkv][D][tk_pad] (pipelined kernel)
  int tk_pad;
  int hq, hkv, G;
  int grain;                 // step of the clean row limits: block size, or 1 (token-causal)
  float scale_log2;          // softmax scale * log2(e)
  float scale;               // softmax scale
  // list and tensor sizes, read only by the record-checking instantiations
  int64_t tq, tk;            // packed query / key tokens
  int n_qtiles, n_slots;     // query tiles; partial slots of the split path
  bool checks;               // launch the record-checking instantiations (host side)
  // regular split grid (split path; grid_parts = 0: the items are loaded): one query
  // tile whose key range of grid_tiles tiles each kv head cuts into grid_parts parts
  // of grid_tps tiles; workgroup i is part i / Hkv of kv head i % Hkv
  QTile grid_qt;
  int grid_parts, grid_tps, grid_tiles;
};

struct MergeArgs {
  const MergeItem* items;    // one per workgroup, launch order
  const void* part_o;        // [slot][kQRows][D] bf16
  const float* part_lse;     // [slot][kQRows]
  void* o;
  float* lse;
  int hq, G;
  int64_t tq;                // (record checks) packed query tokens
  int n_slots;               // (record checks) partial slots
  bool checks;               // launch the record-checking instantiation (host side)
};

struct BwdArgs {
  const int32_t* qtiles;     // dQ kernel
  const FwdItem* dq_items;
  const int32_t* ktiles;     // dK/dV kernel
  const CanvasQ* canvq;
  const BwdItem* bwd_items;
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  float* delta;              // [Tq, Hq] fp32 (workspace)
  float* lse2;               // [Tq, Hq] fp32 (workspace): LSE * log2(e), written by bwd_pre
  float* dkv_part;           // partial dK/dV slots (workspace): [slot][dK, dV][kKBlock][D] fp32
  const BwdMerge* bmerge;    // merge items of the split key tiles
  void* dq;
  void* dk;
  void* dv;
  int64_t rows_q;            // Tq * Hq
  int hq, hkv, G, B;
  int grain;                 // step of the clean row limits: block size, or 1 (token-causal)
  float scale_log2;
  float scale;
  // list and tensor sizes, read only by the record-checking instantiations
  int64_t tq, tk;
  int n_qtiles, n_ktiles, n_canvq, n_dkv_slots;
  bool checks;               // launch the record-checking instantiations (host side)
};

hipError_t launch_fwd_bf16(const FwdArgs& a, int head_dim, int grid, hipStream_t s);
hipError_t launch_fwd_split_direct(const FwdArgs& a, int head_dim, int grid, hipStream_t s);
hipError_t launch_fwd_split_vt(const FwdArgs& a, int head_dim, int grid, hipStream_t s);
hipError_t launch_merge(const MergeArgs& a, int head_dim, int grid, hipStream_t s);
hipError_t launch_bwd_pre(const BwdArgs& a, int head_dim, bool bf16, hipStream_t s);
hipError_t launch_dkdv_bf16(const BwdArgs& a, int head_dim, bool masked, int grid, hipStream_t s);
hipError_t launch_dq_bf16(const BwdArgs& a, int head_dim, int grid, hipStream_t s);
hipError_t launch_dkdv_merge(const BwdArgs& a, int head_dim, int n_merge, hipStream_t s);

hipError_t launch_transpose_v(const void* v, void* vt, int tk, int tk_pad, int hkv, int head_dim, hipStream_t s);
hipError_t launch_fwd_vt(const FwdArgs& a, int head_dim, int grid, hipStream_t s);

hipError_t launch_fwd_f32(const FwdArgs& a, int head_dim, int grid, hipStream_t s);

hipError_t launch_dkdv_f32(const BwdArgs& a, int head_dim, int grid, hipStream_t s);
hipError_t launch_dq_f32(const BwdArgs& a, int head_dim, int grid, hipStream_t s);

// Workgroups of record-checking launches that rejected a work record on the
// current device since the last reset, one counter per source file, added to
// *count (blocking: waits for all work on the current device).
hipError_t device_errors_fwd(uint64_t* count, bool reset);
hipError_t device_errors_fwd_vt(uint64_t* count, bool reset);
hipError_t device_errors_bwd(uint64_t* count, bool reset);
hipError_t device_errors_dq(uint64_t* count, bool reset);
hipError_t device_errors_f32(uint64_t* count, bool reset);

}  // namespace bdattn
