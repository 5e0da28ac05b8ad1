// Work-list records shared by the host planner and the gfx950 kernels.
//
// Visibility is never stored as a mask: a query tile carries the ranges of keys
// it can see and a key tile the ranges of queries that can see it, both derived
// from the per-segment metadata (ORL paper, appendix D.2 paragraph on the
// kernel: visible key ranges come from per-document metadata, invisible tiles
// are skipped, the predicate is applied only inside boundary tiles; dK/dV use
// valid query ranges per key tile).
//
// Row limit. Every query row r has a limit L(r) on the context positions of the
// clean keys it sees (positions p < L(r)). With the segment's block-grid offset o
// (context position t lies at grid position t + o, in block (t + o) / B) and the
// grain Bc (B for block-causal clean rows, 1 for token-causal ones):
//   clean query at context position t : L = ((t + o) / Bc + 1) * Bc - o
//   query of a canvas at block index b: L = max(b * B - o, 0)   (blocks before b)
// and a canvas query additionally sees the B keys of its own canvas. The query
// tiles carry context-position limits; the key-side records (KTile, CanvasQ)
// work in grid positions, where the same rule reads P_key < (P_q / Bc + 1) * Bc
// and P_key < b * B.
#pragma once
#include <stdint.h>

namespace bdattn {

// Query tile: up to kQRows rows, row r = token (r / G) x head (r % G) of one kv head.
constexpr int kQRows = 128;
// Forward / dQ key tile (keys per main-loop step).
constexpr int kKTile = 64;
// dK/dV: keys per workgroup (4 waves of 32 keys each).
constexpr int kKBlock = 128;
// dK/dV workgroups resident at once (one per CU of a 256-CU device); the planner
// splits key tiles whose chunk count is far above the per-workgroup average.
constexpr int kDkdvResident = 256;
// Largest supported group size (query heads per kv head).
constexpr int kMaxGroup = 32;

// Serialized plan: a header of kBlobHeaderInts int32 (magic, format version,
// then count and int32 offset of each section: query tiles, forward items,
// split-forward items, merge items, dQ items, key tiles, canvas-query entries,
// dK/dV items, dK/dV merge items), followed by the sections, each 16-byte
// aligned.
constexpr int kBlobHeaderInts = 32;
constexpr int kBlobVersion = 3;
constexpr int kBlobSections = 9;
constexpr int32_t kBlobMagic = 0x62646174;   // "bdat"

struct QTile {         // 8 x int32
  int32_t q_tok;       // first packed query token
  int32_t n_tok;       // tokens in the tile (>= 1)
  int32_t k_ctx;       // packed index of the segment's first clean key
  int32_t pos0;        // grid position of the first token, or -1 for a canvas tile
  int32_t lim_max;     // clean keys [k_ctx, k_ctx + lim_max) may be visible to some row
  int32_t lim_min;     // limit of the first row: every row sees the clean keys below it
  int32_t k_own;       // packed index of the canvas' own keys (canvas tile)
  int32_t n_own;       // own canvas keys (B for a canvas tile, 0 for a clean tile)
};

struct FwdItem {       // 4 x int32: one workgroup of the forward / dQ kernels
  int32_t qtile;       // index into the query-tile list, or -1 for an empty slot
  int32_t kvh;         // kv head
  int32_t kt_begin;    // first key tile (tiles of range 1, then of range 2)
  int32_t kt_end;      // one past the last key tile
};

// Forward split path (short query streams over long key ranges): the key range
// of a (query tile, kv head) is cut into parts of a few key tiles; each part is
// one workgroup that writes a partial result (bf16 O normalized by its own row
// sums, fp32 LSE) into its slot, and a merge kernel combines the slots.
// Both record kinds carry a copy of their query tile, so one scalar load of
// 16 dwords gives a workgroup everything it needs; both lists are in launch
// order (empty launch slots have kvh = -1).
struct SplitItem {     // 16 x int32: one workgroup of the split forward
  QTile qt;            // the query tile
  int32_t kvh;         // kv head, or -1 for an empty launch slot
  int32_t kt_begin;    // key tiles [kt_begin, kt_end) of the tile's list
  int32_t kt_end;
  int32_t slot;        // partial slot written
  int32_t pad[4];
};

struct MergeItem {     // 16 x int32: one workgroup of the merge kernel
  QTile qt;            // the query tile
  int32_t kvh;         // kv head, or -1 for an empty launch slot
  int32_t first;       // first partial slot of the tile's parts
  int32_t count;       // consecutive slots, one per part, in key order
  int32_t block;       // partial block merged: split wave w, 32-column block db and
                       // 16-column pair p as (w * (D / 32) + db) * 2 + p
  int32_t pad[4];
};

struct KTile {         // 8 x int32
  int32_t k_tok;       // first packed key token
  int32_t n_keys;      // keys in the tile (1..kKBlock)
  int32_t p0;          // grid position of the first key, or -1 for canvas keys
  int32_t cq_tok;      // first packed query token of the clean query range
  int32_t cq_len;      // clean query tokens that may see the tile (0 if none)
  int32_t cq_pos;      // grid position of cq_tok
  int32_t cv_begin;    // first entry of the canvas-query list
  int32_t cv_count;    // canvas-query entries that may see the tile
};

struct CanvasQ {       // 4 x int32
  int32_t q_tok;       // first packed query token of the canvas
  int32_t n_tok;       // B
  int32_t lim;         // b * B: grid positions of the clean keys visible to the canvas
  int32_t own;         // 1 for the entry of a canvas key tile (sees all of the tile)
};

struct BwdItem {       // 4 x int32: one workgroup of the dK/dV kernel
  int32_t ktile;       // index into the key-tile list, or -1 for an empty slot
  int32_t kvh_slot;    // kv head + Hkv * (partial slot + 1); slot -1: the item covers
                       // all of the tile's chunks and writes dK/dV itself
  int32_t c_begin;     // chunk range [c_begin, min(c_end, chunks)) in visiting order
  int32_t c_end;
};

struct BwdMerge {      // 4 x int32: sum of the partial dK/dV of one split key tile
  int32_t ktile;
  int32_t kvh;
  int32_t first;       // first partial slot
  int32_t count;       // consecutive partial slots, summed in slot order
};

// Partial O of a split part is stored in the order the forward kernel's
// registers hold it, so every store instruction writes 1 KiB contiguously:
// slot s, wave w (rows 32 w .. 32 w + 31), 32-column block db, pair p of
// 8-column groups, lane l = j + 32 h (row 32 w + j) -> 8 bf16 at element
//   ((s * 4 + w) * (D / 32) * 2 + db * 2 + p) * 512 + 8 l,
// holding columns 32 db + 16 p + 4 h + e and 32 db + 16 p + 8 + 4 h + e
// (e = 0..3). One merge wave per (part block w, db, p): 32 rows x 16 columns.
constexpr int kMergeThreads = 64;

static_assert(sizeof(QTile) == 32, "QTile layout");
static_assert(sizeof(SplitItem) == 64 && sizeof(MergeItem) == 64, "split record layout");
static_assert(sizeof(KTile) == 32, "KTile layout");

}  // namespace bdattn
