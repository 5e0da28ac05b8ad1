// Host planner: validates the per-segment metadata and derives the work lists
// (query tiles with their visible key ranges, key tiles with their visible query
// ranges), ordered largest-cost-first and grouped per XCD.
//
// The visibility rule and the range derivation follow the ORL paper, section 3.2
// "Staircase attention kernel" and the appendix D.2 paragraph on the kernel; the
// largest-cost-first order follows section 3.2 "Packed and cost-balanced state
// training" / appendix D.3, applied here to workgroups instead of data-parallel
// groups. Pure C++17, no HIP calls.
#include "planner.h"

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <numeric>
#include <string>

namespace bdattn {

namespace {

constexpr int kNumXcd = 8;
// dK/dV key tiles per run under BD_ATTN_FLAG_DKDV_RUNS (see launch_order).
constexpr int kDkdvRun = 8;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Orders work items for launch: workgroup i is dispatched to XCD i % 8. Items
// of one affinity class (same segment and kv head, i.e. the same K/V or Q/dO
// rows) are kept on one XCD so they share its L2; classes go to XCDs
// largest-total-first; inside an XCD items run largest-cost-first. With run > 1,
// the largest remaining item of an XCD opens a run that also takes the next
// run - 1 largest remaining items of its class, so that items of one class start
// together and read the same rows at about the same time (under the plain order,
// each segment has about one dK/dV key tile per cost level, so the tiles running
// at one time come from different segments). Falls back to one global
// largest-cost-first order when the class split is unbalanced.
// Returns item indices, -1 for empty slots.
std::vector<int32_t> launch_order(const std::vector<int64_t>& cost,
                                  const std::vector<int64_t>& cls, bool xcd_groups, int run = 1) {
  const int64_t n = (int64_t)cost.size();
  std::vector<int32_t> idx(n);
  std::iota(idx.begin(), idx.end(), 0);
  auto by_cost = [&](int32_t a, int32_t b) {
    if (cost[a] != cost[b]) return cost[a] > cost[b];
    if (cls[a] != cls[b]) return cls[a] < cls[b];
    return a < b;
  };
  std::sort(idx.begin(), idx.end(), by_cost);
  if (!xcd_groups || n < 2 * kNumXcd) return idx;

  // class totals
  int64_t ncls = 0;
  for (auto c : cls) ncls = std::max<int64_t>(ncls, c + 1);
  if (ncls < kNumXcd) return idx;
  std::vector<int64_t> tot(ncls, 0);
  int64_t maxc = 0, sum = 0;
  for (int64_t i = 0; i < n; ++i) { tot[cls[i]] += cost[i]; maxc = std::max(maxc, cost[i]); sum += cost[i]; }
  std::vector<int64_t> corder(ncls);
  std::iota(corder.begin(), corder.end(), 0);
  std::sort(corder.begin(), corder.end(), [&](int64_t a, int64_t b) {
    return tot[a] != tot[b] ? tot[a] > tot[b] : a < b; });
  std::vector<int64_t> load(kNumXcd, 0);
  std::vector<int> cx(ncls, 0);
  for (int64_t c : corder) {
    int best = 0;
    for (int x = 1; x < kNumXcd; ++x) if (load[x] < load[best]) best = x;
    cx[c] = best;
    load[best] += tot[c];
  }
  int64_t mx = *std::max_element(load.begin(), load.end());
  double mean = (double)sum / kNumXcd;
  if ((double)mx > 1.03 * mean + (double)maxc) return idx;   // unbalanced: keep global order

  std::vector<std::vector<int32_t>> per(kNumXcd);
  for (int32_t i : idx) per[cx[cls[i]]].push_back(i);       // idx is already cost-sorted
  if (run > 1) {
    // A class lives on one XCD, and both lists keep idx's order, so the first item
    // of a class not yet placed is the XCD's first item not yet placed when it
    // opens a run.
    std::vector<std::vector<int32_t>> of_cls(ncls);
    for (int32_t i : idx) of_cls[cls[i]].push_back(i);
    std::vector<size_t> next(ncls, 0);
    std::vector<char> placed(n, 0);
    for (auto& lst : per) {
      std::vector<int32_t> out;
      out.reserve(lst.size());
      for (int32_t i : lst) {
        if (placed[i]) continue;
        const int64_t c = cls[i];
        for (int taken = 0; taken < run && next[c] < of_cls[c].size(); ++next[c]) {
          const int32_t k = of_cls[c][next[c]];
          if (placed[k]) continue;
          placed[k] = 1;
          out.push_back(k);
          ++taken;
        }
      }
      lst.swap(out);
    }
  }
  size_t rows = 0;
  for (auto& p : per) rows = std::max(rows, p.size());
  std::vector<int32_t> out(rows * kNumXcd, -1);
  for (int x = 0; x < kNumXcd; ++x)
    for (size_t r = 0; r < per[x].size(); ++r) out[r * kNumXcd + x] = per[x][r];
  // drop trailing empty slots
  while (!out.empty() && out.back() < 0) out.pop_back();
  return out;
}

template <class T>
void append_records(std::vector<int32_t>& blob, const std::vector<T>& v, int64_t& off) {
  // 16-byte aligned sections
  while (blob.size() % 4) blob.push_back(0);
  off = (int64_t)blob.size();
  const int32_t* p = reinterpret_cast<const int32_t*>(v.data());
  blob.insert(blob.end(), p, p + v.size() * (sizeof(T) / sizeof(int32_t)));
}

// Sets p.grid_* when the split items follow the regular grid described in
// planner.h (a single query tile, e.g. one request's denoising step). The merge
// items read their slots from their records, which the grid's slot numbering
// matches by construction (slot = index of the raw item = kv head * parts + part).
void find_split_grid(Plan& p, int Hkv, int64_t tps) {
  p.grid_parts = p.grid_tps = p.grid_tiles = 0;
  if (p.qtiles.size() != 1 || tps <= 0) return;
  const QTile& qt = p.qtiles[0];
  const int64_t nt = ceil_div(qt.lim_max, kKTile) + ceil_div(qt.n_own, kKTile);
  const int64_t parts = ceil_div(nt, tps);
  if ((int64_t)p.split_items.size() != parts * Hkv || p.n_split_slots != parts * Hkv) return;
  for (int64_t i = 0; i < parts * Hkv; ++i) {
    const SplitItem& it = p.split_items[i];
    const int64_t kvh = i % Hkv, part = i / Hkv;
    if (it.kvh != kvh || it.kt_begin != part * tps || it.kt_end != std::min(nt, (part + 1) * tps) ||
        it.slot != kvh * parts + part || std::memcmp(&it.qt, &qt, sizeof qt) != 0)
      return;
  }
  p.grid_parts = (int)parts;
  p.grid_tps = (int)tps;
  p.grid_tiles = (int)nt;
}

}  // namespace

bd_attn_status build_plan(const bd_attn_desc* d, Plan* P, std::string* err) {
  if (!d) { *err = "desc is NULL"; return BD_ATTN_EINVAL; }
  const int S = d->num_segments;
  if (S < 1) { *err = "num_segments must be >= 1"; return BD_ATTN_EINVAL; }
  if (!d->ctx_len || !d->canvas_offsets) { *err = "ctx_len and canvas_offsets must not be NULL"; return BD_ATTN_EINVAL; }
  const int B = d->block_size;
  if (B < 1) { *err = "block_size must be >= 1"; return BD_ATTN_EINVAL; }
  if (d->num_q_heads < 1 || d->num_kv_heads < 1) { *err = "head counts must be >= 1"; return BD_ATTN_EINVAL; }
  if (d->num_q_heads % d->num_kv_heads) { *err = "num_q_heads must be a multiple of num_kv_heads"; return BD_ATTN_EINVAL; }
  if (d->dtype != BD_ATTN_BF16 && d->dtype != BD_ATTN_FP32) { *err = "unknown dtype"; return BD_ATTN_EINVAL; }
  if (d->head_dim < 1) { *err = "head_dim must be >= 1"; return BD_ATTN_EINVAL; }
  if (d->head_dim != 64 && d->head_dim != 128) { *err = "head_dim must be 64 or 128"; return BD_ATTN_EUNSUPPORTED; }
  if (!(std::isfinite(d->softmax_scale))) { *err = "softmax_scale must be finite"; return BD_ATTN_EINVAL; }
  const int G = d->num_q_heads / d->num_kv_heads;
  if (G > kMaxGroup) { *err = "group size num_q_heads/num_kv_heads above 32 is not supported"; return BD_ATTN_EUNSUPPORTED; }
  if (d->canvas_offsets[0] != 0) { *err = "canvas_offsets[0] must be 0"; return BD_ATTN_EINVAL; }
  for (int s = 0; s < S; ++s)
    if (d->canvas_offsets[s + 1] < d->canvas_offsets[s]) { *err = "canvas_offsets must be non-decreasing"; return BD_ATTN_EINVAL; }
  const int64_t ncv = d->canvas_offsets[S];
  if (ncv > 0 && !d->canvas_block_idx) { *err = "canvas_block_idx must not be NULL"; return BD_ATTN_EINVAL; }

  Plan& p = *P;
  p.desc = *d;
  p.desc.ctx_len = nullptr; p.desc.ctx_q_begin = nullptr;
  p.desc.canvas_offsets = nullptr; p.desc.canvas_block_idx = nullptr;
  p.desc.block_offset = nullptr;
  p.G = G;
  p.scale = d->softmax_scale > 0.f ? d->softmax_scale : 1.0f / std::sqrt((float)d->head_dim);
  p.ctx.assign(d->ctx_len, d->ctx_len + S);
  p.q0.assign(S, 0);
  if (d->ctx_q_begin) p.q0.assign(d->ctx_q_begin, d->ctx_q_begin + S);
  p.coff.assign(d->canvas_offsets, d->canvas_offsets + S + 1);
  p.cb.assign(d->canvas_block_idx, d->canvas_block_idx + ncv);
  p.off.assign(S, 0);
  if (d->block_offset) p.off.assign(d->block_offset, d->block_offset + S);
  // Clean row limits come in steps of the block size (block-causal) or of one
  // token (token-causal): a clean query at context position t of a segment with
  // grid offset o sees the clean positions below ((t + o) / Bc + 1) * Bc - o.
  const bool causal = (d->flags & BD_ATTN_FLAG_CLEAN_CAUSAL) != 0;
  const int64_t Bc = causal ? 1 : B;
  p.grain = (int)Bc;
  auto clean_lim = [Bc](int64_t t, int64_t o) { return ((t + o) / Bc + 1) * Bc - o; };

  int64_t tq = 0, tk = 0, pairs = 0;
  const int64_t kMaxTok = (int64_t)INT32_MAX / 2;
  for (int s = 0; s < S; ++s) {
    const int64_t C = p.ctx[s], q0 = p.q0[s], o = p.off[s];
    const std::string ss = "[" + std::to_string(s) + "]";
    if (o < 0 || o >= B) { *err = "block_offset" + ss + " must lie in [0, block_size)"; return BD_ATTN_EINVAL; }
    if (C < 0 || (C + o) % B) { *err = "ctx_len" + ss + " must be >= 0 and ctx_len + block_offset a multiple of block_size"; return BD_ATTN_EINVAL; }
    if (q0 < 0 || q0 > C) { *err = "ctx_q_begin" + ss + " must lie in [0, ctx_len]"; return BD_ATTN_EINVAL; }
    const int64_t n = (C + o) / B;
    const int64_t m = p.coff[s + 1] - p.coff[s];
    for (int64_t c = p.coff[s]; c < p.coff[s + 1]; ++c)
      if (p.cb[c] < 0 || p.cb[c] > n) { *err = "canvas_block_idx[" + std::to_string(c) + "] must lie in [0, (ctx_len + block_offset)/block_size]"; return BD_ATTN_EINVAL; }
    tq += (C - q0) + m * B;
    tk += C + m * B;
    if (tq > kMaxTok || tk > kMaxTok) { *err = "packed token count too large"; return BD_ATTN_EINVAL; }
    // visible pairs: a clean query at t sees clean_lim(t) keys (constant over a
    // block when block-causal); canvas b sees max(bB - o, 0) + B
    if (causal) {
      pairs += (C * (C + 1) - q0 * (q0 + 1)) / 2;
    } else {
      for (int64_t j = (q0 + o) / B; j < n; ++j) {
        const int64_t lo = std::max(q0, j * B - o), hi = (j + 1) * B - o;
        if (hi > lo) pairs += (hi - lo) * hi;
      }
    }
    for (int64_t c = p.coff[s]; c < p.coff[s + 1]; ++c)
      pairs += (int64_t)B * (std::max<int64_t>((int64_t)p.cb[c] * B - o, 0) + B);
  }
  if (tq == 0) { *err = "the batch has no query tokens"; return BD_ATTN_EINVAL; }
  if (tq * d->num_q_heads > (int64_t)INT32_MAX || tk * d->num_kv_heads > (int64_t)INT32_MAX) {
    *err = "tensor rows (tokens x heads) must fit in int32"; return BD_ATTN_EINVAL; }
  p.tq = tq; p.tk = tk; p.pairs = pairs;

  const bool xcd = !(d->flags & BD_ATTN_FLAG_NO_XCD);
  const int Hkv = d->num_kv_heads;
  const int QT = std::max(1, kQRows / G);         // tokens per query tile
  p.qt_tokens = QT;

  // ---------------- query tiles (forward, dQ)
  p.qtiles.clear();
  std::vector<int> qtile_seg;
  {
    int64_t qo = 0, ko = 0;
    for (int s = 0; s < S; ++s) {
      const int64_t C = p.ctx[s], q0 = p.q0[s], o = p.off[s];
      const int64_t m = p.coff[s + 1] - p.coff[s];
      // clean queries, tiles of QT tokens that stay inside one block when B >= QT.
      // pos0 is the grid position t + o; the kernels step the first row's limit
      // by Bc at every multiple of Bc crossed from there.
      for (int64_t t = q0; t < C;) {
        int64_t len = std::min<int64_t>(QT, C - t);
        if (B >= QT) len = std::min<int64_t>(len, ((t + o) / B + 1) * B - o - t);
        QTile q{};
        q.q_tok = (int32_t)(qo + (t - q0));
        q.n_tok = (int32_t)len;
        q.k_ctx = (int32_t)ko;
        q.pos0 = (int32_t)(t + o);
        q.lim_min = (int32_t)clean_lim(t, o);
        q.lim_max = (int32_t)clean_lim(t + len - 1, o);
        q.k_own = (int32_t)ko; q.n_own = 0;
        p.qtiles.push_back(q); qtile_seg.push_back(s);
        t += len;
      }
      for (int64_t c = 0; c < m; ++c) {
        const int64_t b = p.cb[p.coff[s] + c];
        for (int64_t t = 0; t < B; t += QT) {
          QTile q{};
          q.q_tok = (int32_t)(qo + (C - q0) + c * B + t);
          q.n_tok = (int32_t)std::min<int64_t>(QT, B - t);
          q.k_ctx = (int32_t)ko;
          q.pos0 = -1;
          q.lim_min = q.lim_max = (int32_t)std::max<int64_t>(b * B - o, 0);
          q.k_own = (int32_t)(ko + C + c * B);
          q.n_own = B;
          p.qtiles.push_back(q); qtile_seg.push_back(s);
        }
      }
      qo += (C - q0) + m * B;
      ko += C + m * B;
    }
  }
  auto tiles_of = [&](const QTile& q) -> int64_t {
    return ceil_div(q.lim_max, kKTile) + ceil_div(q.n_own, kKTile);
  };

  // ---------------- forward items: direct, or split along the key range
  const int64_t nq = (int64_t)p.qtiles.size();
  int64_t total_tiles = 0, max_tiles = 0;
  for (auto& q : p.qtiles) { total_tiles += tiles_of(q); max_tiles = std::max(max_tiles, tiles_of(q)); }
  const int64_t direct_items = nq * Hkv;
  bool split = false;
  int64_t tps = 0;   // key tiles per split
  if (!(d->flags & BD_ATTN_FLAG_NO_SPLIT) && d->dtype == BD_ATTN_BF16) {
    const int64_t want = (d->flags >> 8) & 0xff;     // caller's key tiles per split
    if (d->flags & BD_ATTN_FLAG_FORCE_SPLIT) {
      tps = want > 0 ? want : std::max<int64_t>(1, (max_tiles + 1) / 2);
      split = tps < max_tiles;
    } else if (direct_items < 2 * 256 && max_tiles >= 4) {
      // Short query streams over long key ranges (fewer direct items than two
      // per compute unit): parts of about total / 256 key tiles, so that every
      // compute unit gets one part, each part's loads are all in flight at once
      // and a part's partial result is no larger than the keys it read.
      tps = want > 0 ? want : std::max<int64_t>(1, ceil_div(total_tiles * Hkv, 256));
      split = tps < max_tiles;
    }
  }
  p.split = split;
  p.fwd_items.clear(); p.split_items.clear(); p.merge_items.clear();
  {
    // raw items: (query tile, kv head, key-tile range); on the split path their
    // index is the partial slot, and each (query tile, kv head) has a merge entry
    std::vector<FwdItem> raw;
    std::vector<int64_t> cost, cls;
    struct Merge { int32_t qtile, kvh, first, count; };
    std::vector<Merge> merges;
    for (int64_t i = 0; i < nq; ++i) {
      const int64_t nt = tiles_of(p.qtiles[i]);
      for (int h = 0; h < Hkv; ++h) {
        const int64_t step = split ? tps : nt;
        Merge mg{(int32_t)i, h, (int32_t)raw.size(), 0};
        for (int64_t b0 = 0; b0 < nt; b0 += step) {
          const int64_t b1 = std::min(nt, b0 + step);
          raw.push_back(FwdItem{(int32_t)i, h, (int32_t)b0, (int32_t)b1});
          cost.push_back(b1 - b0 + 1);
          cls.push_back((int64_t)qtile_seg[i] * Hkv + h);
          mg.count++;
        }
        if (split) merges.push_back(mg);
      }
    }
    std::vector<int32_t> ord;
    if (split && nq == 1 && Hkv % kNumXcd == 0 && xcd) {
      // one query tile (a single request's step) and kv heads a multiple of the XCD
      // count: part-major order, workgroup i = part i / Hkv of kv head i % Hkv. It is
      // largest-first (only the last part can be shorter), keeps each kv head's parts
      // on one XCD (i % 8), and is the regular grid whose workgroups need no record
      // (find_split_grid). With fewer kv heads a head's parts would span several XCDs
      // either way, and the plain order measured as fast or faster.
      const int64_t parts = ceil_div(tiles_of(p.qtiles[0]), tps);
      for (int64_t i = 0; i < parts * Hkv; ++i) ord.push_back((int32_t)((i % Hkv) * parts + i / Hkv));
    } else {
      ord = launch_order(cost, cls, xcd);
    }
    if (!split) {
      for (int32_t o : ord) p.fwd_items.push_back(o < 0 ? FwdItem{-1, 0, 0, 0} : raw[o]);
    } else {
      // split workgroups in launch order; workgroup i runs on XCD i % 8, which
      // the merge workgroups of the same (query tile, kv head) then share, so
      // they find the partial results (and the tile's queries) in that L2
      std::vector<int> xcd_of(raw.size(), 0);
      for (size_t i = 0; i < ord.size(); ++i) {
        SplitItem it{};
        it.kvh = -1;
        if (ord[i] >= 0) {
          const FwdItem& r = raw[ord[i]];
          it.qt = p.qtiles[r.qtile];
          it.kvh = r.kvh;
          it.kt_begin = r.kt_begin;
          it.kt_end = r.kt_end;
          it.slot = ord[i];
          xcd_of[ord[i]] = (int)(i % kNumXcd);
        }
        p.split_items.push_back(it);
      }
      // one merge wave per block of the partials' register-order layout: 32 rows
      // (one wave of the part) x 16 columns, for the waves that hold real rows
      const int blocks_per_wave = 2 * (d->head_dim / 32);
      std::vector<std::vector<MergeItem>> per(kNumXcd);
      for (const Merge& mg : merges) {
        const QTile& qt = p.qtiles[mg.qtile];
        const int waves = (int)ceil_div((int64_t)qt.n_tok * G, 32);
        for (int blk = 0; blk < waves * blocks_per_wave; ++blk) {
          MergeItem m{};
          m.qt = qt;
          m.kvh = mg.kvh;
          m.first = mg.first;
          m.count = mg.count;
          m.block = blk;
          per[xcd_of[mg.first]].push_back(m);
        }
      }
      size_t depth = 0;
      for (auto& v : per) depth = std::max(depth, v.size());
      MergeItem empty{};
      empty.kvh = -1;
      p.merge_items.assign(depth * kNumXcd, empty);
      for (int x = 0; x < kNumXcd; ++x)
        for (size_t r = 0; r < per[x].size(); ++r) p.merge_items[r * kNumXcd + x] = per[x][r];
      while (!p.merge_items.empty() && p.merge_items.back().kvh < 0) p.merge_items.pop_back();
      p.n_split_slots = (int64_t)raw.size();
      find_split_grid(p, Hkv, tps);
    }
    // dQ items: every (query tile, kv head), whole key range, same order policy
    p.dq_items.clear();
    std::vector<FwdItem> dq_raw;
    std::vector<int64_t> dcost, dcls;
    for (int64_t i = 0; i < nq; ++i)
      for (int h = 0; h < Hkv; ++h) {
        dq_raw.push_back(FwdItem{(int32_t)i, h, 0, (int32_t)tiles_of(p.qtiles[i])});
        dcost.push_back(tiles_of(p.qtiles[i]) + 1);
        dcls.push_back((int64_t)qtile_seg[i] * Hkv + h);
      }
    const auto dord = launch_order(dcost, dcls, xcd);
    for (int32_t o : dord) p.dq_items.push_back(o < 0 ? FwdItem{-1, 0, 0, 0} : dq_raw[o]);
  }

  // ---------------- key tiles (dK / dV) and canvas-query lists
  p.ktiles.clear(); p.canvq.clear(); p.bwd_items.clear();
  std::vector<int> ktile_seg;
  std::vector<int64_t> kcost;
  {
    int64_t qo = 0, ko = 0;
    for (int s = 0; s < S; ++s) {
      const int64_t C = p.ctx[s], q0 = p.q0[s], o = p.off[s];
      const int64_t m = p.coff[s + 1] - p.coff[s];
      // Key-side positions are grid positions (context position + o): a clean
      // key at grid position P is seen by the canvases with b*B > P and by the
      // clean queries whose grid limit (P_q / Bc + 1) * Bc exceeds P.
      // canvases of the segment sorted by block index, largest first: those
      // visible to a clean key at grid position p0 (b*B > p0) form a prefix.
      std::vector<int64_t> ord(m);
      std::iota(ord.begin(), ord.end(), 0);
      std::stable_sort(ord.begin(), ord.end(), [&](int64_t a, int64_t b) {
        return p.cb[p.coff[s] + a] > p.cb[p.coff[s] + b]; });
      const int32_t cv_first = (int32_t)p.canvq.size();
      for (int64_t c : ord) {
        CanvasQ e{};
        e.q_tok = (int32_t)(qo + (C - q0) + c * B);
        e.n_tok = B;
        e.lim = (int32_t)(p.cb[p.coff[s] + c] * B);
        e.own = 0;
        p.canvq.push_back(e);
      }
      // clean key tiles
      for (int64_t k0 = 0; k0 < C; k0 += kKBlock) {
        KTile t{};
        t.k_tok = (int32_t)(ko + k0);
        t.n_keys = (int32_t)std::min<int64_t>(kKBlock, C - k0);
        t.p0 = (int32_t)(k0 + o);
        // first clean query that can see key k0: the start of its block
        // (block-causal) or k0 itself (token-causal)
        const int64_t cpos = std::max<int64_t>(q0, ((k0 + o) / Bc) * Bc - o);
        t.cq_pos = (int32_t)(cpos + o);
        t.cq_len = (int32_t)std::max<int64_t>(0, C - cpos);
        t.cq_tok = (int32_t)(qo + std::max<int64_t>(0, cpos - q0));
        t.cv_begin = cv_first;
        int32_t cnt = 0;
        for (int64_t c = 0; c < m; ++c) if (p.canvq[cv_first + c].lim > k0 + o) cnt++;
        t.cv_count = cnt;
        p.ktiles.push_back(t); ktile_seg.push_back(s);
        kcost.push_back((int64_t)t.cq_len + (int64_t)cnt * B);
      }
      // canvas key tiles: each canvas' own keys, seen only by that canvas
      for (int64_t c = 0; c < m; ++c) {
        for (int64_t k0 = 0; k0 < B; k0 += kKBlock) {
          CanvasQ e{};
          e.q_tok = (int32_t)(qo + (C - q0) + c * B);
          e.n_tok = B;
          e.lim = 0;
          e.own = 1;
          KTile t{};
          t.k_tok = (int32_t)(ko + C + c * B + k0);
          t.n_keys = (int32_t)std::min<int64_t>(kKBlock, B - k0);
          t.p0 = -1;
          t.cq_tok = (int32_t)qo; t.cq_len = 0; t.cq_pos = 0;
          t.cv_begin = (int32_t)p.canvq.size();
          t.cv_count = 1;
          p.canvq.push_back(e);
          p.ktiles.push_back(t); ktile_seg.push_back(s);
          kcost.push_back(B);
        }
      }
      qo += (C - q0) + m * B;
      ko += C + m * B;
    }
  }
  {
    // dK/dV items: one per (key tile, kv head), over the tile's 64-row query
    // chunks (64/G tokens of one block each; the same count as the kernel's).
    // The kernel runs one workgroup per CU. When a few key tiles see far more
    // chunks than the average CU has to process (the first key tiles of one long
    // context, which every later query sees), the bf16 plan splits their chunk
    // ranges into parts of about that average; the parts write fp32 partial
    // dK/dV that a merge kernel sums in part order (deterministic).
    const int64_t qct = 64 / G;
    const int64_t cpc = ceil_div(B, qct);
    std::vector<int64_t> nch(p.ktiles.size());
    int64_t total = 0;
    for (size_t i = 0; i < p.ktiles.size(); ++i) {
      nch[i] = ceil_div(p.ktiles[i].cq_len, qct) + (int64_t)p.ktiles[i].cv_count * cpc;
      total += nch[i] * Hkv;
    }
    const bool can_split = d->dtype == BD_ATTN_BF16 && !(d->flags & BD_ATTN_FLAG_NO_SPLIT);
    const bool force = (d->flags & BD_ATTN_FLAG_FORCE_SPLIT) != 0;
    // parts of at most 3/4 of the per-workgroup average: the largest-cost-first
    // order then packs them with a short tail (0.89 of the ideal on the staircase
    // workload, against 0.53 unsplit)
    const int64_t cap = std::max<int64_t>(ceil_div(3 * total, 4 * kDkdvResident), 16);
    auto parts_of = [&](int64_t n) -> int64_t {
      if (!can_split || n < 2) return 1;
      if (force) return 2;
      return n > cap ? ceil_div(n, cap) : 1;
    };
    std::vector<BwdItem> raw;
    std::vector<int64_t> cost, cls;
    p.bwd_merge.clear();
    int64_t slots = 0;
    for (size_t i = 0; i < p.ktiles.size(); ++i) {
      const int64_t n = nch[i], np = parts_of(n);
      for (int h = 0; h < Hkv; ++h) {
        if (np == 1) {
          raw.push_back(BwdItem{(int32_t)i, h, 0, INT32_MAX});
          cost.push_back(n + 1);
          cls.push_back((int64_t)ktile_seg[i] * Hkv + h);
          continue;
        }
        p.bwd_merge.push_back(BwdMerge{(int32_t)i, h, (int32_t)slots, (int32_t)np});
        for (int64_t k = 0; k < np; ++k) {
          const int64_t c0 = n * k / np, c1 = n * (k + 1) / np;
          raw.push_back(BwdItem{(int32_t)i, (int32_t)(h + (int64_t)Hkv * (slots + k + 1)), (int32_t)c0, (int32_t)c1});
          cost.push_back(c1 - c0 + 1);
          cls.push_back((int64_t)ktile_seg[i] * Hkv + h);
        }
        slots += np;
      }
    }
    p.n_dkv_slots = slots;
    if ((int64_t)Hkv * (slots + 1) + Hkv > INT32_MAX) { *err = "too many dK/dV partial slots"; return BD_ATTN_EUNSUPPORTED; }
    auto ord = launch_order(cost, cls, xcd, (d->flags & BD_ATTN_FLAG_DKDV_RUNS) ? kDkdvRun : 1);
    for (int32_t o : ord) p.bwd_items.push_back(o < 0 ? BwdItem{-1, 0, 0, 0} : raw[o]);
  }

  // ---------------- serialize (int32 blob, 16-byte aligned sections)
  // Header: magic, version, then (count, offset) of every section in order.
  p.blob.assign(kBlobHeaderInts, 0);
  append_records(p.blob, p.qtiles, p.off_qtiles);
  append_records(p.blob, p.fwd_items, p.off_fwd);
  append_records(p.blob, p.split_items, p.off_split);
  append_records(p.blob, p.merge_items, p.off_merge);
  append_records(p.blob, p.dq_items, p.off_dq);
  append_records(p.blob, p.ktiles, p.off_ktiles);
  append_records(p.blob, p.canvq, p.off_canvq);
  append_records(p.blob, p.bwd_items, p.off_bwd);
  append_records(p.blob, p.bwd_merge, p.off_bmerge);
  while (p.blob.size() % 4) p.blob.push_back(0);
  {
    int32_t* hd = p.blob.data();
    hd[0] = kBlobMagic;
    hd[1] = kBlobVersion;
    const int64_t cnt[kBlobSections] = {
        (int64_t)p.qtiles.size(), (int64_t)p.fwd_items.size(), (int64_t)p.split_items.size(),
        (int64_t)p.merge_items.size(), (int64_t)p.dq_items.size(), (int64_t)p.ktiles.size(),
        (int64_t)p.canvq.size(), (int64_t)p.bwd_items.size(), (int64_t)p.bwd_merge.size()};
    const int64_t off[kBlobSections] = {p.off_qtiles, p.off_fwd, p.off_split, p.off_merge, p.off_dq,
                                        p.off_ktiles, p.off_canvq, p.off_bwd, p.off_bmerge};
    static_assert(2 + 2 * kBlobSections <= kBlobHeaderInts, "blob header too small");
    for (int i = 0; i < kBlobSections; ++i) { hd[2 + 2 * i] = (int32_t)cnt[i]; hd[3 + 2 * i] = (int32_t)off[i]; }
  }

  const int64_t D = d->head_dim;
  const int64_t Hq = d->num_q_heads;
  // forward workspace: [V transposed (pipelined path)] [partial O fp32] [partial LSE]
  // The forward through a transposed V copy (a pre-pass writing V^T once per
  // call) is taken only on request: with swizzled row-major K/V tiles, the direct
  // kernel's transposing LDS reads of V measured faster than the copy plus its
  // launch on every workload here.
  // Its V^T tiles are read with 32-bit byte offsets within a kv head's rows of
  // tk_pad keys (up to D - 1 rows from a tile's start), so very long key streams
  // take the direct kernel.
  p.tk_pad = ceil_div(tk, 64) * 64 + 64;
  p.use_vt = !(d->flags & BD_ATTN_FLAG_FWD_DIRECT) && (d->flags & BD_ATTN_FLAG_FWD_VT) &&
             d->dtype == BD_ATTN_BF16 && B % 8 == 0 &&
             (int64_t)d->head_dim * p.tk_pad * 2 < ((int64_t)1 << 31);
  int64_t off = 0;
  p.off_ws_vt = 0;
  if (p.use_vt) off = ceil_div((int64_t)Hkv * D * p.tk_pad * 2, 256) * 256;
  p.off_ws_part = off;
  if (split) {
    // partial O in bf16 (normalized by the part's own row sums), partial LSE fp32
    const int64_t nsplit = p.n_split_slots;
    p.off_ws_lse = off + ceil_div(nsplit * kQRows * D * 2, 256) * 256;
    off = p.off_ws_lse + nsplit * kQRows * 4;
  }
  p.ws_fwd = (size_t)off;
  // dK/dV without per-score limits: a wave's 32 keys start at a grid position
  // that is a multiple of 32 (grid offset a multiple of 32); if every row limit
  // is a multiple of 32 (block-causal, block size a multiple of 32), every 64-row
  // query chunk lies inside one block (64 / G tokens dividing B, query ranges
  // starting at block boundaries) and no chunk is partial (B * G a multiple of
  // 64), each (chunk, wave) pair is seen either whole or not at all.
  {
    const int qct = 64 / G;
    bool aligned = !causal && B % 32 == 0 && 64 % G == 0 && B % qct == 0;
    for (int s = 0; s < S && aligned; ++s) aligned = (p.q0[s] + p.off[s]) % B == 0 && p.off[s] % 32 == 0;
    p.dkdv_masked = !aligned;
  }
  p.off_ws_lse2 = ceil_div(tq * Hq * 4, 256) * 256;          // delta [Tq, Hq] fp32, then LSE*log2(e)
  p.off_ws_dkv = 2 * p.off_ws_lse2;                          // then the partial dK/dV slots
  p.ws_bwd = (size_t)(p.off_ws_dkv + p.n_dkv_slots * 2 * kKBlock * D * 4);
  p.checks = (d->flags & BD_ATTN_FLAG_DEBUG_CHECKS) != 0;
  if (d->flags & (BD_ATTN_FLAG_CHECK_PLAN | BD_ATTN_FLAG_DEBUG_CHECKS)) {
    std::string why;
    if (check_blob(p, p.blob.data(), p.blob.size(), &why) != BD_ATTN_OK) {
      *err = "plan self-check failed: " + why;
      return BD_ATTN_EINVAL;
    }
  }
  return BD_ATTN_OK;
}

namespace {

// Bounds of one query tile as the forward / dQ kernels read it: its rows, its
// clean key range and its own canvas keys all inside the packed tensors.
bool qtile_ok(const Plan& p, const QTile& t, std::string* why) {
  const int64_t rows = (int64_t)t.n_tok * p.G;
  if (t.q_tok < 0 || t.n_tok < 1 || rows > kQRows || (int64_t)t.q_tok + t.n_tok > p.tq) {
    *why = "query rows outside [0, Tq) or more than a tile";
    return false;
  }
  if (t.lim_min < 0 || t.lim_min > t.lim_max || t.k_ctx < 0 || (int64_t)t.k_ctx + t.lim_max > p.tk) {
    *why = "clean key range outside [0, Tk)";
    return false;
  }
  if (t.n_own < 0 || (t.n_own > 0 && (t.k_own < 0 || (int64_t)t.k_own + t.n_own > p.tk))) {
    *why = "own canvas keys outside [0, Tk)";
    return false;
  }
  return true;
}

// Key tiles a query tile's list holds: its clean range, then its own keys.
int64_t qtile_key_tiles(const QTile& t) { return ceil_div(t.lim_max, kKTile) + ceil_div(t.n_own, kKTile); }

bool key_range_ok(const QTile& t, int32_t b, int32_t e) {
  return b >= 0 && b <= e && e <= qtile_key_tiles(t);
}

}  // namespace

bd_attn_status check_blob(const Plan& p, const int32_t* blob, size_t n_ints, std::string* why) {
  const int Hkv = p.desc.num_kv_heads;
  char buf[160];
  auto bad = [&](const char* sec, int64_t i, const std::string& what) {
    std::snprintf(buf, sizeof buf, "%s record %lld: ", sec, (long long)i);
    *why = buf + what;
    return BD_ATTN_EINVAL;
  };
  if (!blob || n_ints < (size_t)kBlobHeaderInts) { *why = "blob shorter than its header"; return BD_ATTN_EINVAL; }
  if (blob[0] != kBlobMagic || blob[1] != kBlobVersion) { *why = "bad blob magic or version"; return BD_ATTN_EINVAL; }
  static const char* names[kBlobSections] = {"qtiles", "fwd", "split", "merge", "dq",
                                             "ktiles", "canvq", "bwd", "bmerge"};
  static const int width[kBlobSections] = {8, 4, 16, 16, 4, 8, 4, 4, 4};
  const int64_t expect[kBlobSections] = {
      (int64_t)p.qtiles.size(), (int64_t)p.fwd_items.size(), (int64_t)p.split_items.size(),
      (int64_t)p.merge_items.size(), (int64_t)p.dq_items.size(), (int64_t)p.ktiles.size(),
      (int64_t)p.canvq.size(), (int64_t)p.bwd_items.size(), (int64_t)p.bwd_merge.size()};
  const int32_t* sec[kBlobSections];
  for (int i = 0; i < kBlobSections; ++i) {
    const int64_t cnt = blob[2 + 2 * i], off = blob[3 + 2 * i];
    if (cnt != expect[i]) return bad(names[i], -1, "record count differs from the plan's");
    if (off < kBlobHeaderInts || off % 4 || off + cnt * width[i] > (int64_t)n_ints)
      return bad(names[i], -1, "section outside the blob or misaligned");
    sec[i] = blob + off;
  }
  const int64_t nq = expect[0], nkt = expect[5], ncv = expect[6];
  const QTile* qt = reinterpret_cast<const QTile*>(sec[0]);
  std::string w;
  for (int64_t i = 0; i < nq; ++i)
    if (!qtile_ok(p, qt[i], &w)) return bad("qtiles", i, w);
  for (int s = 1; s <= 4; s += 3) {   // fwd, dq: FwdItem lists
    const FwdItem* it = reinterpret_cast<const FwdItem*>(sec[s]);
    for (int64_t i = 0; i < expect[s]; ++i) {
      if (it[i].qtile < 0) continue;   // empty launch slot
      if (it[i].qtile >= nq) return bad(names[s], i, "query tile index outside its section");
      if (it[i].kvh < 0 || it[i].kvh >= Hkv) return bad(names[s], i, "kv head out of range");
      if (!key_range_ok(qt[it[i].qtile], it[i].kt_begin, it[i].kt_end))
        return bad(names[s], i, "key tile range outside the query tile's list");
    }
  }
  {
    const SplitItem* it = reinterpret_cast<const SplitItem*>(sec[2]);
    for (int64_t i = 0; i < expect[2]; ++i) {
      if (it[i].kvh < 0) continue;
      if (it[i].kvh >= Hkv) return bad("split", i, "kv head out of range");
      if (!qtile_ok(p, it[i].qt, &w)) return bad("split", i, w);
      if (!key_range_ok(it[i].qt, it[i].kt_begin, it[i].kt_end))
        return bad("split", i, "key tile range outside the query tile's list");
      if (it[i].slot < 0 || it[i].slot >= p.n_split_slots) return bad("split", i, "partial slot out of range");
    }
    const MergeItem* mt = reinterpret_cast<const MergeItem*>(sec[3]);
    const int blocks = 4 * (p.desc.head_dim / 32) * 2;
    for (int64_t i = 0; i < expect[3]; ++i) {
      if (mt[i].kvh < 0) continue;
      if (mt[i].kvh >= Hkv) return bad("merge", i, "kv head out of range");
      if (!qtile_ok(p, mt[i].qt, &w)) return bad("merge", i, w);
      if (mt[i].first < 0 || mt[i].count < 1 || (int64_t)mt[i].first + mt[i].count > p.n_split_slots)
        return bad("merge", i, "partial slots out of range");
      if (mt[i].block < 0 || mt[i].block >= blocks) return bad("merge", i, "partial block out of range");
    }
  }
  const KTile* kt = reinterpret_cast<const KTile*>(sec[5]);
  for (int64_t i = 0; i < nkt; ++i) {
    const KTile& t = kt[i];
    if (t.k_tok < 0 || t.n_keys < 1 || t.n_keys > kKBlock || (int64_t)t.k_tok + t.n_keys > p.tk)
      return bad("ktiles", i, "keys outside [0, Tk) or more than a tile");
    if (t.cq_len < 0 || (t.cq_len > 0 && (t.cq_tok < 0 || (int64_t)t.cq_tok + t.cq_len > p.tq)))
      return bad("ktiles", i, "clean query range outside [0, Tq)");
    if (t.cv_begin < 0 || t.cv_count < 0 || (int64_t)t.cv_begin + t.cv_count > ncv)
      return bad("ktiles", i, "canvas-query entries outside their section");
  }
  const CanvasQ* cv = reinterpret_cast<const CanvasQ*>(sec[6]);
  for (int64_t i = 0; i < ncv; ++i)
    if (cv[i].q_tok < 0 || cv[i].n_tok != p.desc.block_size || (int64_t)cv[i].q_tok + cv[i].n_tok > p.tq ||
        cv[i].lim < 0 || (cv[i].own != 0 && cv[i].own != 1))
      return bad("canvq", i, "not one whole canvas of rows in [0, Tq), or bad limit");
  const BwdItem* bt = reinterpret_cast<const BwdItem*>(sec[7]);
  for (int64_t i = 0; i < expect[7]; ++i) {
    if (bt[i].ktile < 0) continue;
    if (bt[i].ktile >= nkt) return bad("bwd", i, "key tile index outside its section");
    if (bt[i].kvh_slot < 0) return bad("bwd", i, "negative kv head / slot");
    const int64_t slot = bt[i].kvh_slot / Hkv - 1;
    if (slot >= p.n_dkv_slots) return bad("bwd", i, "partial dK/dV slot out of range");
    if (bt[i].c_begin < 0 || bt[i].c_begin > bt[i].c_end) return bad("bwd", i, "bad chunk range");
  }
  const BwdMerge* bm = reinterpret_cast<const BwdMerge*>(sec[8]);
  for (int64_t i = 0; i < expect[8]; ++i) {
    if (bm[i].ktile < 0 || bm[i].ktile >= nkt) return bad("bmerge", i, "key tile index outside its section");
    if (bm[i].kvh < 0 || bm[i].kvh >= Hkv) return bad("bmerge", i, "kv head out of range");
    if (bm[i].first < 0 || bm[i].count < 1 || (int64_t)bm[i].first + bm[i].count > p.n_dkv_slots)
      return bad("bmerge", i, "partial dK/dV slots out of range");
  }
  return BD_ATTN_OK;
}

}  // namespace bdattn
