// Host packer: builds replay rows from captured denoising states and assigns
// them to data-parallel groups, largest estimated cost first.
//
// Follows the ORL paper, section 3.2 "Packed and cost-balanced state training"
// and appendix D.3. What this file does: for every (response, step) pair it emits
// one row that stores the response's clean tokens a single time and appends, as
// canvases at their block indices, the captured states of that step; the canvases
// then attend to the shared clean prefix instead of carrying copies of it. Rows of
// different responses become separate documents of one packed sequence (no
// attention across them). Each row gets a cost estimate, a weighted sum of its
// token count, its supervised positions and its KV pages, and rows are handed to
// the data-parallel groups in decreasing cost order, each to the group with the
// least cost so far (ties broken by index, so the result is deterministic). Every
// state, and every label it carries, lands in exactly one row. Pure C++17, no HIP
// calls.
#include "packer.h"

#include <algorithm>
#include <numeric>
#include <string>
#include <utility>

namespace bdattn {

bd_attn_status build_pack(const bd_pack_desc* d, bd_pack_out* out, std::string* err) {
  if (!d || !out) { *err = "desc and out must not be NULL"; return BD_ATTN_EINVAL; }
  const int R = d->num_responses, N = d->num_states, G = d->num_groups, B = d->block_size;
  if (R < 1) { *err = "num_responses must be >= 1"; return BD_ATTN_EINVAL; }
  if (N < 0) { *err = "num_states must be >= 0"; return BD_ATTN_EINVAL; }
  if (G < 1) { *err = "num_groups must be >= 1"; return BD_ATTN_EINVAL; }
  if (B < 1) { *err = "block_size must be >= 1"; return BD_ATTN_EINVAL; }
  if (d->w_tokens < 0 || d->w_supervised < 0 || d->w_pages < 0) {
    *err = "cost weights must be >= 0"; return BD_ATTN_EINVAL; }
  if (!d->clean_len) { *err = "clean_len must not be NULL"; return BD_ATTN_EINVAL; }
  if (N > 0 && (!d->state_resp || !d->state_block || !d->state_step)) {
    *err = "state_resp, state_block and state_step must not be NULL"; return BD_ATTN_EINVAL; }
  if (!out->state_row || !out->row_resp || !out->row_step || !out->row_ctx_len || !out->row_group ||
      !out->row_cost || !out->row_state_offsets || !out->row_states || !out->group_row_offsets ||
      !out->group_rows || !out->group_cost) {
    *err = "every output array must be given"; return BD_ATTN_EINVAL; }

  std::vector<int64_t> off(R, 0);
  for (int r = 0; r < R; ++r) {
    const int64_t C = d->clean_len[r], o = d->block_offset ? d->block_offset[r] : 0;
    const std::string rs = "[" + std::to_string(r) + "]";
    if (o < 0 || o >= B) { *err = "block_offset" + rs + " must lie in [0, block_size)"; return BD_ATTN_EINVAL; }
    if (C < 0 || (C + o) % B) { *err = "clean_len" + rs + " must be >= 0 and clean_len + block_offset a multiple of block_size"; return BD_ATTN_EINVAL; }
    off[r] = o;
  }
  auto bad = [err](const char* field, int i, const char* rule) {
    *err = std::string(field) + "[" + std::to_string(i) + "] " + rule;
    return BD_ATTN_EINVAL;
  };
  for (int i = 0; i < N; ++i) {
    const int r = d->state_resp[i];
    if (r < 0 || r >= R) return bad("state_resp", i, "must lie in [0, num_responses)");
    const int64_t nb = (d->clean_len[r] + off[r]) / B;
    if (d->state_block[i] < 0 || d->state_block[i] > nb)
      return bad("state_block", i, "must lie in [0, (clean_len + block_offset)/block_size]");
    if (d->state_step[i] < 0) return bad("state_step", i, "must be >= 0");
    if (d->state_supervised && (d->state_supervised[i] < 0 || d->state_supervised[i] > B))
      return bad("state_supervised", i, "must lie in [0, block_size]");
    if (d->state_pages && d->state_pages[i] < 0) return bad("state_pages", i, "must be >= 0");
  }

  // rows: one per (response, step) present, numbered in (response, step) order;
  // a row's states keep their input order. States are bucketed by response
  // (counting sort, stable), each bucket ordered by step (stable), and every run
  // of one (response, step) is a row.
  std::vector<int32_t> rstart(R + 1, 0);
  for (int i = 0; i < N; ++i) rstart[d->state_resp[i] + 1]++;
  for (int r = 0; r < R; ++r) rstart[r + 1] += rstart[r];
  {
    std::vector<int32_t> fill(rstart.begin(), rstart.end() - 1);
    for (int i = 0; i < N; ++i) out->row_states[fill[d->state_resp[i]]++] = i;
  }
  for (int r = 0; r < R; ++r)
    std::stable_sort(out->row_states + rstart[r], out->row_states + rstart[r + 1],
                     [&](int32_t a, int32_t b) { return d->state_step[a] < d->state_step[b]; });
  int nr = 0;
  for (int e = 0; e < N; ++e) {
    const int i = out->row_states[e];
    if (e == 0 || d->state_resp[i] != out->row_resp[nr - 1] || d->state_step[i] != out->row_step[nr - 1]) {
      out->row_resp[nr] = d->state_resp[i];
      out->row_step[nr] = d->state_step[i];
      out->row_state_offsets[nr] = e;
      ++nr;
    }
    out->state_row[i] = nr - 1;
  }
  out->row_state_offsets[nr] = N;
  out->n_rows = nr;

  // clean tokens a row needs: up to the clean copy of its furthest block, i.e.
  // the context its largest-index state sees (b*B - o), within the response
  for (int r = 0; r < nr; ++r) {
    const int resp = out->row_resp[r];
    int64_t need = 0, sup = 0, pages = 0;
    for (int e = out->row_state_offsets[r]; e < out->row_state_offsets[r + 1]; ++e) {
      const int i = out->row_states[e];
      need = std::max<int64_t>(need, (int64_t)d->state_block[i] * B - off[resp]);
      sup += d->state_supervised ? d->state_supervised[i] : B;
      pages += d->state_pages ? d->state_pages[i] : 0;
    }
    const int64_t ctx = std::min<int64_t>(std::max<int64_t>(need, 0), d->clean_len[resp]);
    out->row_ctx_len[r] = (int32_t)ctx;
    const int64_t tokens = ctx + (int64_t)(out->row_state_offsets[r + 1] - out->row_state_offsets[r]) * B;
    out->row_cost[r] = (int64_t)d->w_tokens * tokens + (int64_t)d->w_supervised * sup + (int64_t)d->w_pages * pages;
  }

  // largest cost first (ties: row number), each row to the least-loaded group
  // (ties: lowest group index)
  std::vector<int32_t> order(nr);
  std::iota(order.begin(), order.end(), 0);
  std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
    return out->row_cost[a] > out->row_cost[b]; });
  std::vector<int64_t> load(G, 0);
  std::vector<std::vector<int32_t>> per(G);
  for (int32_t r : order) {
    int g = 0;
    for (int x = 1; x < G; ++x) if (load[x] < load[g]) g = x;
    load[g] += out->row_cost[r];
    out->row_group[r] = g;
    per[g].push_back(r);
  }
  out->group_row_offsets[0] = 0;
  for (int g = 0; g < G; ++g) {
    out->group_row_offsets[g + 1] = out->group_row_offsets[g] + (int32_t)per[g].size();
    std::copy(per[g].begin(), per[g].end(), out->group_rows + out->group_row_offsets[g]);
    out->group_cost[g] = load[g];
  }
  return BD_ATTN_OK;
}

}  // namespace bdattn
