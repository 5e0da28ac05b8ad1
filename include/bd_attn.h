/*
 * bd_attn.h — C ABI of libbdattn.so: staircase block-diffusion attention on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (ORL paper, arXiv 2610.20687, section 3.2 "Staircase attention
 * kernel" and the appendix D.2 paragraph on the kernel): softmax attention over
 * packed, mutually invisible documents, where each document (segment) holds a
 * clean context followed by m captured canvases of one block each (section 3.1:
 * the canvas is replayed after its clean context). Visibility:
 *   - a canvas with block index b sees the clean context blocks 0..b-1 and its
 *     own B tokens (bidirectionally); never its own clean copy (block b), later
 *     blocks, other canvases or other segments;
 *   - a clean query sees clean keys block-causally (key block <= query block,
 *     bidirectional inside a block) and never a canvas key.
 * Two variants of the clean rule, both per plan (ORL section 3.3 "Commit
 * folding" runs the finished block's commit pass together with the next
 * canvas; appendix F.1 calls that pass causal; the pages fix neither the
 * granularity of "causal" nor where a prompt's blocks begin):
 *   - BD_ATTN_FLAG_CLEAN_CAUSAL: a clean query sees the clean keys at context
 *     positions up to its own (token-causal) instead of whole blocks;
 *   - block_offset[s] = o (0 <= o < B): the segment's block grid starts o
 *     positions before its first context token, i.e. context position p lies
 *     in block (p + o) / B and the first block holds B - o tokens (a prompt
 *     whose length is not a multiple of B, followed by whole blocks).
 *     ctx_len[s] + o must be a multiple of B; a canvas with block index b sees
 *     the context positions p < b*B - o.
 * The commit-folded step is ctx_q_begin[s] = ctx_len[s] - B (the finished block's
 * tokens as queries) with one canvas at the next block index.
 * The forward pass returns O = softmax(scale * Q K^T under that visibility) V and
 * the natural-log LSE of the scaled scores; the backward pass returns dQ, dK,
 * dV of L = <dO, O>. Visible key ranges are derived from per-segment metadata;
 * no dense mask is ever built and fully invisible tiles are never visited
 * (same section and appendix paragraph).
 *
 * Packed "THD" layouts, row-major, contiguous, element type = desc.dtype:
 *   Q, O, dO, dQ : [Tq, Hq, D]      K, V, dK, dV : [Tk, Hkv, D]
 *   LSE          : [Tq, Hq] float32 (always float32)
 * Segment s occupies, in order of s:
 *   keys    : ctx_len[s] clean tokens, then its canvases (B tokens each) in the
 *             order they appear in canvas_block_idx;
 *   queries : clean tokens at positions ctx_q_begin[s] .. ctx_len[s]-1, then the
 *             same canvases in the same order.
 *   Tq = sum_s (ctx_len[s] - ctx_q_begin[s] + m_s * B), Tk = sum_s (ctx_len[s] + m_s * B).
 * ctx_q_begin[s] = 0 is replay (every context token is also a query);
 * ctx_q_begin[s] = ctx_len[s] is the single-request denoising step (only the
 * canvas queries; appendix F.1 "Kernels": attention of the canvas over a KV
 * arena).
 * Query head h reads kv head h / (Hq / Hkv).
 *
 * Ownership: the caller owns every device buffer (tensors, the metadata buffer
 * and the workspace). The library never allocates device memory and never
 * synchronises the host; every device operation is enqueued on the stream
 * passed in. A plan owns host memory only and is immutable after creation:
 * one plan may serve any number of calls on any streams.
 *
 * Errors: every function returns a bd_attn_status; nothing aborts or throws
 * across the ABI. On a non-OK status, bd_attn_last_error() returns a message
 * (thread-local, valid until the next call on the same thread) and no device
 * work was enqueued by the failing call.
 */
#ifndef BD_ATTN_H_
#define BD_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP stream type, declared opaquely so host-only users need no HIP headers. */
typedef struct ihipStream_t* bd_attn_stream_t;

typedef enum {
  BD_ATTN_OK = 0,
  BD_ATTN_EINVAL = 1,        /* invalid metadata, pointer, size or alignment */
  BD_ATTN_EUNSUPPORTED = 2,  /* valid but not implemented (head_dim, group size) */
  BD_ATTN_EWORKSPACE = 3,    /* workspace or metadata buffer too small */
  BD_ATTN_EHIP = 4           /* a HIP runtime call or kernel launch failed */
} bd_attn_status;

typedef enum { BD_ATTN_BF16 = 0, BD_ATTN_FP32 = 1 } bd_attn_dtype;

/* flags */
#define BD_ATTN_FLAG_NO_SPLIT   1u  /* never split a query tile's key range (forward) */
#define BD_ATTN_FLAG_FORCE_SPLIT 2u /* always split long key ranges (forward; for tests) */
#define BD_ATTN_FLAG_NO_XCD     4u  /* plain largest-cost-first order, no XCD grouping
                                       (nor the part-major order of single-request
                                       splits) */
#define BD_ATTN_FLAG_FWD_DIRECT 8u /* bf16 forward without the transposed V copy (the
                                       default; kept for callers that set it) */
#define BD_ATTN_FLAG_FWD_VT     16u /* bf16 forward through a transposed copy of V (a
                                       pre-pass) when the block size is a multiple of 8
                                       and the packed key stream holds fewer than about
                                       2^30 / head_dim keys (8M at head_dim 128; longer
                                       streams take the direct kernel);
                                       FWD_DIRECT wins if both are set */
#define BD_ATTN_FLAG_CLEAN_CAUSAL 32u /* clean queries see clean keys token-causally
                                         (position <= own) instead of block-causally */
/* Bits 8..15: key tiles (of 64 keys) per split of the forward split path;
 * 0 selects the library's choice. Ignored unless the plan splits. */
#define BD_ATTN_FLAG_CHECK_PLAN  64u /* bd_attn_plan runs bd_attn_plan_check on its own
                                       work lists before returning (EINVAL if they
                                       break an invariant; a debugging aid) */
#define BD_ATTN_FLAG_DEBUG_CHECKS 128u /* debugging: the plan runs the record-checking
                                         kernels (see bd_attn_device_check_errors), and
                                         bd_attn_plan self-checks its work lists as with
                                         CHECK_PLAN */
#define BD_ATTN_FLAG_SPLIT_TILES(n) ((((uint32_t)(n)) & 0xffu) << 8)
#define BD_ATTN_FLAG_DKDV_RUNS (1u << 16) /* dK/dV: launch the key tiles of one (segment,
                                       kv head) in runs of 8 on one XCD, so that tiles
                                       walking the same query chunks start together and
                                       fetch each chunk into the XCD's L2 once. On packs
                                       of many segments the kernel fetches about a third
                                       of the HBM bytes, but runs slower on MI355X (about
                                       8 % on the 16-segment packed replay), so it is off
                                       by default: for callers that share HBM bandwidth
                                       with other work. No effect with NO_XCD, or when
                                       the plan falls back to one global order. */

typedef struct bd_attn_plan_s* bd_attn_plan_t;

typedef struct {
  int32_t num_segments;             /* S >= 1 */
  const int32_t* ctx_len;           /* host [S]: C_s >= 0, C_s + o_s a multiple of block_size */
  const int32_t* ctx_q_begin;       /* host [S] or NULL (= 0 for all): 0 <= q0_s <= C_s */
  const int32_t* canvas_offsets;    /* host [S+1]: prefix sums, canvas_offsets[0] = 0 */
  const int32_t* canvas_block_idx;  /* host [canvas_offsets[S]]: 0 <= b <= (C_s + o_s) / B,
                                       any order */
  int32_t block_size;               /* B >= 1 */
  int32_t num_q_heads;              /* Hq >= 1, multiple of num_kv_heads */
  int32_t num_kv_heads;             /* Hkv >= 1 */
  int32_t head_dim;                 /* 64 or 128 */
  int32_t dtype;                    /* bd_attn_dtype */
  float softmax_scale;              /* <= 0 selects 1/sqrt(head_dim) */
  uint32_t flags;                   /* BD_ATTN_FLAG_* */
  const int32_t* block_offset;      /* host [S] or NULL (= 0 for all): 0 <= o_s < B, the
                                       block grid's start before the first context token */
} bd_attn_desc;

/* Validates the metadata and builds a plan (host only; copies everything it
 * needs). Work lists: query tiles with their visible key ranges (forward and
 * dQ), key tiles with their visible query ranges (dK/dV), each ordered
 * largest-cost-first (ORL section 3.2 "Packed and cost-balanced state training"
 * and appendix D.3 apply that order to data-parallel groups; here it orders
 * workgroups across compute units). Errors: EINVAL on bad metadata, EUNSUPPORTED
 * on an unsupported head_dim / group size, both with *out untouched. */
bd_attn_status bd_attn_plan(const bd_attn_desc* desc, bd_attn_plan_t* out);

/* Sizes implied by a plan: packed token counts, bytes of the device metadata
 * buffer, bytes of forward / backward workspace (0 when none is needed) and
 * the number of visible (query token, key token) pairs per query head. Any
 * output pointer may be NULL. */
bd_attn_status bd_attn_plan_sizes(bd_attn_plan_t plan, int64_t* tq, int64_t* tk,
                                  size_t* meta_bytes, size_t* ws_fwd_bytes,
                                  size_t* ws_bwd_bytes, int64_t* visible_pairs);

/* Copies the plan's host work lists into meta_host (meta_bytes bytes, host
 * memory owned by the caller), e.g. to stage them into pinned memory. */
bd_attn_status bd_attn_plan_serialize(bd_attn_plan_t plan, void* meta_host, size_t bytes);

/* Checks a work-list image (meta_bytes bytes of host memory laid out as
 * bd_attn_plan_serialize writes it) against plan: the header and the section
 * counts match the plan, every section lies inside the image, and every index a
 * kernel follows lies inside its list or tensor (query / key tile indices,
 * canvas-query entries, kv heads, key tile ranges of a query tile, partial
 * slots, query and key token ranges inside [0, Tq) / [0, Tk)). For debugging a
 * planner change or an image that was edited or copied by hand: the kernels
 * re-check these bounds only for plans made with BD_ATTN_FLAG_DEBUG_CHECKS (see
 * bd_attn_device_check_errors). Errors: EINVAL naming the first bad section and
 * record (bd_attn_last_error), EWORKSPACE if bytes is smaller than meta_bytes. */
bd_attn_status bd_attn_plan_check(bd_attn_plan_t plan, const void* meta_host, size_t bytes);

/* Debugging. For a plan made with BD_ATTN_FLAG_DEBUG_CHECKS, bd_attn_fwd and
 * bd_attn_bwd launch instantiations of their kernels that check each work record
 * a workgroup reads against the plan's list and tensor sizes before following any
 * index or token range in it (the bounds bd_attn_plan_check tests on the host,
 * applied to the image in device memory as the kernels see it). A workgroup that
 * finds a bad record is counted and does nothing, so its part of the outputs is
 * left unwritten; one bad record can be counted by several workgroups (the dK/dV
 * merge reads each record from several, and an fp32 plan's forward and dQ
 * kernels read the same list). Other plans run kernels without these checks
 * (their code is unchanged by them). This call waits for all work on the current
 * device, stores in *count the number of such workgroups on that device since
 * the last reset, and clears the counters when reset is non-zero. Calls that
 * overlap with kernels running on other host threads race with them. Errors:
 * EINVAL if count is NULL, EHIP if a HIP call fails. */
bd_attn_status bd_attn_device_check_errors(uint64_t* count, int reset);

/* Enqueues an asynchronous copy of the work lists into meta_dev (device memory
 * of at least meta_bytes bytes, 16-byte aligned) on stream. The source is the
 * plan's own host memory, so the plan must outlive the copy. Call once before
 * the first bd_attn_fwd / bd_attn_bwd with this meta_dev. */
bd_attn_status bd_attn_plan_upload(bd_attn_plan_t plan, void* meta_dev, bd_attn_stream_t stream);

/* Forward. q [Tq,Hq,D], k/v [Tk,Hkv,D] in desc.dtype; writes o [Tq,Hq,D] and
 * lse [Tq,Hq] (float32). ws: ws_fwd_bytes of device memory (may be NULL when
 * that size is 0): for bf16 plans made with BD_ATTN_FLAG_FWD_VT (and a block
 * size that is a multiple of 8) it holds a transposed copy of V (rewritten by
 * every call), and on the split path the partial results. All pointers device
 * pointers, 16-byte aligned.
 * Errors: EINVAL (NULL or misaligned pointer), EWORKSPACE (ws NULL while
 * needed), EHIP (launch failure). */
bd_attn_status bd_attn_fwd(bd_attn_plan_t plan, const void* meta_dev,
                           const void* q, const void* k, const void* v,
                           void* o, float* lse, void* ws, bd_attn_stream_t stream);

/* Backward of L = <dO, O> with o / lse from bd_attn_fwd on the same inputs.
 * Writes (does not accumulate) dq [Tq,Hq,D], dk and dv [Tk,Hkv,D]; dK and dV
 * are summed over the query heads of each kv head. Deterministic: no atomics,
 * bitwise identical across runs. ws: ws_bwd_bytes of device memory (holds the
 * float32 row terms delta = rowsum(dO * O) and LSE * log2(e), [Tq, Hq] each, and
 * for plans that split dK/dV key tiles the float32 partial dK/dV of the parts).
 * Errors as bd_attn_fwd. */
bd_attn_status bd_attn_bwd(bd_attn_plan_t plan, const void* meta_dev,
                           const void* q, const void* k, const void* v,
                           const void* o, const float* lse, const void* dout,
                           void* dq, void* dk, void* dv, void* ws, bd_attn_stream_t stream);

/* Forward for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc. Same as
 * bd_attn_fwd, except that the forward workspace is a fixed array of
 * BD_ATTN_NOALLOC_WS_BYTES inside the library's device code object (one copy per
 * GPU, held until the process ends) instead of a caller buffer; the call itself
 * allocates nothing. Nothing in it needs to start at zero (every call writes what
 * it later reads). All calls on one GPU share that array and it keeps the last
 * call's contents: calls that overlap on one GPU (different streams, or host
 * threads without ordering) race and may return wrong results.
 * Errors: EWORKSPACE (checked before any device call) when the plan's
 * ws_fwd_bytes exceeds BD_ATTN_NOALLOC_WS_BYTES; otherwise as bd_attn_fwd, plus
 * EHIP if the array's device address cannot be looked up. */
#define BD_ATTN_NOALLOC_WS_BYTES (32u << 20)
bd_attn_status bd_attn_fwd_noalloc(bd_attn_plan_t plan, const void* meta_dev,
                                   const void* q, const void* k, const void* v,
                                   void* o, float* lse, bd_attn_stream_t stream);

/* Same as bd_attn_fwd / bd_attn_bwd, and in addition records caller-created
 * hipEvent_t handles (passed as void*) on the stream around the kernels, for
 * per-kernel timing on the stream that runs them: events[0] before the first
 * kernel and events[i] right after the i-th one. The forward pass launches 1 to
 * 3 kernels (V transpose on the pipelined path, the attention kernel, and the
 * merge of partial results on the split path; bd_attn_plan_kernels(plan, 0) and
 * bd_attn_plan_kernel_name give the count and names), the backward pass 2 or 3
 * in bf16 (dQ, which also computes delta = rowsum(dO * O); dK/dV; the merge of
 * split key tiles when the plan splits them) and 3 in fp32 (delta, dK/dV, dQ).
 * n_events must be at least kernels + 1, else EINVAL and nothing is enqueued. */
bd_attn_status bd_attn_fwd_timed(bd_attn_plan_t plan, const void* meta_dev,
                                 const void* q, const void* k, const void* v,
                                 void* o, float* lse, void* ws, bd_attn_stream_t stream,
                                 void* const* events, int n_events);
bd_attn_status bd_attn_bwd_timed(bd_attn_plan_t plan, const void* meta_dev,
                                 const void* q, const void* k, const void* v,
                                 const void* o, const float* lse, const void* dout,
                                 void* dq, void* dk, void* dv, void* ws, bd_attn_stream_t stream,
                                 void* const* events, int n_events);

/* Number of kernels bd_attn_fwd (backward = 0) or bd_attn_bwd (backward = 1)
 * launches for this plan; 0 for a NULL plan. */
int32_t bd_attn_plan_kernels(bd_attn_plan_t plan, int32_t backward);

/* Short name of the i-th kernel (0-based, launch order) that bd_attn_fwd
 * (backward = 0) or bd_attn_bwd (backward = 1) launches for this plan, e.g.
 * "transpose_v", "fwd", "merge", "bwd_pre", "dq", "dkdv", "dkdv_merge"; NULL when i is out of
 * range or the plan is NULL. "dkdv_masked" names the bf16 dK/dV kernel that
 * applies a row limit to every score: plans whose query chunks are not all either
 * seen whole by a 32-key group or not at all (block size not a multiple of 32,
 * 64 / G not dividing it, or a query range starting inside a block). The string
 * is static. */
const char* bd_attn_plan_kernel_name(bd_attn_plan_t plan, int32_t backward, int32_t i);

/* The scheduling choices a plan made (all filled by bd_attn_plan_info). */
typedef struct {
  int32_t split;              /* 1: the forward splits key ranges (partials + merge) */
  int32_t split_tiles;        /* key tiles (of 64 keys) per split part, 0 if not split */
  int32_t split_grid;         /* 1: the split is a regular grid (one query tile, kv heads a
                                 multiple of 8, part-major launch order): its workgroups
                                 compute their part from their index instead of loading
                                 their record */
  int32_t fwd_vt;             /* 1: the forward goes through the transposed V copy */
  int32_t dkdv_masked;        /* 1: dK/dV applies per-score row limits */
  int32_t debug_checks;       /* 1: the kernels check their records (BD_ATTN_FLAG_DEBUG_CHECKS) */
  int64_t query_tiles;        /* query tiles (up to 128 rows of one segment) */
  int64_t key_tiles;          /* key tiles (up to 128 keys of one segment) */
  int64_t fwd_workgroups;     /* workgroups of the forward attention kernel */
  int64_t dq_workgroups;      /* workgroups of the dQ kernel */
  int64_t dkdv_workgroups;    /* workgroups of the dK/dV kernel */
  int64_t dkdv_split_tiles;   /* key tiles whose chunks are split over several workgroups */
} bd_attn_plan_info_t;

/* Fills *out with the plan's scheduling choices and list sizes (host only).
 * Errors: EINVAL if plan or out is NULL. */
bd_attn_status bd_attn_plan_info(bd_attn_plan_t plan, bd_attn_plan_info_t* out);

/* ---------------------------------------------------------------------------
 * Host packer (ORL section 3.2 "Packed and cost-balanced state training",
 * appendix D.3): builds replay rows from captured denoising states and assigns
 * them to data-parallel groups. A row holds one response's clean tokens once,
 * followed by the states of its blocks captured at the same denoising step k
 * (each state a canvas at its block index), so every state reuses the clean
 * context before it. A row keeps the clean tokens its states can see: up to
 * max_b (b*B - o) of its states (at most the response's clean length). Rows are
 * ordered by (response, step); each state, and so each of its supervised labels,
 * belongs to exactly one row.
 * Cost proxy of a row (integer): w_tokens * (clean tokens + states * B)
 *   + w_supervised * (sum of supervised positions) + w_pages * (sum of pages).
 * Assignment: rows in decreasing cost (ties: lower row number first), each to
 * the group with the smallest total cost so far (ties: lowest group index) --
 * deterministic largest-cost-first. A group's rows, in that order, are the
 * segments of one bd_attn_desc (ctx_len = row_ctx_len, ctx_q_begin = 0,
 * canvas_block_idx = the blocks of the row's states, block_offset = the
 * response's offset, or 0 for a row that holds no clean token).
 * Host-only; touches no device memory.
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t num_responses;            /* R >= 1 */
  const int32_t* clean_len;         /* host [R]: clean tokens C_r of each response */
  const int32_t* block_offset;      /* host [R] or NULL (= 0): grid offset o_r, 0 <= o_r < B,
                                       C_r + o_r a multiple of B (as in bd_attn_desc) */
  int32_t num_states;               /* N >= 0 */
  const int32_t* state_resp;        /* host [N]: response of each state, 0..R-1 */
  const int32_t* state_block;       /* host [N]: block index b, 0 <= b <= (C_r + o_r) / B */
  const int32_t* state_step;        /* host [N]: denoising step k >= 0 */
  const int32_t* state_supervised;  /* host [N] or NULL (= B): supervised positions, 0..B */
  const int32_t* state_pages;       /* host [N] or NULL (= 0): resident residual pages >= 0 */
  int32_t block_size;               /* B >= 1 */
  int32_t num_groups;               /* data-parallel groups G >= 1 */
  int32_t w_tokens;                 /* cost weights >= 0 */
  int32_t w_supervised;
  int32_t w_pages;
} bd_pack_desc;

/* Outputs, every array host memory owned by the caller; sizes in brackets
 * (rows never outnumber states, so N bounds every row array). */
typedef struct {
  int32_t* state_row;           /* [N]   row of each state */
  int32_t* row_resp;            /* [N]   response of row i (i < n_rows) */
  int32_t* row_step;            /* [N]   its step k */
  int32_t* row_ctx_len;         /* [N]   clean tokens it holds */
  int32_t* row_group;           /* [N]   the group it is assigned to */
  int64_t* row_cost;            /* [N]   its cost proxy */
  int32_t* row_state_offsets;   /* [N+1] states of row i: row_states[off[i] .. off[i+1]) */
  int32_t* row_states;          /* [N]   state indices, input order within a row */
  int32_t* group_row_offsets;   /* [G+1] rows of group g: group_rows[off[g] .. off[g+1]) */
  int32_t* group_rows;          /* [N]   in assignment order */
  int64_t* group_cost;          /* [G]   total cost per group */
  int32_t n_rows;               /* written: number of rows */
} bd_pack_out;

/* Builds the rows and the assignment. Errors: EINVAL on bad input (message in
 * bd_attn_last_error), outputs then unspecified. */
bd_attn_status bd_attn_pack(const bd_pack_desc* desc, bd_pack_out* out);

/* ---------------------------------------------------------------------------
 * Normalized entropy and the adjacent-entropy-contraction (AEC) loss over
 * vocabulary logits (ORL paper, paragraph "Learning how fast to refine"; the
 * appendix paragraph on valid AEC pairs, their weights and the gate):
 *   per row i (a position):  lse_i = log sum_v exp(x_iv)           (natural log)
 *                            hbar_i = -sum_v p_iv log p_iv / log V, p_i = softmax(x_i)
 *   per state s:             h_state_s = mean of hbar over its unresolved rows,
 *                            NaN when it has none
 *   per pair p (source -> next state):
 *                            hinge_p = max(0, h_state[next_p] - (1 - rho) h_source_p)^2
 *   loss = sum_p w_p g_p hinge_p / D, D = sum_p w_p g_p, over valid pairs; 0 if D = 0
 * A pair is valid when next_p lies in [0, S), that state has an unresolved row
 * and h_source_p (the captured mean of the source state) is finite; the gate
 * g_p = 1 if h_source_p <= gate_max (+inf keeps every pair). The combination of
 * the pairs is a reading: its equation is lost from the pages' text, which fixes
 * the weights before the gate, D as their gated sum and a zero loss for D = 0.
 * Logits must be finite. Results are deterministic (no atomics).
 * ------------------------------------------------------------------------- */
typedef struct {
  int32_t num_rows;                 /* N >= 1 */
  int32_t vocab;                    /* V >= 2 */
  int64_t row_stride;               /* elements from one row to the next, >= V; a multiple
                                       of 8 (bf16) or 4 (fp32) */
  int32_t dtype;                    /* logits: BD_ATTN_BF16 or BD_ATTN_FP32 */
  int32_t num_states;               /* S >= 0 */
  int32_t num_pairs;                /* P >= 0 */
  float rho;                        /* target contraction rate, 0 <= rho <= 1 */
  float gate_max;                   /* not NaN */
} bd_aec_desc;

/* Bytes of device workspace for bd_aec_fwd and bd_aec_bwd (one buffer serves
 * both; bd_aec_fwd also accepts NULL when the rows are not split). */
bd_attn_status bd_aec_workspace(const bd_aec_desc* desc, size_t* ws_bytes);

/* Enqueues the reduction on stream. Device pointers: logits [N][row_stride]
 * (16-byte aligned), unresolved [N] (uint8, nonzero = unresolved), state_rows
 * [S+1] (state s owns rows state_rows[s] .. state_rows[s+1]-1, ranges clamped to
 * [0, N]), pair_next / pair_h_source / pair_weight [P]; outputs lse [N], hbar
 * [N], h_state [S], loss [1] (float32). unresolved and state_rows may be NULL
 * only when S = 0, the pair arrays only when P = 0. Errors: EINVAL (bad sizes,
 * NULL or misaligned pointer), EWORKSPACE (ws NULL while needed), EHIP. */
bd_attn_status bd_aec_fwd(const bd_aec_desc* desc, const void* logits, const uint8_t* unresolved,
                          const int32_t* state_rows, const int32_t* pair_next,
                          const float* pair_h_source, const float* pair_weight, float* lse,
                          float* hbar, float* h_state, float* loss, void* ws,
                          bd_attn_stream_t stream);

/* Same, recording caller-created hipEvent_t handles (as void*) around the
 * kernels: events[0] before the first, events[i] after the i-th; the kernels are
 * "aec_entropy" (one pass over the logits; short batches split each row over
 * several workgroups and leave partial results in ws) and "aec_reduce" (one
 * workgroup: the merge of split rows, the state means, the loss).
 * n_events >= kernels + 1 (bd_aec_kernels gives the count). */
bd_attn_status bd_aec_fwd_timed(const bd_aec_desc* desc, const void* logits, const uint8_t* unresolved,
                                const int32_t* state_rows, const int32_t* pair_next,
                                const float* pair_h_source, const float* pair_weight, float* lse,
                                float* hbar, float* h_state, float* loss, void* ws,
                                bd_attn_stream_t stream, void* const* events, int n_events);

/* Number of kernels bd_aec_fwd launches for desc (0 if desc is invalid). */
int32_t bd_aec_kernels(const bd_aec_desc* desc);

/* Gradient of grad_loss[0] * loss with respect to the logits, written to dlogits
 * [N][row_stride] (the logits' type; only the first V columns are written):
 *   dL/dx_iv = -c_i p_iv (log p_iv + H_i),  H_i = hbar_i ln V,
 *   c_i = (1 / (|U_s| ln V)) sum over kept valid pairs p with next state s of
 *         2 w_p hinge_p / D, for an unresolved row i of state s; 0 otherwise.
 * The captured source means are constants. lse, hbar and h_state are the outputs
 * of bd_aec_fwd on the same inputs; grad_loss is a device scalar. state_rows must
 * be non-decreasing (states own disjoint row ranges). Launches "aec_grad_coef" (one
 * workgroup) and "aec_grad" (one pass over the logits). dlogits may be the logits
 * buffer itself (in place; columns past V then keep the logits); otherwise the two
 * must not overlap. ws: bd_aec_workspace bytes (required). Errors as bd_aec_fwd. */
bd_attn_status bd_aec_bwd(const bd_aec_desc* desc, const void* logits, const uint8_t* unresolved,
                          const int32_t* state_rows, const int32_t* pair_next,
                          const float* pair_h_source, const float* pair_weight, const float* lse,
                          const float* hbar, const float* h_state, const float* grad_loss,
                          void* dlogits, void* ws, bd_attn_stream_t stream);
/* Same, with events[0..2] recorded before, between and after the two kernels. */
bd_attn_status bd_aec_bwd_timed(const bd_aec_desc* desc, const void* logits, const uint8_t* unresolved,
                                const int32_t* state_rows, const int32_t* pair_next,
                                const float* pair_h_source, const float* pair_weight, const float* lse,
                                const float* hbar, const float* h_state, const float* grad_loss,
                                void* dlogits, void* ws, bd_attn_stream_t stream, void* const* events,
                                int n_events);

/* Frees a plan (NULL is accepted). */
bd_attn_status bd_attn_plan_destroy(bd_attn_plan_t plan);

/* Message for the last non-OK status returned on this thread ("" if none). */
const char* bd_attn_last_error(void);

/* Library version, "major.minor.patch". */
const char* bd_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BD_ATTN_H_ */
