/* A plain C99 user of libbdattn: everything goes through include/bd_attn.h, with
 * device memory from the HIP runtime and nothing else (no Python, no torch).
 *
 *   bd_attn_consumer            plans a small packed batch, checks the statuses of
 *                               a few invalid calls and the plan's work-list image,
 *                               and prints the plan's sizes as one JSON line
 *                               (host only: no GPU needed)
 *   bd_attn_consumer --gpu F    also runs the forward and the backward on the
 *                               current GPU with seeded bf16 inputs and writes the
 *                               inputs and outputs to F for the test to compare
 *                               with the oracle
 *
 * The batch: two segments with block size 16, 4 query heads over 2 kv heads,
 * head_dim 64. Segment 0 replays a 48-token context (queries from position 0)
 * with canvases at blocks 1 and 3; segment 1 is a canvas-only step over a
 * 32-token context with one canvas at block 2.
 *
 * File F: int32 tq, tk, hq, hkv, d; then q [tq, hq, d], k and v [tk, hkv, d],
 * dout [tq, hq, d] as bf16 bit patterns; then o [tq, hq, d] bf16, lse [tq, hq]
 * float, dq [tq, hq, d], dk and dv [tk, hkv, d] bf16. Exit status 0 on success. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "bd_attn.h"

#define FAIL(...)                                   \
  do {                                              \
    fprintf(stderr, "bd_attn_consumer: " __VA_ARGS__); \
    fprintf(stderr, "\n");                          \
    exit(1);                                        \
  } while (0)

static void expect(bd_attn_status got, bd_attn_status want, const char* what) {
  if (got != want) FAIL("%s: status %d, expected %d (%s)", what, (int)got, (int)want, bd_attn_last_error());
}

static void hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) FAIL("%s: %s", what, hipGetErrorString(e));
}

/* xorshift32: a seeded stream of uniform values in [-1, 1) */
static uint32_t g_state = 2463534242u;
static float uniform(void) {
  g_state ^= g_state << 13;
  g_state ^= g_state >> 17;
  g_state ^= g_state << 5;
  return (float)((double)g_state / 2147483648.0 - 1.0);
}

/* float -> bf16 bit pattern, round to nearest even (inputs are finite) */
static uint16_t to_bf16(float x) {
  uint32_t u;
  memcpy(&u, &x, sizeof u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static uint16_t* seeded_bf16(size_t n, float scale) {
  uint16_t* h = (uint16_t*)malloc(n * sizeof *h);
  if (!h) FAIL("out of host memory");
  for (size_t i = 0; i < n; ++i) h[i] = to_bf16(scale * uniform());
  return h;
}

static void* dev_copy(const void* host, size_t bytes) {
  void* d = NULL;
  hip_ok(hipMalloc(&d, bytes ? bytes : 16), "hipMalloc");
  if (host) hip_ok(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice), "hipMemcpy to device");
  return d;
}

static void* host_copy(const void* dev, size_t bytes) {
  void* h = malloc(bytes);
  if (!h) FAIL("out of host memory");
  hip_ok(hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost), "hipMemcpy to host");
  return h;
}

static void write_all(FILE* f, const void* p, size_t bytes) {
  if (fwrite(p, 1, bytes, f) != bytes) FAIL("short write");
}

int main(int argc, char** argv) {
  const char* gpu_out = NULL;
  if (argc == 3 && strcmp(argv[1], "--gpu") == 0) gpu_out = argv[2];
  else if (argc != 1) FAIL("usage: bd_attn_consumer [--gpu FILE]");

  const int32_t ctx_len[2] = {48, 32}, ctx_q_begin[2] = {0, 32};
  const int32_t canvas_offsets[3] = {0, 2, 3}, canvas_block_idx[3] = {1, 3, 2};
  bd_attn_desc desc;
  memset(&desc, 0, sizeof desc);
  desc.num_segments = 2;
  desc.ctx_len = ctx_len;
  desc.ctx_q_begin = ctx_q_begin;
  desc.canvas_offsets = canvas_offsets;
  desc.canvas_block_idx = canvas_block_idx;
  desc.block_size = 16;
  desc.num_q_heads = 4;
  desc.num_kv_heads = 2;
  desc.head_dim = 64;
  desc.dtype = BD_ATTN_BF16;
  desc.softmax_scale = 0.f;
  desc.flags = BD_ATTN_FLAG_CHECK_PLAN;

  /* invalid calls report their status and a message, and touch nothing */
  bd_attn_plan_t plan = NULL;
  expect(bd_attn_plan(NULL, &plan), BD_ATTN_EINVAL, "plan(NULL desc)");
  if (plan != NULL || bd_attn_last_error()[0] == '\0') FAIL("plan(NULL desc) left a plan or no message");
  desc.head_dim = 96;
  expect(bd_attn_plan(&desc, &plan), BD_ATTN_EUNSUPPORTED, "plan(head_dim 96)");
  desc.head_dim = 64;

  expect(bd_attn_plan(&desc, &plan), BD_ATTN_OK, "plan");
  int64_t tq = 0, tk = 0, pairs = 0;
  size_t meta_bytes = 0, ws_fwd = 0, ws_bwd = 0;
  expect(bd_attn_plan_sizes(plan, &tq, &tk, &meta_bytes, &ws_fwd, &ws_bwd, &pairs), BD_ATTN_OK, "plan_sizes");

  /* the serialized work lists pass the self-check; a short buffer is refused */
  void* meta_host = malloc(meta_bytes);
  if (!meta_host) FAIL("out of host memory");
  expect(bd_attn_plan_serialize(plan, meta_host, meta_bytes), BD_ATTN_OK, "plan_serialize");
  expect(bd_attn_plan_check(plan, meta_host, meta_bytes), BD_ATTN_OK, "plan_check");
  expect(bd_attn_plan_serialize(plan, meta_host, meta_bytes - 4), BD_ATTN_EWORKSPACE, "plan_serialize(short)");
  free(meta_host);

  bd_attn_plan_info_t info;
  expect(bd_attn_plan_info(plan, &info), BD_ATTN_OK, "plan_info");
  expect(bd_attn_plan_info(plan, NULL), BD_ATTN_EINVAL, "plan_info(NULL)");
  printf("{\"version\": \"%s\", \"tq\": %lld, \"tk\": %lld, \"meta_bytes\": %zu, \"ws_fwd\": %zu, "
         "\"ws_bwd\": %zu, \"pairs\": %lld, \"fwd_kernels\": %d, \"bwd_kernels\": %d, \"split\": %d, "
         "\"dkdv_masked\": %d, \"fwd_workgroups\": %lld, \"dkdv_workgroups\": %lld}\n",
         bd_attn_version(), (long long)tq, (long long)tk, meta_bytes, ws_fwd, ws_bwd, (long long)pairs,
         (int)bd_attn_plan_kernels(plan, 0), (int)bd_attn_plan_kernels(plan, 1), (int)info.split,
         (int)info.dkdv_masked, (long long)info.fwd_workgroups, (long long)info.dkdv_workgroups);
  fflush(stdout);

  if (gpu_out) {
    const int hq = desc.num_q_heads, hkv = desc.num_kv_heads, d = desc.head_dim;
    const size_t nq = (size_t)tq * hq * d, nk = (size_t)tk * hkv * d, nl = (size_t)tq * hq;
    uint16_t* q_h = seeded_bf16(nq, 1.0f);
    uint16_t* k_h = seeded_bf16(nk, 1.0f);
    uint16_t* v_h = seeded_bf16(nk, 1.0f);
    uint16_t* do_h = seeded_bf16(nq, 1.0f);
    void* meta = dev_copy(NULL, meta_bytes);
    void* q = dev_copy(q_h, nq * 2);
    void* k = dev_copy(k_h, nk * 2);
    void* v = dev_copy(v_h, nk * 2);
    void* dout = dev_copy(do_h, nq * 2);
    void* o = dev_copy(NULL, nq * 2);
    void* lse = dev_copy(NULL, nl * 4);
    void* dq = dev_copy(NULL, nq * 2);
    void* dk = dev_copy(NULL, nk * 2);
    void* dv = dev_copy(NULL, nk * 2);
    void* wsf = ws_fwd ? dev_copy(NULL, ws_fwd) : NULL;
    void* wsb = dev_copy(NULL, ws_bwd);

    /* all work on the default (null) stream */
    expect(bd_attn_plan_upload(plan, meta, NULL), BD_ATTN_OK, "plan_upload");
    expect(bd_attn_fwd(plan, NULL, q, k, v, o, (float*)lse, wsf, NULL), BD_ATTN_EINVAL, "fwd(NULL meta)");
    expect(bd_attn_fwd(plan, meta, q, k, v, o, (float*)lse, wsf, NULL), BD_ATTN_OK, "fwd");
    expect(bd_attn_bwd(plan, meta, q, k, v, o, (const float*)lse, dout, dq, dk, dv, wsb, NULL), BD_ATTN_OK, "bwd");
    hip_ok(hipDeviceSynchronize(), "hipDeviceSynchronize");

    FILE* f = fopen(gpu_out, "wb");
    if (!f) FAIL("cannot open %s", gpu_out);
    const int32_t hdr[5] = {(int32_t)tq, (int32_t)tk, hq, hkv, d};
    write_all(f, hdr, sizeof hdr);
    write_all(f, q_h, nq * 2);
    write_all(f, k_h, nk * 2);
    write_all(f, v_h, nk * 2);
    write_all(f, do_h, nq * 2);
    void* outs[5] = {o, lse, dq, dk, dv};
    const size_t bytes[5] = {nq * 2, nl * 4, nq * 2, nk * 2, nk * 2};
    for (int i = 0; i < 5; ++i) {
      void* h = host_copy(outs[i], bytes[i]);
      write_all(f, h, bytes[i]);
      free(h);
    }
    if (fclose(f) != 0) FAIL("close %s", gpu_out);
    void* bufs[12] = {meta, q, k, v, dout, o, lse, dq, dk, dv, wsf, wsb};
    for (int i = 0; i < 12; ++i)
      if (bufs[i]) hip_ok(hipFree(bufs[i]), "hipFree");
    free(q_h);
    free(k_h);
    free(v_h);
    free(do_h);
    printf("gpu: wrote %s\n", gpu_out);
  }
  expect(bd_attn_plan_destroy(plan), BD_ATTN_OK, "plan_destroy");
  return 0;
}
