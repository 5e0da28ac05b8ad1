// C ABI of libbdattn.so: argument checks, plan handling and kernel launches.
// Every entry point returns a status; no exception crosses the boundary.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstring>
#include <mutex>
#include <new>
#include <string>

#include "../../include/bd_attn.h"
#include "aec.h"
#include "kernels.h"
#include "packer.h"
#include "planner.h"

using bdattn::Plan;

namespace {

thread_local std::string g_last_error;

bd_attn_status fail(bd_attn_status st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bd_attn_status check_ptr(const void* p, const char* name) {
  if (!p) return fail(BD_ATTN_EINVAL, std::string(name) + " is NULL");
  if (!aligned16(p)) return fail(BD_ATTN_EINVAL, std::string(name) + " is not 16-byte aligned");
  return BD_ATTN_OK;
}

bd_attn_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return BD_ATTN_OK;
  return fail(BD_ATTN_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

// Records events[i] (if any) on the stream; i beyond n is ignored.
struct EventMarks {
  void* const* ev;
  int n;
  hipStream_t s;
  hipError_t mark(int i) const {
    if (!ev || i >= n || !ev[i]) return hipSuccess;
    return hipEventRecord(reinterpret_cast<hipEvent_t>(ev[i]), s);
  }
};

// Kernels launched by bd_attn_fwd / bd_attn_bwd, in order.
int fwd_kernels(const Plan& p) {
  const bool bf16 = p.desc.dtype == BD_ATTN_BF16;
  return 1 + (bf16 && p.use_vt ? 1 : 0) + (bf16 && p.split ? 1 : 0);
}
// bf16: dQ (which also writes the row terms), dK/dV, [merge of split key tiles];
// fp32: row terms, dK/dV, dQ.
int bwd_kernels(const Plan& p) {
  return p.desc.dtype == BD_ATTN_BF16 ? (p.bwd_merge.empty() ? 2 : 3) : 3;
}
const char* kernel_name(const Plan& p, bool backward, int i) {
  if (backward) {
    if (i < 0 || i >= bwd_kernels(p)) return nullptr;
    if (p.desc.dtype != BD_ATTN_BF16) {
      static const char* const f32[] = {"bwd_pre", "dkdv", "dq"};
      return f32[i];
    }
    if (i == 0) return "dq";
    if (i == 1) return p.dkdv_masked ? "dkdv_masked" : "dkdv";
    return "dkdv_merge";
  }
  if (i < 0 || i >= fwd_kernels(p)) return nullptr;
  const bool bf16 = p.desc.dtype == BD_ATTN_BF16;
  if (bf16 && p.use_vt) {
    if (i == 0) return "transpose_v";
    --i;
  }
  return i == 0 ? "fwd" : "merge";
}

template <class T>
const T* section(const void* meta, int64_t off) {
  return reinterpret_cast<const T*>(static_cast<const int32_t*>(meta) + off);
}

}  // namespace

extern "C" {

bd_attn_status bd_attn_plan(const bd_attn_desc* desc, bd_attn_plan_t* out) {
  if (!out) return fail(BD_ATTN_EINVAL, "out is NULL");
  try {
    auto* h = new bd_attn_plan_s;
    std::string err;
    const bd_attn_status st = bdattn::build_plan(desc, &h->p, &err);
    if (st != BD_ATTN_OK) {
      delete h;
      return fail(st, err);
    }
    *out = h;
    return BD_ATTN_OK;
  } catch (const std::bad_alloc&) {
    return fail(BD_ATTN_EINVAL, "out of host memory while planning");
  } catch (...) {
    return fail(BD_ATTN_EINVAL, "unexpected error while planning");
  }
}

bd_attn_status bd_attn_plan_sizes(bd_attn_plan_t plan, int64_t* tq, int64_t* tk, size_t* meta_bytes,
                                  size_t* ws_fwd_bytes, size_t* ws_bwd_bytes, int64_t* visible_pairs) {
  if (!plan) return fail(BD_ATTN_EINVAL, "plan is NULL");
  const Plan& p = plan->p;
  if (tq) *tq = p.tq;
  if (tk) *tk = p.tk;
  if (meta_bytes) *meta_bytes = p.blob.size() * sizeof(int32_t);
  if (ws_fwd_bytes) *ws_fwd_bytes = p.ws_fwd;
  if (ws_bwd_bytes) *ws_bwd_bytes = p.ws_bwd;
  if (visible_pairs) *visible_pairs = p.pairs;
  return BD_ATTN_OK;
}

bd_attn_status bd_attn_plan_serialize(bd_attn_plan_t plan, void* meta_host, size_t bytes) {
  if (!plan) return fail(BD_ATTN_EINVAL, "plan is NULL");
  if (!meta_host) return fail(BD_ATTN_EINVAL, "meta_host is NULL");
  const size_t need = plan->p.blob.size() * sizeof(int32_t);
  if (bytes < need) return fail(BD_ATTN_EWORKSPACE, "meta_host buffer smaller than meta_bytes");
  std::memcpy(meta_host, plan->p.blob.data(), need);
  return BD_ATTN_OK;
}

bd_attn_status bd_attn_plan_check(bd_attn_plan_t plan, const void* meta_host, size_t bytes) {
  if (!plan) return fail(BD_ATTN_EINVAL, "plan is NULL");
  if (!meta_host) return fail(BD_ATTN_EINVAL, "meta_host is NULL");
  const size_t need = plan->p.blob.size() * sizeof(int32_t);
  if (bytes < need) return fail(BD_ATTN_EWORKSPACE, "meta_host buffer smaller than meta_bytes");
  std::string why;
  if (bdattn::check_blob(plan->p, static_cast<const int32_t*>(meta_host), need / sizeof(int32_t), &why) !=
      BD_ATTN_OK)
    return fail(BD_ATTN_EINVAL, why);
  return BD_ATTN_OK;
}

bd_attn_status bd_attn_device_check_errors(uint64_t* count, int reset) {
  if (!count) return fail(BD_ATTN_EINVAL, "count is NULL");
  uint64_t n = 0;
  hipError_t e = bdattn::device_errors_fwd(&n, reset != 0);
  if (e == hipSuccess) e = bdattn::device_errors_fwd_vt(&n, reset != 0);
  if (e == hipSuccess) e = bdattn::device_errors_bwd(&n, reset != 0);
  if (e == hipSuccess) e = bdattn::device_errors_dq(&n, reset != 0);
  if (e == hipSuccess) e = bdattn::device_errors_f32(&n, reset != 0);
  if (bd_attn_status st = hip_status(e, "device check counters")) return st;
  *count = n;
  return BD_ATTN_OK;
}

bd_attn_status bd_attn_plan_upload(bd_attn_plan_t plan, void* meta_dev, bd_attn_stream_t stream) {
  if (!plan) return fail(BD_ATTN_EINVAL, "plan is NULL");
  if (bd_attn_status st = check_ptr(meta_dev, "meta_dev")) return st;
  const size_t need = plan->p.blob.size() * sizeof(int32_t);
  return hip_status(hipMemcpyAsync(meta_dev, plan->p.blob.data(), need, hipMemcpyHostToDevice,
                                   reinterpret_cast<hipStream_t>(stream)),
                    "hipMemcpyAsync(meta)");
}

static bd_attn_status fwd_impl(bd_attn_plan_t plan, const void* meta_dev, const void* q, const void* k,
                               const void* v, void* o, float* lse, void* ws, bd_attn_stream_t stream,
                               void* const* events, int n_events) {
  if (!plan) return fail(BD_ATTN_EINVAL, "plan is NULL");
  const Plan& p = plan->p;
  if (events && n_events < fwd_kernels(p) + 1)
    return fail(BD_ATTN_EINVAL, "n_events must be at least the number of forward kernels + 1");
  bd_attn_status st;
  if ((st = check_ptr(meta_dev, "meta_dev")) || (st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) ||
      (st = check_ptr(v, "v")) || (st = check_ptr(o, "o")) || (st = check_ptr(lse, "lse")))
    return st;
  const bool bf16 = p.desc.dtype == BD_ATTN_BF16;
  const bool split = bf16 && p.split;
  if (p.ws_fwd > 0) {
    if (!ws) return fail(BD_ATTN_EWORKSPACE, "this plan needs a forward workspace (ws_fwd_bytes)");
    if (!aligned16(ws)) return fail(BD_ATTN_EINVAL, "ws is not 16-byte aligned");
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const EventMarks ev{events, events ? n_events : 0, s};
  bdattn::FwdArgs a{};
  a.qtiles = section<int32_t>(meta_dev, p.off_qtiles);
  a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
  a.hq = p.desc.num_q_heads; a.hkv = p.desc.num_kv_heads; a.G = p.G; a.grain = p.grain;
  a.scale = p.scale;
  a.scale_log2 = p.scale * 1.4426950408889634f;
  a.tq = p.tq; a.tk = p.tk;
  a.n_qtiles = (int)p.qtiles.size(); a.n_slots = (int)p.n_split_slots;
  a.checks = p.checks;
  const int D = p.desc.head_dim;
  hipError_t e;
  if ((st = hip_status(ev.mark(0), "hipEventRecord"))) return st;
  if (!bf16) {
    a.items = section<bdattn::FwdItem>(meta_dev, p.off_dq);
    e = bdattn::launch_fwd_f32(a, D, (int)p.dq_items.size(), s);
    if ((st = hip_status(e, "fwd_f32 launch"))) return st;
    return hip_status(ev.mark(1), "hipEventRecord");
  }
  a.items = section<bdattn::FwdItem>(meta_dev, p.off_fwd);
  int mark = 1;
  if (p.use_vt) {
    void* vt = static_cast<char*>(ws) + p.off_ws_vt;
    e = bdattn::launch_transpose_v(v, vt, (int)p.tk, (int)p.tk_pad, a.hkv, D, s);
    if ((st = hip_status(e, "transpose_v launch"))) return st;
    if ((st = hip_status(ev.mark(mark++), "hipEventRecord"))) return st;
    a.vt = vt;
    a.tk_pad = (int)p.tk_pad;
  }
  if (!split) {
    const int grid = (int)p.fwd_items.size();
    e = p.use_vt ? bdattn::launch_fwd_vt(a, D, grid, s) : bdattn::launch_fwd_bf16(a, D, grid, s);
    if ((st = hip_status(e, "fwd launch"))) return st;
    return hip_status(ev.mark(mark), "hipEventRecord");
  }
  a.splits = section<bdattn::SplitItem>(meta_dev, p.off_split);
  if (p.grid_parts > 0) {
    a.grid_qt = p.qtiles[0];
    a.grid_parts = p.grid_parts; a.grid_tps = p.grid_tps; a.grid_tiles = p.grid_tiles;
  }
  a.part_o = static_cast<char*>(ws) + p.off_ws_part;
  a.part_lse = reinterpret_cast<float*>(static_cast<char*>(ws) + p.off_ws_lse);
  const int grid = (int)p.split_items.size();
  e = p.use_vt ? bdattn::launch_fwd_split_vt(a, D, grid, s) : bdattn::launch_fwd_split_direct(a, D, grid, s);
  if ((st = hip_status(e, "fwd (split) launch"))) return st;
  if ((st = hip_status(ev.mark(mark++), "hipEventRecord"))) return st;
  bdattn::MergeArgs c{};
  c.items = section<bdattn::MergeItem>(meta_dev, p.off_merge);
  c.part_o = a.part_o; c.part_lse = a.part_lse; c.o = o; c.lse = lse;
  c.hq = a.hq; c.G = a.G;
  c.tq = p.tq; c.n_slots = (int)p.n_split_slots;
  c.checks = p.checks;
  e = bdattn::launch_merge(c, D, (int)p.merge_items.size(), s);
  if ((st = hip_status(e, "merge launch"))) return st;
  return hip_status(ev.mark(mark), "hipEventRecord");
}

bd_attn_status bd_attn_fwd(bd_attn_plan_t plan, const void* meta_dev, const void* q, const void* k,
                           const void* v, void* o, float* lse, void* ws, bd_attn_stream_t stream) {
  return fwd_impl(plan, meta_dev, q, k, v, o, lse, ws, stream, nullptr, 0);
}

bd_attn_status bd_attn_fwd_timed(bd_attn_plan_t plan, const void* meta_dev, const void* q, const void* k,
                                 const void* v, void* o, float* lse, void* ws, bd_attn_stream_t stream,
                                 void* const* events, int n_events) {
  if (!events) return fail(BD_ATTN_EINVAL, "events is NULL");
  return fwd_impl(plan, meta_dev, q, k, v, o, lse, ws, stream, events, n_events);
}

}  // extern "C"

namespace {

// Forward workspace of bd_attn_fwd_noalloc: a fixed array in the code object's
// device memory, so a call allocates nothing. Each GPU the library runs on holds
// its own copy until the process ends; host code only ever uses the address
// hipGetSymbolAddress returns for the device (the array's name is a host-side
// stand-in, not a device address).
static __device__ __align__(256) unsigned char scratch[BD_ATTN_NOALLOC_WS_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices];   // scratch's device address per GPU, looked up once

// Device address of scratch on the GPU that runs `stream`, looked up with that
// GPU current (restoring the caller's current device afterwards).
bd_attn_status scratch_for(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return hip_status(e, "hipStreamGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(BD_ATTN_EUNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return hip_status(e, "hipGetDevice");
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e, "hipSetDevice");
    void* p = nullptr;
    const hipError_t es = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev && (e = hipSetDevice(cur)) != hipSuccess) return hip_status(e, "hipSetDevice (restore)");
    if (es != hipSuccess) return hip_status(es, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(BD_ATTN_EHIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_dev[dev] = p;
  }
  *out = g_scratch_dev[dev];
  return BD_ATTN_OK;
}

}  // namespace

extern "C" {

bd_attn_status bd_attn_fwd_noalloc(bd_attn_plan_t plan, const void* meta_dev, const void* q, const void* k,
                                   const void* v, void* o, float* lse, bd_attn_stream_t stream) {
  if (!plan) return fail(BD_ATTN_EINVAL, "plan is NULL");
  if (plan->p.ws_fwd > (size_t)BD_ATTN_NOALLOC_WS_BYTES)
    return fail(BD_ATTN_EWORKSPACE, "the plan's forward workspace (" + std::to_string(plan->p.ws_fwd) +
                                        " bytes) exceeds the fixed array of bd_attn_fwd_noalloc (" +
                                        std::to_string((size_t)BD_ATTN_NOALLOC_WS_BYTES) + " bytes)");
  void* ws = nullptr;
  if (plan->p.ws_fwd > 0) {
    if (bd_attn_status st = scratch_for(reinterpret_cast<hipStream_t>(stream), &ws)) return st;
  }
  return fwd_impl(plan, meta_dev, q, k, v, o, lse, ws, stream, nullptr, 0);
}

static bd_attn_status bwd_impl(bd_attn_plan_t plan, const void* meta_dev, const void* q, const void* k,
                               const void* v, const void* o, const float* lse, const void* dout, void* dq,
                               void* dk, void* dv, void* ws, bd_attn_stream_t stream,
                               void* const* events, int n_events) {
  if (!plan) return fail(BD_ATTN_EINVAL, "plan is NULL");
  const Plan& p = plan->p;
  const int nk = bwd_kernels(p);
  if (events && n_events < nk + 1)
    return fail(BD_ATTN_EINVAL, "n_events must be at least bd_attn_plan_kernels(plan, 1) + 1");
  bd_attn_status st;
  if ((st = check_ptr(meta_dev, "meta_dev")) || (st = check_ptr(q, "q")) || (st = check_ptr(k, "k")) ||
      (st = check_ptr(v, "v")) || (st = check_ptr(o, "o")) || (st = check_ptr(lse, "lse")) ||
      (st = check_ptr(dout, "dout")) || (st = check_ptr(dq, "dq")) || (st = check_ptr(dk, "dk")) ||
      (st = check_ptr(dv, "dv")))
    return st;
  if (!ws) return fail(BD_ATTN_EWORKSPACE, "bd_attn_bwd needs a workspace of ws_bwd_bytes");
  if (!aligned16(ws)) return fail(BD_ATTN_EINVAL, "ws is not 16-byte aligned");
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const EventMarks ev{events, events ? n_events : 0, s};
  const bool bf16 = p.desc.dtype == BD_ATTN_BF16;
  const int D = p.desc.head_dim;
  bdattn::BwdArgs a{};
  a.qtiles = section<int32_t>(meta_dev, p.off_qtiles);
  a.dq_items = section<bdattn::FwdItem>(meta_dev, p.off_dq);
  a.ktiles = section<int32_t>(meta_dev, p.off_ktiles);
  a.canvq = section<bdattn::CanvasQ>(meta_dev, p.off_canvq);
  a.bwd_items = section<bdattn::BwdItem>(meta_dev, p.off_bwd);
  a.q = q; a.k = k; a.v = v; a.o = o; a.dout = dout; a.lse = lse;
  a.delta = static_cast<float*>(ws);
  a.lse2 = reinterpret_cast<float*>(static_cast<char*>(ws) + p.off_ws_lse2);
  a.dkv_part = reinterpret_cast<float*>(static_cast<char*>(ws) + p.off_ws_dkv);
  a.bmerge = section<bdattn::BwdMerge>(meta_dev, p.off_bmerge);
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.rows_q = p.tq * p.desc.num_q_heads;
  a.hq = p.desc.num_q_heads; a.hkv = p.desc.num_kv_heads; a.G = p.G; a.B = p.desc.block_size;
  a.grain = p.grain;
  a.scale = p.scale;
  a.scale_log2 = p.scale * 1.4426950408889634f;
  a.tq = p.tq; a.tk = p.tk;
  a.n_qtiles = (int)p.qtiles.size(); a.n_ktiles = (int)p.ktiles.size();
  a.n_canvq = (int)p.canvq.size(); a.n_dkv_slots = (int)p.n_dkv_slots;
  a.checks = p.checks;
  if ((st = hip_status(ev.mark(0), "hipEventRecord"))) return st;
  hipError_t e;
  if (bf16) {
    e = bdattn::launch_dq_bf16(a, D, (int)p.dq_items.size(), s);
    if ((st = hip_status(e, "dq launch"))) return st;
    if ((st = hip_status(ev.mark(1), "hipEventRecord"))) return st;
    e = bdattn::launch_dkdv_bf16(a, D, p.dkdv_masked, (int)p.bwd_items.size(), s);
    if ((st = hip_status(e, "dkdv launch"))) return st;
    if ((st = hip_status(ev.mark(2), "hipEventRecord"))) return st;
    if (p.bwd_merge.empty()) return BD_ATTN_OK;
    e = bdattn::launch_dkdv_merge(a, D, (int)p.bwd_merge.size(), s);
    if ((st = hip_status(e, "dkdv merge launch"))) return st;
    return hip_status(ev.mark(3), "hipEventRecord");
  }
  e = bdattn::launch_bwd_pre(a, D, bf16, s);
  if ((st = hip_status(e, "bwd_pre launch"))) return st;
  if ((st = hip_status(ev.mark(1), "hipEventRecord"))) return st;
  e = bdattn::launch_dkdv_f32(a, D, (int)p.bwd_items.size(), s);
  if ((st = hip_status(e, "dkdv launch"))) return st;
  if ((st = hip_status(ev.mark(2), "hipEventRecord"))) return st;
  e = bdattn::launch_dq_f32(a, D, (int)p.dq_items.size(), s);
  if ((st = hip_status(e, "dq launch"))) return st;
  return hip_status(ev.mark(3), "hipEventRecord");
}

bd_attn_status bd_attn_bwd(bd_attn_plan_t plan, const void* meta_dev, const void* q, const void* k,
                           const void* v, const void* o, const float* lse, const void* dout, void* dq,
                           void* dk, void* dv, void* ws, bd_attn_stream_t stream) {
  return bwd_impl(plan, meta_dev, q, k, v, o, lse, dout, dq, dk, dv, ws, stream, nullptr, 0);
}

bd_attn_status bd_attn_bwd_timed(bd_attn_plan_t plan, const void* meta_dev, const void* q, const void* k,
                                 const void* v, const void* o, const float* lse, const void* dout, void* dq,
                                 void* dk, void* dv, void* ws, bd_attn_stream_t stream,
                                 void* const* events, int n_events) {
  if (!events) return fail(BD_ATTN_EINVAL, "events is NULL");
  return bwd_impl(plan, meta_dev, q, k, v, o, lse, dout, dq, dk, dv, ws, stream, events, n_events);
}

int32_t bd_attn_plan_kernels(bd_attn_plan_t plan, int32_t backward) {
  if (!plan) return 0;
  return backward ? bwd_kernels(plan->p) : fwd_kernels(plan->p);
}

const char* bd_attn_plan_kernel_name(bd_attn_plan_t plan, int32_t backward, int32_t i) {
  if (!plan) return nullptr;
  return kernel_name(plan->p, backward != 0, i);
}

bd_attn_status bd_attn_plan_info(bd_attn_plan_t plan, bd_attn_plan_info_t* out) {
  if (!plan) return fail(BD_ATTN_EINVAL, "plan is NULL");
  if (!out) return fail(BD_ATTN_EINVAL, "out is NULL");
  const Plan& p = plan->p;
  bd_attn_plan_info_t r{};
  r.split = p.split ? 1 : 0;
  r.split_tiles = 0;
  for (const auto& it : p.split_items)
    if (it.kvh >= 0) r.split_tiles = std::max<int32_t>(r.split_tiles, it.kt_end - it.kt_begin);
  r.split_grid = p.grid_parts > 0 ? 1 : 0;
  r.fwd_vt = p.use_vt ? 1 : 0;
  r.dkdv_masked = p.dkdv_masked ? 1 : 0;
  r.debug_checks = p.checks ? 1 : 0;
  r.query_tiles = (int64_t)p.qtiles.size();
  r.key_tiles = (int64_t)p.ktiles.size();
  r.fwd_workgroups = (int64_t)(p.desc.dtype != BD_ATTN_BF16 ? p.dq_items.size()
                               : p.split ? p.split_items.size() : p.fwd_items.size());
  r.dq_workgroups = (int64_t)p.dq_items.size();
  r.dkdv_workgroups = (int64_t)p.bwd_items.size();
  r.dkdv_split_tiles = (int64_t)p.bwd_merge.size();
  *out = r;
  return BD_ATTN_OK;
}

bd_attn_status bd_attn_plan_destroy(bd_attn_plan_t plan) {
  delete plan;
  return BD_ATTN_OK;
}

namespace {

// Validated AEC launch geometry: workgroups per row and entries per split.
struct AecGeom {
  int nsplit = 1;
  int64_t chunk = 0;
  size_t ws = 0;          // workspace of the forward (partials) or the backward, the larger
  size_t ws_rows = 0;     // backward: byte offset of the row coefficients (after the state gradients)
};

bd_attn_status aec_geom(const bd_aec_desc* d, AecGeom* g) {
  if (!d) return fail(BD_ATTN_EINVAL, "desc is NULL");
  if (d->num_rows < 1) return fail(BD_ATTN_EINVAL, "num_rows must be >= 1");
  if (d->vocab < 2) return fail(BD_ATTN_EINVAL, "vocab must be >= 2");
  if (d->dtype != BD_ATTN_BF16 && d->dtype != BD_ATTN_FP32) return fail(BD_ATTN_EINVAL, "unknown dtype");
  const int epv = d->dtype == BD_ATTN_BF16 ? 8 : 4;
  if (d->row_stride < d->vocab || d->row_stride % epv)
    return fail(BD_ATTN_EINVAL, "row_stride must be >= vocab and a multiple of 8 (bf16) or 4 (fp32)");
  if (d->num_states < 0 || d->num_pairs < 0) return fail(BD_ATTN_EINVAL, "num_states and num_pairs must be >= 0");
  if (!(d->rho >= 0.f && d->rho <= 1.f)) return fail(BD_ATTN_EINVAL, "rho must lie in [0, 1]");
  if (d->gate_max != d->gate_max) return fail(BD_ATTN_EINVAL, "gate_max must not be NaN");
  // about 2048 workgroups in all, each split at least kAecMinChunk entries
  const int64_t V = d->vocab, N = d->num_rows;
  const int64_t max_split = std::max<int64_t>(1, V / bdattn::kAecMinChunk);
  const int64_t want = std::min<int64_t>(max_split, std::max<int64_t>(1, (2048 + N - 1) / N));
  int64_t chunk = (V + want - 1) / want;
  chunk = (chunk + epv - 1) / epv * epv;
  const int64_t nsplit = (V + chunk - 1) / chunk;
  if (N * nsplit > INT32_MAX) return fail(BD_ATTN_EINVAL, "num_rows too large");
  g->nsplit = (int)nsplit;
  g->chunk = chunk;
  const size_t ws_fwd = nsplit > 1 ? (size_t)(N * nsplit * 3 * sizeof(float)) : 0;
  g->ws_rows = ((size_t)std::max(d->num_states, 1) * sizeof(float) + 255) / 256 * 256;
  const size_t ws_bwd = g->ws_rows + (size_t)N * sizeof(float);
  g->ws = std::max(ws_fwd, ws_bwd);
  return BD_ATTN_OK;
}

bd_attn_status aec_impl(const bd_aec_desc* d, const void* logits, const uint8_t* unresolved,
                        const int32_t* state_rows, const int32_t* pair_next, const float* pair_h_source,
                        const float* pair_weight, float* lse, float* hbar, float* h_state, float* loss,
                        void* ws, bd_attn_stream_t stream, void* const* events, int n_events) {
  AecGeom g;
  bd_attn_status st;
  if ((st = aec_geom(d, &g))) return st;
  const int nk = 2;
  if (events && n_events < nk + 1) return fail(BD_ATTN_EINVAL, "n_events must be at least the number of kernels + 1");
  if ((st = check_ptr(logits, "logits"))) return st;
  if (!lse || !hbar || !loss) return fail(BD_ATTN_EINVAL, "lse, hbar and loss must not be NULL");
  if (d->num_states > 0 && (!unresolved || !state_rows || !h_state))
    return fail(BD_ATTN_EINVAL, "unresolved, state_rows and h_state must not be NULL when num_states > 0");
  if (d->num_pairs > 0 && (!pair_next || !pair_h_source || !pair_weight))
    return fail(BD_ATTN_EINVAL, "the pair arrays must not be NULL when num_pairs > 0");
  if (g.nsplit > 1 && !ws) return fail(BD_ATTN_EWORKSPACE, "this call needs a workspace (bd_aec_workspace)");
  if (ws && !aligned16(ws)) return fail(BD_ATTN_EINVAL, "ws is not 16-byte aligned");
  bdattn::AecArgs a{};
  a.logits = logits; a.row_stride = d->row_stride; a.n_rows = d->num_rows; a.vocab = d->vocab;
  a.nsplit = g.nsplit; a.chunk = g.chunk; a.part = static_cast<float*>(ws);
  a.lse = lse; a.hbar = hbar; a.unresolved = unresolved; a.state_rows = state_rows;
  a.n_states = d->num_states; a.pair_next = pair_next; a.pair_h_source = pair_h_source;
  a.pair_weight = pair_weight; a.n_pairs = d->num_pairs; a.rho = d->rho; a.gate_max = d->gate_max;
  a.h_state = h_state; a.loss = loss;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const EventMarks ev{events, events ? n_events : 0, s};
  int mark = 0;
  if ((st = hip_status(ev.mark(mark++), "hipEventRecord"))) return st;
  if ((st = hip_status(bdattn::launch_aec_entropy(a, d->dtype == BD_ATTN_BF16, s), "aec_entropy launch"))) return st;
  if ((st = hip_status(ev.mark(mark++), "hipEventRecord"))) return st;
  if ((st = hip_status(bdattn::launch_aec_reduce(a, s), "aec_reduce launch"))) return st;
  return hip_status(ev.mark(mark), "hipEventRecord");
}

bd_attn_status aec_bwd_impl(const bd_aec_desc* d, const void* logits, const uint8_t* unresolved,
                            const int32_t* state_rows, const int32_t* pair_next, const float* pair_h_source,
                            const float* pair_weight, const float* lse, const float* hbar, const float* h_state,
                            const float* grad_loss, void* dlogits, void* ws, bd_attn_stream_t stream,
                            void* const* events, int n_events) {
  AecGeom g;
  bd_attn_status st;
  if ((st = aec_geom(d, &g))) return st;
  if (events && n_events < 3) return fail(BD_ATTN_EINVAL, "n_events must be at least the number of kernels + 1");
  if ((st = check_ptr(logits, "logits")) || (st = check_ptr(dlogits, "dlogits"))) return st;
  if (!lse || !hbar || !grad_loss) return fail(BD_ATTN_EINVAL, "lse, hbar and grad_loss must not be NULL");
  if (d->num_states > 0 && (!unresolved || !state_rows || !h_state))
    return fail(BD_ATTN_EINVAL, "unresolved, state_rows and h_state must not be NULL when num_states > 0");
  if (d->num_pairs > 0 && (!pair_next || !pair_h_source || !pair_weight))
    return fail(BD_ATTN_EINVAL, "the pair arrays must not be NULL when num_pairs > 0");
  if (!ws) return fail(BD_ATTN_EWORKSPACE, "the backward needs a workspace (bd_aec_workspace)");
  if (!aligned16(ws)) return fail(BD_ATTN_EINVAL, "ws is not 16-byte aligned");
  bdattn::AecArgs a{};
  a.logits = logits; a.row_stride = d->row_stride; a.n_rows = d->num_rows; a.vocab = d->vocab;
  a.nsplit = g.nsplit; a.chunk = g.chunk;
  a.lse = const_cast<float*>(lse); a.hbar = const_cast<float*>(hbar);
  a.unresolved = unresolved; a.state_rows = state_rows; a.n_states = d->num_states;
  a.pair_next = pair_next; a.pair_h_source = pair_h_source; a.pair_weight = pair_weight;
  a.n_pairs = d->num_pairs; a.rho = d->rho; a.gate_max = d->gate_max;
  a.h_state = const_cast<float*>(h_state); a.grad_loss = grad_loss;
  a.state_grad = static_cast<float*>(ws);
  a.row_coef = reinterpret_cast<float*>(static_cast<char*>(ws) + g.ws_rows);
  a.dlogits = dlogits;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const EventMarks ev{events, events ? n_events : 0, s};
  if ((st = hip_status(ev.mark(0), "hipEventRecord"))) return st;
  if ((st = hip_status(bdattn::launch_aec_grad_coef(a, s), "aec_grad_coef launch"))) return st;
  if ((st = hip_status(ev.mark(1), "hipEventRecord"))) return st;
  if ((st = hip_status(bdattn::launch_aec_grad(a, d->dtype == BD_ATTN_BF16, s), "aec_grad launch"))) return st;
  return hip_status(ev.mark(2), "hipEventRecord");
}

}  // namespace

bd_attn_status bd_aec_bwd(const bd_aec_desc* desc, const void* logits, const uint8_t* unresolved,
                          const int32_t* state_rows, const int32_t* pair_next, const float* pair_h_source,
                          const float* pair_weight, const float* lse, const float* hbar, const float* h_state,
                          const float* grad_loss, void* dlogits, void* ws, bd_attn_stream_t stream) {
  return aec_bwd_impl(desc, logits, unresolved, state_rows, pair_next, pair_h_source, pair_weight, lse, hbar,
                      h_state, grad_loss, dlogits, ws, stream, nullptr, 0);
}

bd_attn_status bd_aec_bwd_timed(const bd_aec_desc* desc, const void* logits, const uint8_t* unresolved,
                                const int32_t* state_rows, const int32_t* pair_next, const float* pair_h_source,
                                const float* pair_weight, const float* lse, const float* hbar,
                                const float* h_state, const float* grad_loss, void* dlogits, void* ws,
                                bd_attn_stream_t stream, void* const* events, int n_events) {
  return aec_bwd_impl(desc, logits, unresolved, state_rows, pair_next, pair_h_source, pair_weight, lse, hbar,
                      h_state, grad_loss, dlogits, ws, stream, events, n_events);
}

bd_attn_status bd_aec_workspace(const bd_aec_desc* desc, size_t* ws_bytes) {
  AecGeom g;
  bd_attn_status st;
  if ((st = aec_geom(desc, &g))) return st;
  if (ws_bytes) *ws_bytes = g.ws;
  return BD_ATTN_OK;
}

bd_attn_status bd_aec_fwd(const bd_aec_desc* desc, const void* logits, const uint8_t* unresolved,
                          const int32_t* state_rows, const int32_t* pair_next, const float* pair_h_source,
                          const float* pair_weight, float* lse, float* hbar, float* h_state, float* loss,
                          void* ws, bd_attn_stream_t stream) {
  return aec_impl(desc, logits, unresolved, state_rows, pair_next, pair_h_source, pair_weight, lse, hbar,
                  h_state, loss, ws, stream, nullptr, 0);
}

bd_attn_status bd_aec_fwd_timed(const bd_aec_desc* desc, const void* logits, const uint8_t* unresolved,
                                const int32_t* state_rows, const int32_t* pair_next, const float* pair_h_source,
                                const float* pair_weight, float* lse, float* hbar, float* h_state, float* loss,
                                void* ws, bd_attn_stream_t stream, void* const* events, int n_events) {
  return aec_impl(desc, logits, unresolved, state_rows, pair_next, pair_h_source, pair_weight, lse, hbar,
                  h_state, loss, ws, stream, events, n_events);
}

int32_t bd_aec_kernels(const bd_aec_desc* desc) {
  AecGeom g;
  const std::string keep = g_last_error;
  if (aec_geom(desc, &g) != BD_ATTN_OK) { g_last_error = keep; return 0; }
  return 2;
}

bd_attn_status bd_attn_pack(const bd_pack_desc* desc, bd_pack_out* out) {
  std::string err;
  try {
    const bd_attn_status st = bdattn::build_pack(desc, out, &err);
    if (st != BD_ATTN_OK) return fail(st, err);
  } catch (const std::bad_alloc&) {
    return fail(BD_ATTN_EINVAL, "out of host memory while packing");
  }
  return BD_ATTN_OK;
}

const char* bd_attn_last_error(void) { return g_last_error.c_str(); }

const char* bd_attn_version(void) { return "0.1.0"; }

}  // extern "C"
