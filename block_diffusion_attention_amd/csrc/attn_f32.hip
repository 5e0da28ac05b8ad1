// fp32 path of the staircase block-diffusion attention (true fp32 multiply-adds
// on the vector ALUs; no reduced-precision operands). It consumes the same work
// lists as the bf16 MFMA kernels, so it exercises the same planner ranges:
//   forward and dQ: one thread per query row of a query tile, K/V tiles staged
//                   in LDS;
//   dK / dV       : one thread per key of a key tile, query rows staged in LDS.
// Same mathematics as the bf16 path (ORL paper, section 3.2 "Staircase attention
// kernel" and the appendix D.2 paragraph on the kernel).
#include "kcommon.h"
#include "kernels.h"

namespace bdattn {

namespace {

constexpr int kF32Tile = 32;   // keys per LDS stage

// Key-tile geometry over the two visible ranges of a query tile, in kF32Tile units.
struct F32Ranges {
  int n1, n2;
  __device__ F32Ranges(const QTile& qt)
      : n1((qt.lim_max + kF32Tile - 1) / kF32Tile), n2((qt.n_own + kF32Tile - 1) / kF32Tile) {}
};

template <int D, bool CHK>
__global__ void __launch_bounds__(128) fwd_f32_kernel(FwdArgs a) {
  __shared__ float sK[kF32Tile][D];
  __shared__ float sV[kF32Tile][D];
  const int4 itv = reinterpret_cast<const int4*>(a.items)[blockIdx.x];
  if (itv.x < 0) return;
  if (reject_record<CHK>(itv.x >= a.n_qtiles)) return;
  const int kvh = itv.y;
  const QTile qt = load_qtile(a.qtiles, itv.x);
  if (reject_record<CHK>(kvh < 0 || kvh >= a.hkv || !qtile_in_bounds(qt, a.G, a.tq, a.tk))) return;
  const float* __restrict__ Q = static_cast<const float*>(a.q);
  const float* __restrict__ K = static_cast<const float*>(a.k);
  const float* __restrict__ V = static_cast<const float*>(a.v);
  const int G = a.G, row = threadIdx.x;
  int t = row / G;
  const int gh = row - t * G;
  const bool row_ok = row < qt.n_tok * G;
  if (t >= qt.n_tok) t = qt.n_tok - 1;
  const int64_t qrow = (int64_t)(qt.q_tok + t) * a.hq + kvh * G + gh;
  float q[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) { q[d] = Q[qrow * D + d]; acc[d] = 0.f; }
  const int L = row_limit(qt, t, a.grain);
  const F32Ranges rg(qt);
  float m = -INFINITY, l = 0.f;
  for (int kt = 0; kt < rg.n1 + rg.n2; ++kt) {
    const bool r1 = kt < rg.n1;
    const int kpos0 = r1 ? kt * kF32Tile : (kt - rg.n1) * kF32Tile;
    const int base = r1 ? qt.k_ctx + kpos0 : qt.k_own + kpos0;
    const int nvalid = min(kF32Tile, (r1 ? qt.lim_max : qt.n_own) - kpos0);
    const int lim = r1 ? L : qt.n_own;
    __syncthreads();
    for (int u = threadIdx.x; u < kF32Tile * D; u += blockDim.x) {
      const int kk = u / D, d = u - kk * D;
      float kv = 0.f, vv = 0.f;
      if (kk < nvalid) {
        const int64_t off = ((int64_t)(base + kk) * a.hkv + kvh) * D + d;
        kv = K[off]; vv = V[off];
      }
      sK[kk][d] = kv; sV[kk][d] = vv;
    }
    __syncthreads();
    for (int kk = 0; kk < nvalid; ++kk) {
      if (kpos0 + kk >= lim) break;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s = fmaf(q[d], sK[kk][d], s);
      s *= a.scale;
      const float mn = fmaxf(m, s);
      const float alpha = expf(m - mn);   // m = -inf on the first key -> 0
      const float p = expf(s - mn);
      l = l * alpha + p;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(p, sV[kk][d], acc[d] * alpha);
      m = mn;
    }
  }
  if (row_ok) {
    float* o = static_cast<float*>(a.o) + qrow * D;
    const float inv = 1.f / l;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] = acc[d] * inv;
    a.lse[qrow] = m + logf(l);
  }
}

template <int D, bool CHK>
__global__ void __launch_bounds__(128) dq_f32_kernel(BwdArgs a) {
  __shared__ float sK[kF32Tile][D];
  __shared__ float sV[kF32Tile][D];
  const int4 itv = reinterpret_cast<const int4*>(a.dq_items)[blockIdx.x];
  if (itv.x < 0) return;
  if (reject_record<CHK>(itv.x >= a.n_qtiles)) return;
  const int kvh = itv.y;
  const QTile qt = load_qtile(a.qtiles, itv.x);
  if (reject_record<CHK>(kvh < 0 || kvh >= a.hkv || !qtile_in_bounds(qt, a.G, a.tq, a.tk))) return;
  const float* __restrict__ Q = static_cast<const float*>(a.q);
  const float* __restrict__ K = static_cast<const float*>(a.k);
  const float* __restrict__ V = static_cast<const float*>(a.v);
  const float* __restrict__ dO = static_cast<const float*>(a.dout);
  const int G = a.G, row = threadIdx.x;
  int t = row / G;
  const int gh = row - t * G;
  const bool row_ok = row < qt.n_tok * G;
  if (t >= qt.n_tok) t = qt.n_tok - 1;
  const int64_t qrow = (int64_t)(qt.q_tok + t) * a.hq + kvh * G + gh;
  float q[D], g[D], acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) { q[d] = Q[qrow * D + d]; g[d] = dO[qrow * D + d]; acc[d] = 0.f; }
  const float lse = a.lse[qrow], dl = a.delta[qrow];
  const int L = row_limit(qt, t, a.grain);
  const F32Ranges rg(qt);
  for (int kt = 0; kt < rg.n1 + rg.n2; ++kt) {
    const bool r1 = kt < rg.n1;
    const int kpos0 = r1 ? kt * kF32Tile : (kt - rg.n1) * kF32Tile;
    const int base = r1 ? qt.k_ctx + kpos0 : qt.k_own + kpos0;
    const int nvalid = min(kF32Tile, (r1 ? qt.lim_max : qt.n_own) - kpos0);
    const int lim = r1 ? L : qt.n_own;
    __syncthreads();
    for (int u = threadIdx.x; u < kF32Tile * D; u += blockDim.x) {
      const int kk = u / D, d = u - kk * D;
      float kv = 0.f, vv = 0.f;
      if (kk < nvalid) {
        const int64_t off = ((int64_t)(base + kk) * a.hkv + kvh) * D + d;
        kv = K[off]; vv = V[off];
      }
      sK[kk][d] = kv; sV[kk][d] = vv;
    }
    __syncthreads();
    for (int kk = 0; kk < nvalid; ++kk) {
      if (kpos0 + kk >= lim) break;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) { s = fmaf(q[d], sK[kk][d], s); dp = fmaf(g[d], sV[kk][d], dp); }
      const float p = expf(s * a.scale - lse);
      const float ds = p * (dp - dl);
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] = fmaf(ds, sK[kk][d], acc[d]);
    }
  }
  if (row_ok) {
    float* o = static_cast<float*>(a.dq) + qrow * D;
#pragma unroll
    for (int d = 0; d < D; ++d) o[d] = acc[d] * a.scale;
  }
}

// dK/dV: thread = key of the tile; the query rows of each chunk are staged in LDS.
template <int D, bool CHK>
__global__ void __launch_bounds__(128) dkdv_f32_kernel(BwdArgs a) {
  constexpr int R = 8;                      // query rows per stage
  __shared__ float sQ[R][D];
  __shared__ float sG[R][D];
  __shared__ float sL[R], sDl[R];
  __shared__ int sLim[R];
  const int4 itv = reinterpret_cast<const int4*>(a.bwd_items)[blockIdx.x];
  if (itv.x < 0) return;
  if (reject_record<CHK>(itv.x >= a.n_ktiles || itv.y < 0 || itv.y >= a.hkv)) return;   // fp32 tiles are never split
  const int kvh = itv.y;
  const KTile kt = load_ktile(a.ktiles, itv.x);
  if (CHK && reject_record<CHK>(!ktile_in_bounds(kt, a.tq, a.tk, a.n_canvq) ||
                                !ktile_canvq_in_bounds(kt, a.canvq, a.B, a.tq)))
    return;
  const float* __restrict__ Q = static_cast<const float*>(a.q);
  const float* __restrict__ K = static_cast<const float*>(a.k);
  const float* __restrict__ V = static_cast<const float*>(a.v);
  const float* __restrict__ dO = static_cast<const float*>(a.dout);
  const int G = a.G, B = a.B;
  const int kidx = threadIdx.x;
  const bool key_ok = kidx < kt.n_keys;
  const int64_t krow = (int64_t)(kt.k_tok + min(kidx, kt.n_keys - 1)) * a.hkv + kvh;
  const float* kp = K + krow * D;
  const float* vp = V + krow * D;
  const int kpos = kt.p0 >= 0 ? kt.p0 + kidx : -1;
  float dk[D], dv[D];
#pragma unroll
  for (int d = 0; d < D; ++d) { dk[d] = 0.f; dv[d] = 0.f; }

  // the query stream: clean range, then each canvas entry, as (token, head) rows
  const int n_clean_rows = kt.cq_len * G;
  const int n_rows = n_clean_rows + kt.cv_count * B * G;
  for (int r0 = 0; r0 < n_rows; r0 += R) {
    __syncthreads();
    for (int u = threadIdx.x; u < R * D; u += blockDim.x) {
      const int rr = u / D, d = u - rr * D, r = r0 + rr;
      float qv = 0.f, gv = 0.f;
      if (r < n_rows) {
        int tok, gh;
        if (r < n_clean_rows) { tok = kt.cq_tok + r / G; gh = r % G; }
        else {
          const int rc = r - n_clean_rows, e = rc / (B * G), w = rc - e * B * G;
          tok = a.canvq[kt.cv_begin + e].q_tok + w / G; gh = w % G;
        }
        const int64_t off = ((int64_t)tok * a.hq + kvh * G + gh) * D + d;
        qv = Q[off]; gv = dO[off];
      }
      sQ[rr][d] = qv; sG[rr][d] = gv;
    }
    if (threadIdx.x < R) {
      const int r = r0 + threadIdx.x;
      float lv = 0.f, dv0 = 0.f;
      int lim = -1;                          // -1: row absent
      if (r < n_rows) {
        int tok, gh;
        if (r < n_clean_rows) {
          tok = kt.cq_tok + r / G; gh = r % G;
          lim = ((kt.cq_pos + r / G) / a.grain + 1) * a.grain;
        } else {
          const int rc = r - n_clean_rows, e = rc / (B * G), w = rc - e * B * G;
          const CanvasQ cq = a.canvq[kt.cv_begin + e];
          tok = cq.q_tok + w / G; gh = w % G;
          lim = cq.own ? 0x7fffffff : cq.lim;
        }
        const int64_t qr = (int64_t)tok * a.hq + kvh * G + gh;
        lv = a.lse[qr]; dv0 = a.delta[qr];
      }
      sL[threadIdx.x] = lv; sDl[threadIdx.x] = dv0; sLim[threadIdx.x] = lim;
    }
    __syncthreads();
    if (!key_ok) continue;
    for (int rr = 0; rr < R; ++rr) {
      const int lim = sLim[rr];
      if (lim < 0) break;
      if (kpos >= 0 && kpos >= lim) continue;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) { s = fmaf(sQ[rr][d], kp[d], s); dp = fmaf(sG[rr][d], vp[d], dp); }
      const float p = expf(s * a.scale - sL[rr]);
      const float ds = p * (dp - sDl[rr]);
#pragma unroll
      for (int d = 0; d < D; ++d) { dk[d] = fmaf(ds, sQ[rr][d], dk[d]); dv[d] = fmaf(p, sG[rr][d], dv[d]); }
    }
  }
  if (key_ok) {
    float* dkp = static_cast<float*>(a.dk) + krow * D;
    float* dvp = static_cast<float*>(a.dv) + krow * D;
#pragma unroll
    for (int d = 0; d < D; ++d) { dkp[d] = dk[d] * a.scale; dvp[d] = dv[d]; }
  }
}

}  // namespace

// Launches kernel template K<D, CHK> for the head dimension and check mode.
#define BD_F32_LAUNCH(K, a, head_dim, grid, s)                                                        \
  do {                                                                                             \
    const dim3 g_(grid), b_(128);                                                                  \
    if (head_dim == 128) {                                                                         \
      if ((a).checks) hipLaunchKernelGGL((K<128, true>), g_, b_, 0, s, a);                          \
      else hipLaunchKernelGGL((K<128, false>), g_, b_, 0, s, a);                                    \
    } else {                                                                                       \
      if ((a).checks) hipLaunchKernelGGL((K<64, true>), g_, b_, 0, s, a);                           \
      else hipLaunchKernelGGL((K<64, false>), g_, b_, 0, s, a);                                     \
    }                                                                                              \
  } while (0)

hipError_t launch_fwd_f32(const FwdArgs& a, int head_dim, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  BD_F32_LAUNCH(fwd_f32_kernel, a, head_dim, grid, s);
  return hipGetLastError();
}

hipError_t launch_dq_f32(const BwdArgs& a, int head_dim, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  BD_F32_LAUNCH(dq_f32_kernel, a, head_dim, grid, s);
  return hipGetLastError();
}

hipError_t launch_dkdv_f32(const BwdArgs& a, int head_dim, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  BD_F32_LAUNCH(dkdv_f32_kernel, a, head_dim, grid, s);
  return hipGetLastError();
}

BD_ATTN_DEVICE_ERRORS_QUERY(device_errors_f32)

}  // namespace bdattn
