// Backward staircase block-diffusion attention for gfx950 (bf16 in, fp32 accumulate).
//
// Three deterministic kernels, no atomics (ORL paper, appendix D.2 paragraph
// on the kernel: the backward pass uses the same visibility, dQ follows the
// query traversal and dK/dV derive the valid query ranges of each key tile):
//   bwd_pre : delta = rowsum(dO * O) per (token, query head), fp32;
//   dkdv    : one workgroup per (key tile of up to 128 keys, kv head), looping
//             over the query chunks that can see the tile; each wave owns 32 keys;
//   dq      : one workgroup per (query tile, kv head), looping over the same key
//             tiles as the forward pass.
// Gradients of L = <dO, O>: dp = dO V^T, ds = p (dp - delta), dQ = scale ds K,
// dK = scale ds^T Q, dV = p^T dO (dK, dV summed over the heads of a kv group).
#include "kcommon.h"
#include "kernels.h"

namespace bdattn {

namespace {

// ---------------------------------------------------------------- bwd_pre
template <int D, bool BF16>
__global__ void __launch_bounds__(256) bwd_pre_kernel(BwdArgs a) {
  constexpr int EPL = BF16 ? 8 : 4;            // elements per 16-byte load
  constexpr int LPR = D / EPL;                 // lanes per row
  constexpr int RPB = 256 / LPR;               // rows per block
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int c = threadIdx.x % LPR;
  float s = 0.f;
  if (row < a.rows_q) {
    if (BF16) {
      const u32x4 o = *reinterpret_cast<const u32x4*>(static_cast<const bf16*>(a.o) + row * D + c * 8);
      const u32x4 g = *reinterpret_cast<const u32x4*>(static_cast<const bf16*>(a.dout) + row * D + c * 8);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        s += __builtin_bit_cast(float, o[w] << 16) * __builtin_bit_cast(float, g[w] << 16);
        s += __builtin_bit_cast(float, o[w] & 0xffff0000u) * __builtin_bit_cast(float, g[w] & 0xffff0000u);
      }
    } else {
      const f32x4 o = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.o) + row * D + c * 4);
      const f32x4 g = *reinterpret_cast<const f32x4*>(static_cast<const float*>(a.dout) + row * D + c * 4);
      s = o[0] * g[0] + o[1] * g[1] + o[2] * g[2] + o[3] * g[3];
    }
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off, LPR);
  if (row < a.rows_q && c == 0) a.delta[row] = s;
}

// Geometry of query chunk c of a key tile: chunks of the clean range first,
// then those of each canvas entry (largest block index first).
struct ChunkGeom {
  int tok0;      // first packed query token
  int ntok;      // tokens in the chunk
  int pos0;      // context position of tok0 (clean) or -1
  int lim;       // canvas: b*B (or INT_MAX for the canvas' own keys)
};

__device__ __forceinline__ ChunkGeom chunk_geom(const KTile& kt, const CanvasQ* __restrict__ cv, int c,
                                                int nc0, int cpc, int qct) {
  ChunkGeom g;
  if (c < nc0) {
    g.tok0 = kt.cq_tok + c * qct;
    g.ntok = min(qct, kt.cq_len - c * qct);
    g.pos0 = kt.cq_pos + c * qct;
    g.lim = 0;
  } else {
    const int cc = c - nc0;
    const int e = cc / cpc, sub = cc - e * cpc;
    const int4 ev = reinterpret_cast<const int4*>(cv)[kt.cv_begin + e];
    g.tok0 = ev.x + sub * qct;
    g.ntok = min(qct, ev.y - sub * qct);
    g.pos0 = -1;
    g.lim = ev.w ? 0x7fffffff : ev.z;
  }
  return g;
}

// ---------------------------------------------------------------- dK / dV
template <int D>
__global__ void __launch_bounds__(256, 2) dkdv_bf16_kernel(BwdArgs a) {
  constexpr int NKS = D / 16, NDB = D / 32, CH = D / 8;
  constexpr int RG = D / 64;                   // rows per loader thread (32 rows x CH chunks / 256)
  constexpr int QC = kQChunk;
  __shared__ __attribute__((aligned(16))) bf16 sQ[QC * NatTile<D>::kStride];
  __shared__ __attribute__((aligned(16))) bf16 sdO[QC * NatTile<D>::kStride];
  __shared__ __attribute__((aligned(16))) bf16 sQt[D * QC];
  __shared__ __attribute__((aligned(16))) bf16 sdOt[D * QC];
  __shared__ __attribute__((aligned(16))) float sL[QC];
  __shared__ __attribute__((aligned(16))) float sDl[QC];
  __shared__ __attribute__((aligned(16))) int sLim[QC];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 31, h = lane >> 5;
  const int4 itv = reinterpret_cast<const int4*>(a.bwd_items)[blockIdx.x];
  if (itv.x < 0) return;
  const int kvh = itv.y;
  const KTile kt = load_ktile(a.ktiles, itv.x);
  const bf16* __restrict__ Q = static_cast<const bf16*>(a.q);
  const bf16* __restrict__ K = static_cast<const bf16*>(a.k);
  const bf16* __restrict__ V = static_cast<const bf16*>(a.v);
  const bf16* __restrict__ dO = static_cast<const bf16*>(a.dout);
  const int G = a.G, B = a.B;

  // this lane's key (column j of the wave's 32 keys)
  const int kidx = wave * 32 + j;
  const bool key_ok = kidx < kt.n_keys;
  const bool wave_live = wave * 32 < kt.n_keys;
  const int64_t krow = (int64_t)(kt.k_tok + min(kidx, kt.n_keys - 1)) * a.hkv + kvh;
  bf16x8 kf[NKS], vf[NKS];
#pragma unroll
  for (int kk = 0; kk < NKS; ++kk) {
    kf[kk] = *reinterpret_cast<const bf16x8*>(K + krow * D + kk * 16 + h * 8);
    vf[kk] = *reinterpret_cast<const bf16x8*>(V + krow * D + kk * 16 + h * 8);
  }
  const int kpos = kt.p0 >= 0 ? kt.p0 + kidx : 0;
  const int wpos_lo = kt.p0 + wave * 32;                // lowest key position of the wave
  const int wpos_hi = kt.p0 + min(wave * 32 + 31, kt.n_keys - 1);

  f32x16 dkt[NDB], dvt[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) { dkt[db] = f32x16{}; dvt[db] = f32x16{}; }

  const int qct = QC / G;                               // tokens per chunk
  const int nc0 = (kt.cq_len + qct - 1) / qct;
  const int cpc = (B + qct - 1) / qct;
  const int nchunks = nc0 + kt.cv_count * cpc;

  // loader: rows lg*RG.. of the chunk, 16-byte chunk lc
  const int lc = tid % CH, lg = tid / CH;
  u32x4 pq[RG], pd[RG];
  float p_l = 0.f, p_dl = 0.f;
  int p_lim = 0;
  auto load_chunk = [&](int c) {
    const ChunkGeom g = chunk_geom(kt, a.canvq, c, nc0, cpc, qct);
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      const int r = lg * RG + i;
      const int t = r / G, gh = r - (r / G) * G;
      if (t < g.ntok && r < qct * G) {
        const int64_t off = ((int64_t)(g.tok0 + t) * a.hq + kvh * G + gh) * D + lc * 8;
        pq[i] = *reinterpret_cast<const u32x4*>(Q + off);
        pd[i] = *reinterpret_cast<const u32x4*>(dO + off);
      } else {
        pq[i] = u32x4{0, 0, 0, 0};
        pd[i] = u32x4{0, 0, 0, 0};
      }
    }
    if (tid < QC) {
      const int r = tid, t = r / G, gh = r - (r / G) * G;
      if (t < g.ntok && r < qct * G) {
        const int64_t qr = (int64_t)(g.tok0 + t) * a.hq + kvh * G + gh;
        p_l = a.lse[qr] * kLog2e;
        p_dl = a.delta[qr];
        p_lim = g.pos0 >= 0 ? ((g.pos0 + t) / B + 1) * B : g.lim;
      } else {
        p_l = INFINITY; p_dl = 0.f; p_lim = 0;
      }
    }
  };
  auto store_chunk = [&]() {
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      *reinterpret_cast<u32x4*>(sQ + NatTile<D>::off(lg * RG + i, lc * 8)) = pq[i];
      *reinterpret_cast<u32x4*>(sdO + NatTile<D>::off(lg * RG + i, lc * 8)) = pd[i];
    }
    const int col = kperm(lg * RG);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = lc * 8 + e, w = e >> 1;
      if constexpr (RG == 2) {
        *reinterpret_cast<uint32_t*>(sQt + TrTile<QC>::off(d, col)) = pick_pair(pq[0][w], pq[1][w], e & 1);
        *reinterpret_cast<uint32_t*>(sdOt + TrTile<QC>::off(d, col)) = pick_pair(pd[0][w], pd[1][w], e & 1);
      } else {
        sQt[TrTile<QC>::off(d, col)] = __builtin_bit_cast(bf16, (uint16_t)((e & 1) ? (pq[0][w] >> 16) : (pq[0][w] & 0xffffu)));
        sdOt[TrTile<QC>::off(d, col)] = __builtin_bit_cast(bf16, (uint16_t)((e & 1) ? (pd[0][w] >> 16) : (pd[0][w] & 0xffffu)));
      }
    }
    if (tid < QC) { sL[tid] = p_l; sDl[tid] = p_dl; sLim[tid] = p_lim; }
  };

  if (nchunks > 0) load_chunk(0);
  for (int c = 0; c < nchunks; ++c) {
    __syncthreads();
    store_chunk();
    __syncthreads();
    const ChunkGeom g = chunk_geom(kt, a.canvq, c, nc0, cpc, qct);
    if (c + 1 < nchunks) load_chunk(c + 1);

    // visibility of this chunk for the wave's keys
    int lim_lo, lim_hi;
    if (g.pos0 >= 0) { lim_lo = (g.pos0 / B + 1) * B; lim_hi = ((g.pos0 + g.ntok - 1) / B + 1) * B; }
    else { lim_lo = lim_hi = g.lim; }
    const bool canvas_keys = kt.p0 < 0;
    const bool skip = !wave_live || (!canvas_keys && wpos_lo >= lim_hi);
    const bool need_mask = !canvas_keys && wpos_hi >= lim_lo;
    if (skip) continue;

    f32x16 s = f32x16{}, dp = f32x16{};
    const bf16* qp = sQ + NatTile<D>::off(j, h * 8);
    const bf16* gp = sdO + NatTile<D>::off(j, h * 8);
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk) {
      s = mfma32(*reinterpret_cast<const bf16x8*>(qp + kk * 16), kf[kk], s);
      dp = mfma32(*reinterpret_cast<const bf16x8*>(gp + kk * 16), vf[kk], dp);
    }
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int r0 = 8 * g4 + 4 * h;
      const f32x4 lv = *reinterpret_cast<const f32x4*>(sL + r0);
      const f32x4 dv = *reinterpret_cast<const f32x4*>(sDl + r0);
      const int4 mv = *reinterpret_cast<const int4*>(sLim + r0);
      const int lims[4] = {mv.x, mv.y, mv.z, mv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = g4 * 4 + e;
        float x = s[r] * a.scale_log2 - lv[e];
        if (need_mask && kpos >= lims[e]) x = -INFINITY;
        const float p = fast_exp2(x);
        s[r] = p;
        dp[r] = p * (dp[r] - dv[e]);
      }
    }
    bf16x8 pb[2], sb[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float t0[8], t1[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) { t0[e] = s[ks * 8 + e]; t1[e] = dp[ks * 8 + e]; }
      pb[ks] = pack8(t0);
      sb[ks] = pack8(t1);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = db * 32 + j;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        dvt[db] = mfma32(*reinterpret_cast<const bf16x8*>(sdOt + TrTile<QC>::off(d, ks * 16 + h * 8)), pb[ks], dvt[db]);
        dkt[db] = mfma32(*reinterpret_cast<const bf16x8*>(sQt + TrTile<QC>::off(d, ks * 16 + h * 8)), sb[ks], dkt[db]);
      }
    }
  }

  if (key_ok) {
    bf16* dkp = static_cast<bf16*>(a.dk) + krow * D;
    bf16* dvp = static_cast<bf16*>(a.dv) + krow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + g4 * 8 + h * 4;
        u32x2 vk, vv;
        vk[0] = pack_bf16x2(dkt[db][g4 * 4 + 0] * a.scale, dkt[db][g4 * 4 + 1] * a.scale);
        vk[1] = pack_bf16x2(dkt[db][g4 * 4 + 2] * a.scale, dkt[db][g4 * 4 + 3] * a.scale);
        vv[0] = pack_bf16x2(dvt[db][g4 * 4 + 0], dvt[db][g4 * 4 + 1]);
        vv[1] = pack_bf16x2(dvt[db][g4 * 4 + 2], dvt[db][g4 * 4 + 3]);
        *reinterpret_cast<u32x2*>(dkp + d0) = vk;
        *reinterpret_cast<u32x2*>(dvp + d0) = vv;
      }
  }
}

// ---------------------------------------------------------------- dQ
template <int D>
__global__ void __launch_bounds__(256, 2) dq_bf16_kernel(BwdArgs a) {
  constexpr int KT = kKTile;
  constexpr int NDB = D / 32, NKS = D / 16, CH = D / 8, KG = D / 32;
  __shared__ __attribute__((aligned(16))) bf16 sK[KT * NatTile<D>::kStride];
  __shared__ __attribute__((aligned(16))) bf16 sV[KT * NatTile<D>::kStride];
  __shared__ __attribute__((aligned(16))) bf16 sKt[D * KT];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 31, h = lane >> 5;
  const int4 itv = reinterpret_cast<const int4*>(a.dq_items)[blockIdx.x];
  if (itv.x < 0) return;
  const int kvh = itv.y, kt_begin = itv.z, kt_end = itv.w;
  const QTile qt = load_qtile(a.qtiles, itv.x);
  const bf16* __restrict__ Q = static_cast<const bf16*>(a.q);
  const bf16* __restrict__ K = static_cast<const bf16*>(a.k);
  const bf16* __restrict__ V = static_cast<const bf16*>(a.v);
  const bf16* __restrict__ dO = static_cast<const bf16*>(a.dout);

  const int G = a.G;
  const int row = wave * 32 + j;
  int t = row / G;
  const int gh = row - t * G;
  const bool row_ok = row < qt.n_tok * G;
  if (t >= qt.n_tok) t = qt.n_tok - 1;
  const int64_t qrow = (int64_t)(qt.q_tok + t) * a.hq + kvh * G + gh;
  bf16x8 qf[NKS], df[NKS];
#pragma unroll
  for (int kk = 0; kk < NKS; ++kk) {
    qf[kk] = *reinterpret_cast<const bf16x8*>(Q + qrow * D + kk * 16 + h * 8);
    df[kk] = *reinterpret_cast<const bf16x8*>(dO + qrow * D + kk * 16 + h * 8);
  }
  const float lse2 = a.lse[qrow] * kLog2e;
  const float dl = a.delta[qrow];
  const int L = row_limit(qt, t, a.B);
  const int n1 = (qt.lim_max + KT - 1) / KT;

  const int lc = tid % CH, lg = tid / CH;
  u32x4 pk[KG], pv[KG];
  auto load_tile = [&](int kt) {
    int base, nvalid;
    if (kt < n1) { base = qt.k_ctx + kt * KT; nvalid = min(KT, qt.lim_max - kt * KT); }
    else { const int k2 = kt - n1; base = qt.k_own + k2 * KT; nvalid = min(KT, qt.n_own - k2 * KT); }
#pragma unroll
    for (int i = 0; i < KG; ++i) {
      const int key = lg * KG + i;
      if (key < nvalid) {
        const int64_t off = ((int64_t)(base + key) * a.hkv + kvh) * D + lc * 8;
        pk[i] = *reinterpret_cast<const u32x4*>(K + off);
        pv[i] = *reinterpret_cast<const u32x4*>(V + off);
      } else {
        pk[i] = u32x4{0, 0, 0, 0};
        pv[i] = u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < KG; ++i) {
      *reinterpret_cast<u32x4*>(sK + NatTile<D>::off(lg * KG + i, lc * 8)) = pk[i];
      *reinterpret_cast<u32x4*>(sV + NatTile<D>::off(lg * KG + i, lc * 8)) = pv[i];
    }
    const int col = kperm(lg * KG);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = lc * 8 + e, w = e >> 1;
      if constexpr (KG == 4) {
        *reinterpret_cast<u32x2*>(sKt + TrTile<KT>::off(d, col)) =
            u32x2{pick_pair(pk[0][w], pk[1][w], e & 1), pick_pair(pk[2][w], pk[3][w], e & 1)};
      } else {
        *reinterpret_cast<uint32_t*>(sKt + TrTile<KT>::off(d, col)) = pick_pair(pk[0][w], pk[1][w], e & 1);
      }
    }
  };

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
  if (kt_begin < kt_end) load_tile(kt_begin);
  for (int kt = kt_begin; kt < kt_end; ++kt) {
    __syncthreads();
    store_tile();
    __syncthreads();
    const bool r1 = kt < n1;
    const int kpos0 = r1 ? kt * KT : (kt - n1) * KT;
    const int lim = r1 ? L : qt.n_own;
    const bool need_mask = kpos0 + KT > (r1 ? qt.lim_min : qt.n_own);
    if (kt + 1 < kt_end) load_tile(kt + 1);

    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      dp[kb] = f32x16{};
      const bf16* kp = sK + NatTile<D>::off(kb * 32 + j, h * 8);
      const bf16* vp = sV + NatTile<D>::off(kb * 32 + j, h * 8);
#pragma unroll
      for (int kk = 0; kk < NKS; ++kk) {
        s[kb] = mfma32(*reinterpret_cast<const bf16x8*>(kp + kk * 16), qf[kk], s[kb]);
        dp[kb] = mfma32(*reinterpret_cast<const bf16x8*>(vp + kk * 16), df[kk], dp[kb]);
      }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[kb][r] * a.scale_log2 - lse2;
        if (need_mask && (kpos0 + kb * 32 + c_row(r, h) >= lim)) x = -INFINITY;
        const float p = fast_exp2(x);
        dp[kb][r] = p * (dp[kb][r] - dl);
      }
    bf16x8 sb[4];
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      float tmp[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) tmp[e] = dp[kq >> 1][(kq & 1) * 8 + e];
      sb[kq] = pack8(tmp);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = db * 32 + j;
#pragma unroll
      for (int kq = 0; kq < 4; ++kq)
        acc[db] = mfma32(*reinterpret_cast<const bf16x8*>(sKt + TrTile<KT>::off(d, kq * 16 + h * 8)), sb[kq], acc[db]);
    }
  }
  if (row_ok) {
    bf16* op = static_cast<bf16*>(a.dq) + qrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        u32x2 v;
        v[0] = pack_bf16x2(acc[db][g4 * 4 + 0] * a.scale, acc[db][g4 * 4 + 1] * a.scale);
        v[1] = pack_bf16x2(acc[db][g4 * 4 + 2] * a.scale, acc[db][g4 * 4 + 3] * a.scale);
        *reinterpret_cast<u32x2*>(op + db * 32 + g4 * 8 + h * 4) = v;
      }
  }
}

}  // namespace

hipError_t launch_bwd_pre(const BwdArgs& a, int head_dim, bool bf16, hipStream_t s) {
  const int lpr = head_dim / (bf16 ? 8 : 4);
  const int rpb = 256 / lpr;
  const int64_t grid = (a.rows_q + rpb - 1) / rpb;
  if (grid <= 0) return hipSuccess;
  if (head_dim == 128) {
    if (bf16) hipLaunchKernelGGL((bwd_pre_kernel<128, true>), dim3((unsigned)grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((bwd_pre_kernel<128, false>), dim3((unsigned)grid), dim3(256), 0, s, a);
  } else {
    if (bf16) hipLaunchKernelGGL((bwd_pre_kernel<64, true>), dim3((unsigned)grid), dim3(256), 0, s, a);
    else hipLaunchKernelGGL((bwd_pre_kernel<64, false>), dim3((unsigned)grid), dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

hipError_t launch_dkdv_bf16(const BwdArgs& a, int head_dim, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (head_dim == 128) hipLaunchKernelGGL(dkdv_bf16_kernel<128>, dim3(grid), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(dkdv_bf16_kernel<64>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_dq_bf16(const BwdArgs& a, int head_dim, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (head_dim == 128) hipLaunchKernelGGL(dq_bf16_kernel<128>, dim3(grid), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(dq_bf16_kernel<64>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace bdattn
