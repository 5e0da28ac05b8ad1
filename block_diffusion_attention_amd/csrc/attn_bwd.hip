// Backward staircase block-diffusion attention for gfx950 (bf16 in, fp32 accumulate).
//
// Three deterministic kernels, no atomics (ORL paper, appendix D.2 paragraph
// on the kernel: the backward pass uses the same visibility, dQ follows the
// query traversal and dK/dV derive the valid query ranges of each key tile):
//   bwd_pre : delta = rowsum(dO * O) per (token, query head), fp32;
//   dkdv    : one workgroup per (key tile of up to 64 keys, kv head), looping
//             over the 64-row query chunks that can see the tile;
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
// Workgroup: one key tile of up to 64 keys and one kv head. Wave w owns keys
// 32*(w&1) .. +31 and, of every 64-row query chunk, rows 32*(w>>1) .. +31; the
// two waves that share keys add their partial dK/dV through LDS at the end.
// Query chunks (rows = tokens x grouped heads, with their LSE and delta) go
// from global memory straight into LDS, two chunks in flight. The transposed
// operands dO^T and Q^T of dV^T = dO^T P and dK^T = Q^T dS are read with the
// LDS transpose read from the natural tiles.
template <int D>
__global__ void __launch_bounds__(256, 1) dkdv_bf16_kernel(BwdArgs a) {
  constexpr int NKS = D / 16, NDB = D / 32;
  constexpr int QC = 64;                       // query rows per chunk
  constexpr int TE = QC * D;
  __shared__ __attribute__((aligned(1024))) bf16 sQ0[TE];
  __shared__ __attribute__((aligned(1024))) bf16 sG0[TE];
  __shared__ __attribute__((aligned(1024))) bf16 sQ1[TE];
  __shared__ __attribute__((aligned(1024))) bf16 sG1[TE];
  __shared__ __attribute__((aligned(256))) float sL0[QC], sD0[QC], sL1[QC], sD1[QC];
  __shared__ __attribute__((aligned(256))) int sM0[QC], sM1[QC];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 31, h = lane >> 5;
  const CmLane lo(lane);
  const int kg = wave & 1, qh = wave >> 1;
  const int4 itv = reinterpret_cast<const int4*>(a.bwd_items)[blockIdx.x];
  if (itv.x < 0) return;
  const int kvh = itv.y;
  const KTile kt = load_ktile(a.ktiles, itv.x);
  const bf16* __restrict__ Q = static_cast<const bf16*>(a.q);
  const bf16* __restrict__ K = static_cast<const bf16*>(a.k);
  const bf16* __restrict__ V = static_cast<const bf16*>(a.v);
  const bf16* __restrict__ dO = static_cast<const bf16*>(a.dout);
  const int G = a.G, B = a.B;

  const int kidx = kg * 32 + j;
  const bool key_ok = kidx < kt.n_keys;
  const bool wave_live = kg * 32 < kt.n_keys;
  const int64_t krow = (int64_t)(kt.k_tok + min(kidx, kt.n_keys - 1)) * a.hkv + kvh;
  const bool canvas_keys = kt.p0 < 0;
  const int kpos = canvas_keys ? 0 : kt.p0 + kidx;
  const int wpos_lo = kt.p0 + kg * 32;
  const int wpos_hi = kt.p0 + min(kg * 32 + 31, kt.n_keys - 1);

  const int qct = QC / G;                               // tokens per chunk
  const int nc0 = (kt.cq_len + qct - 1) / qct;
  const int cpc = (B + qct - 1) / qct;
  const int nchunks = nc0 + kt.cv_count * cpc;

  // async fetch of chunk c: Q and dO rows, LSE and delta per row, row limits
  auto issue = [&](int c, bf16* dQ_, bf16* dG_, float* dL_, float* dD_, int* dM_) {
    const ChunkGeom g = chunk_geom(kt, a.canvq, c, nc0, cpc, qct);
    const int nrows = g.ntok * G;                       // valid rows (<= qct*G <= 64)
    auto rowp = [&](const bf16* base) {
      return [=](int r) {
        const int t = r / G, gh = r - (r / G) * G;
        return base + ((int64_t)(g.tok0 + t) * a.hq + kvh * G + gh) * D;
      };
    };
    tile_fetch<D>(dQ_, rowp(Q), nrows, wave, lane);
    tile_fetch<D>(dG_, rowp(dO), nrows, wave, lane);
    if (wave < 2) {                                     // 64 rows x 4 bytes each
      const int r = min(lane, nrows - 1);
      const int t = r / G, gh = r - (r / G) * G;
      const int64_t qr = (int64_t)(g.tok0 + t) * a.hq + kvh * G + gh;
      const float* src = wave == 0 ? a.lse + qr : a.delta + qr;
      __builtin_amdgcn_global_load_lds(src, (lds_void*)(wave == 0 ? dL_ : dD_), 4, 0, 0);
    } else if (wave == 2) {
      const int r = lane, t = r / G;
      int lim = -1;                                     // padding rows see nothing
      if (r < nrows) lim = g.pos0 >= 0 ? ((g.pos0 + t) / B + 1) * B : g.lim;
      dM_[r] = lim;
    }
  };

  bf16x8 kf[NKS], vf[NKS];
#pragma unroll
  for (int kk = 0; kk < NKS; ++kk) {
    kf[kk] = *reinterpret_cast<const bf16x8*>(K + krow * D + kk * 16 + h * 8);
    vf[kk] = *reinterpret_cast<const bf16x8*>(V + krow * D + kk * 16 + h * 8);
  }
  f32x16 dkt[NDB], dvt[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) { dkt[db] = f32x16{}; dvt[db] = f32x16{}; }

  if (nchunks > 0) issue(0, sQ0, sG0, sL0, sD0, sM0);

  auto step = [&](int c, const bf16* cQ, const bf16* cG, const float* cL, const float* cD, const int* cM,
                  bf16* nQ, bf16* nG, float* nL, float* nD, int* nM) __attribute__((always_inline)) {
    wait_vmem();
    __syncthreads();                                    // chunk c landed; the other stage is free
    if (c + 1 < nchunks) issue(c + 1, nQ, nG, nL, nD, nM);
    const ChunkGeom g = chunk_geom(kt, a.canvq, c, nc0, cpc, qct);
    // visibility of this wave's 32 rows for its 32 keys
    const int r_lo = qh * 32, r_hi = min(qh * 32 + 31, g.ntok * G - 1);
    if (r_hi < r_lo || !wave_live) return;              // no valid row in this half, or no key
    int lim_lo, lim_hi;
    if (g.pos0 >= 0) {
      lim_lo = ((g.pos0 + r_lo / G) / B + 1) * B;
      lim_hi = ((g.pos0 + r_hi / G) / B + 1) * B;
    } else {
      lim_lo = lim_hi = g.lim;
    }
    const bool half_pad = r_hi < qh * 32 + 31;
    if (!canvas_keys && wpos_lo >= lim_hi) return;      // all of the wave's keys are invisible
    const bool need_mask = half_pad || (!canvas_keys && wpos_hi >= lim_lo);

    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk) {
      s = mfma32(cm_row8(cQ, lo, r_lo, kk), kf[kk], s);
      dp = mfma32(cm_row8(cG, lo, r_lo, kk), vf[kk], dp);
    }
    if (need_mask) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int4 mv = *reinterpret_cast<const int4*>(cM + r_lo + 8 * g4 + 4 * h);
        const int lims[4] = {mv.x, mv.y, mv.z, mv.w};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (kpos >= lims[e]) s[g4 * 4 + e] = -INFINITY;
      }
    }
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int r0 = r_lo + 8 * g4 + 4 * h;
      const f32x4 lv = *reinterpret_cast<const f32x4*>(cL + r0);
      const f32x4 dv = *reinterpret_cast<const f32x4*>(cD + r0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = g4 * 4 + e;
        const float p = fast_exp2(__builtin_fmaf(s[r], a.scale_log2, -lv[e] * kLog2e));
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
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        dvt[db] = mfma32(cm_tr8(cG, lo, r_lo + ks * 16, db * 32), pb[ks], dvt[db]);
        dkt[db] = mfma32(cm_tr8(cQ, lo, r_lo + ks * 16, db * 32), sb[ks], dkt[db]);
      }
  };
  for (int c = 0; c < nchunks; c += 2) {
    step(c, sQ0, sG0, sL0, sD0, sM0, sQ1, sG1, sL1, sD1, sM1);
    if (c + 1 < nchunks) step(c + 1, sQ1, sG1, sL1, sD1, sM1, sQ0, sG0, sL0, sD0, sM0);
  }

  // add the partial sums of the two query halves: waves 2, 3 hand theirs to 0, 1
  wait_vmem();
  __syncthreads();
  float* redk = reinterpret_cast<float*>(kg == 0 ? sQ0 : sQ1);   // NDB*16*64 floats = one tile
  float* redv = reinterpret_cast<float*>(kg == 0 ? sG0 : sG1);
  if (qh == 1) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        redk[(db * 16 + r) * 64 + lane] = dkt[db][r];
        redv[(db * 16 + r) * 64 + lane] = dvt[db][r];
      }
  }
  __syncthreads();
  if (qh == 0 && key_ok) {
    bf16* dkp = static_cast<bf16*>(a.dk) + krow * D;
    bf16* dvp = static_cast<bf16*>(a.dv) + krow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        float kx[4], vx[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = g4 * 4 + e;
          kx[e] = (dkt[db][r] + redk[(db * 16 + r) * 64 + lane]) * a.scale;
          vx[e] = dvt[db][r] + redv[(db * 16 + r) * 64 + lane];
        }
        const int d0 = db * 32 + g4 * 8 + h * 4;
        *reinterpret_cast<u32x2*>(dkp + d0) = u32x2{pack_bf16x2(kx[0], kx[1]), pack_bf16x2(kx[2], kx[3])};
        *reinterpret_cast<u32x2*>(dvp + d0) = u32x2{pack_bf16x2(vx[0], vx[1]), pack_bf16x2(vx[2], vx[3])};
      }
  }
}

// ---------------------------------------------------------------- dQ
// Workgroup: one query tile (up to 128 rows) and one kv head, over the same key
// tiles as the forward pass. Per wave 32 rows; scores transposed as in the
// forward pass. K and V tiles go straight into LDS (two stages); K^T for
// dQ^T = K^T dS^T is read with the LDS transpose read.
template <int D>
__global__ void __launch_bounds__(256, 2) dq_bf16_kernel(BwdArgs a) {
  constexpr int KT = kKTile;
  constexpr int NDB = D / 32, NKS = D / 16;
  constexpr int TE = KT * D;
  __shared__ __attribute__((aligned(1024))) bf16 sK0[TE];
  __shared__ __attribute__((aligned(1024))) bf16 sV0[TE];
  __shared__ __attribute__((aligned(1024))) bf16 sK1[TE];
  __shared__ __attribute__((aligned(1024))) bf16 sV1[TE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int j = lane & 31, h = lane >> 5;
  const CmLane lo(lane);
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
  const int L = row_limit(qt, t, a.B);
  const int n1 = (qt.lim_max + KT - 1) / KT;
  const int64_t kv_stride = (int64_t)a.hkv * D;

  auto issue = [&](int kt, bf16* dK, bf16* dV) {
    int base, nvalid;
    if (kt < n1) { base = qt.k_ctx + kt * KT; nvalid = min(KT, qt.lim_max - kt * KT); }
    else { const int k2 = kt - n1; base = qt.k_own + k2 * KT; nvalid = min(KT, qt.n_own - k2 * KT); }
    const bf16* kb = K + (int64_t)base * kv_stride + kvh * D;
    const bf16* vb = V + (int64_t)base * kv_stride + kvh * D;
    tile_fetch<D>(dK, [&](int r) { return kb + r * kv_stride; }, nvalid, wave, lane);
    tile_fetch<D>(dV, [&](int r) { return vb + r * kv_stride; }, nvalid, wave, lane);
  };
  if (kt_begin < kt_end) issue(kt_begin, sK0, sV0);

  bf16x8 qf[NKS], df[NKS];
#pragma unroll
  for (int kk = 0; kk < NKS; ++kk) {
    qf[kk] = *reinterpret_cast<const bf16x8*>(Q + qrow * D + kk * 16 + h * 8);
    df[kk] = *reinterpret_cast<const bf16x8*>(dO + qrow * D + kk * 16 + h * 8);
  }
  const float lse2 = a.lse[qrow] * kLog2e;
  const float dl = a.delta[qrow];

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  auto step = [&](int kt, const bf16* sK, const bf16* sV, bf16* nK, bf16* nV) __attribute__((always_inline)) {
    wait_vmem();
    __syncthreads();
    if (kt + 1 < kt_end) issue(kt + 1, nK, nV);
    const bool r1 = kt < n1;
    const int kpos0 = r1 ? kt * KT : (kt - n1) * KT;
    const int lim = r1 ? L : qt.n_own;
    const bool need_mask = kpos0 + KT > (r1 ? qt.lim_min : qt.n_own);

    f32x16 s[2], dp[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) { s[kb] = f32x16{}; dp[kb] = f32x16{}; }
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = mfma32(cm_row8(sK, lo, kb * 32, kk), qf[kk], s[kb]);
        dp[kb] = mfma32(cm_row8(sV, lo, kb * 32, kk), df[kk], dp[kb]);
      }
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kpos0 + kb * 32 + c_row(r, h) >= lim) s[kb][r] = -INFINITY;
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(__builtin_fmaf(s[kb][r], a.scale_log2, -lse2));
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
    for (int kq = 0; kq < 4; ++kq)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        acc[db] = mfma32(cm_tr8(sK, lo, kq * 16, db * 32), sb[kq], acc[db]);
  };
  for (int kt = kt_begin; kt < kt_end; kt += 2) {
    step(kt, sK0, sV0, sK1, sV1);
    if (kt + 1 < kt_end) step(kt + 1, sK1, sV1, sK0, sV0);
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
