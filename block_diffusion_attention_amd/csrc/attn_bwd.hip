// Backward staircase block-diffusion attention for gfx950 (bf16 in, fp32 accumulate):
// the dK/dV side (the dQ kernel, which runs first, is in attn_dq.hip).
//
// Deterministic kernels, no atomics (ORL paper, appendix D.2, the paragraph on
// the kernel). The gradients use exactly the forward's visibility: dQ walks each
// query tile's key ranges as the forward does, and dK/dV walks, for each key
// tile, the query ranges that can see it, computed by the planner. In launch
// order:
//   dq         : (attn_dq.hip) one workgroup per (query tile, kv head), looping
//                over the same key tiles as the forward pass; it also writes the
//                row terms delta = rowsum(dO * O) and LSE * log2(e) of its rows;
//   dkdv       : one workgroup per (key tile of up to 128 keys, kv head), looping
//                over the 64-row query chunks that can see the tile (or a
//                contiguous part of them);
//   dkdv_merge : sums the partial dK/dV of split key tiles in part order.
// (bwd_pre computes the row terms on their own for the fp32 path.)
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
  if (row < a.rows_q && c == 0) {
    a.delta[row] = s;
    a.lse2[row] = a.lse[row] * kLog2e;
  }
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
    const int4 ev = ld_rec4(cv, kt.cv_begin + e);
    g.tok0 = ev.x + sub * qct;
    g.ntok = min(qct, ev.y - sub * qct);
    g.pos0 = -1;
    g.lim = ev.w ? 0x7fffffff : ev.z;
  }
  return g;
}

// ---------------------------------------------------------------- dK / dV
// Workgroup: one key tile of up to 128 keys and one kv head. Wave w owns keys
// 32w .. 32w+31 (K and V rows in registers, dK^T and dV^T accumulators) and
// processes every 64-row query chunk that can see the tile, as two 32-row
// halves. Query chunks (rows = tokens x grouped heads, with their log2-domain
// LSE and delta) go from global memory straight into LDS (swizzled row-major
// tiles, a few cache lines per copy instruction), three stages deep, so two
// chunks are in flight while one is consumed. The transposed operands dO^T and
// Q^T of dV^T = dO^T P and dK^T = Q^T dS are read with the LDS transpose read
// from the same tiles.
//
// Per half: S = Q K^T and dP = dO V^T (16 MFMAs), then P = exp2(S*c - lse2),
// dS = P (dP - delta) on the vector ALUs, then dV^T += dO^T P and
// dK^T += Q^T dS (16 MFMAs), in one fixed slot program where the products of
// one half overlap the ALU work of the other. The masked instantiation applies
// per-score row limits; the planner picks the other one when every (chunk,
// 32-key group) pair is either wholly visible or skipped. An item may cover a
// contiguous part of a key tile's chunks only (a split tile); it then writes
// fp32 partial dK/dV for dkdv_merge instead of the bf16 result.
constexpr int kBwdStages = 3;

template <int D>
struct DkdvGeom {
  static constexpr int QC = 64;                 // query rows per chunk
  static constexpr int TE = QC * D;             // elements of one Q or dO chunk
  static constexpr int PW = D / 32;             // global_load_lds per wave per tile
};

// One 64-row query chunk for the 32 keys of a wave, as a fixed program of
// 4 * NS MFMA slots (NS = 2 * D / 16):
//   slots [0, NS)      S = Q K^T, dP = dO V^T for rows 0..31 (alternating)
//   slots [NS, 2NS)    the same for rows 32..63
//   slots [2NS, 3NS)   dV^T += dO^T P, dK^T += Q^T dS for rows 0..31
//   slots [3NS, 4NS)   dV^T, dK^T for rows 32..63
// with the vector work of rows 0..31 in slots [NS, 2NS) and that of rows 32..63
// in [2NS, 3NS), each shifted kPointShift slots later (below).
// Each slot issues one MFMA, the LDS reads of the operand kPrefetch slots ahead
// and its share of the per-score vector work; scheduling barriers between slots
// keep that order, so the vector ALU and the LDS run in the shadow of the MFMAs.
// MASKED applies the row limits to every score (padding rows have limit -1);
// plans whose chunks are all either seen whole by a wave's keys or skipped use
// the program without it (a separate kernel, chosen by the planner).
constexpr int kPrefetch = 4;
// Slots between a half's last S/dP product and the first use of its scores (at
// most 2 NDB: the packed P/dS of score elements 8..15 of a half are complete in
// slot kPointShift - 1 of its dV/dK phase, which first reads them in slot 2 NDB).
// 4 measured best for D = 128 (2 and 6 slower; 8 slower still).
constexpr int kPointShift = 4;

template <int D, bool MASKED>
__device__ __forceinline__ void dkdv_chunk(const bf16x8 (&kf)[D / 16], const bf16x8 (&vf)[D / 16],
                                           f32x16 (&dkt)[D / 32], f32x16 (&dvt)[D / 32], const bf16* cQ,
                                           const bf16* cG, const float* cL, const float* cD, const int* cM,
                                           const SwLane<D>& lo, int h, int kpos, float scale_log2) {
  constexpr int NKS = D / 16, NDB = D / 32;
  constexpr int NS = 2 * NKS;                 // MFMA slots per phase
  constexpr int NSLOT = 4 * NS;
  constexpr int EPS = 16 / NS;                // score elements per slot in the vector phases
  constexpr int SH = kPointShift;
  static_assert(SH <= 2 * NDB, "P/dS of a half must be packed before its dV/dK products read them");
  f32x16 sc[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
  bf16x8 pb[2][2], sb[2][2];
  f32x4 lv[2][4], dl[2][4];
  int4 lm[2][4];
  bf16x8 op[NSLOT];

  // operand of slot i (natural rows for S/dP, transposed for dV/dK)
  auto fetch = [&](int i) {
    if (i < 2 * NS) {
      const int half = i / NS, k = i % NS;
      return sw_row8<D>((k & 1) ? cG : cQ, lo, 32 * half, k >> 1);
    }
    const int half = (i - 2 * NS) / NS, k = (i - 2 * NS) % NS;
    const int ks = k / (2 * NDB), db = (k % (2 * NDB)) >> 1;
    return sw_tr8<D>((k & 1) ? cQ : cG, lo, 32 * half + 16 * ks, 32 * db);
  };
  auto rowterms = [&](int half) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int r0 = 32 * half + 8 * g4 + 4 * h;
      lv[half][g4] = *reinterpret_cast<const f32x4*>(cL + r0);
      dl[half][g4] = *reinterpret_cast<const f32x4*>(cD + r0);
      if (MASKED) lm[half][g4] = *reinterpret_cast<const int4*>(cM + r0);
    }
  };
  // P and dS of score element e of a half
  auto pointwise = [&](int half, int e) {
    const int g4 = e >> 2, q = e & 3;
    float x = sc[half][e];
    if (MASKED) {
      const int lim = q == 0 ? lm[half][g4].x : q == 1 ? lm[half][g4].y : q == 2 ? lm[half][g4].z : lm[half][g4].w;
      x = kpos < lim ? x : -INFINITY;
    }
    const float p = fast_exp2(__builtin_fmaf(x, scale_log2, -lv[half][g4][q]));
    sc[half][e] = p;
    dp[half][e] = p * (dp[half][e] - dl[half][g4][q]);
    if ((e & 7) == 7) {
      const int ks = e >> 3;
      float t0[8], t1[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) { t0[u] = sc[half][8 * ks + u]; t1[u] = dp[half][8 * ks + u]; }
      pb[half][ks] = pack8(t0);
      sb[half][ks] = pack8(t1);
    }
  };
  auto mma = [&](int i) {
    if (i < 2 * NS) {
      const int half = i / NS, k = i % NS;
      if (k & 1) dp[half] = mfma32(op[i], vf[k >> 1], dp[half]);
      else sc[half] = mfma32(op[i], kf[k >> 1], sc[half]);
    } else {
      const int half = (i - 2 * NS) / NS, k = (i - 2 * NS) % NS;
      const int ks = k / (2 * NDB), db = (k % (2 * NDB)) >> 1;
      if (k & 1) dkt[db] = mfma32(op[i], sb[half][ks], dkt[db]);
      else dvt[db] = mfma32(op[i], pb[half][ks], dvt[db]);
    }
  };

  static_for<kPrefetch>([&](auto ic) { op[ic.value] = fetch(ic.value); });
  __builtin_amdgcn_sched_barrier(0);
  static_for<NSLOT>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    mma(i);
    if constexpr (i + kPrefetch < NSLOT) op[i + kPrefetch] = fetch(i + kPrefetch);
    if constexpr (i == NS - 3) rowterms(0);
    if constexpr (i == 2 * NS - 3) rowterms(1);
    // a half's vector work starts SH slots after its last S/dP product,
    // so that product has finished by the time its scores are read
    constexpr int P0 = NS + SH, P1 = 2 * NS + SH;
    if constexpr (i >= P0 && i < P0 + NS) {
      static_for<EPS>([&](auto uc) { pointwise(0, (i - P0) * EPS + uc.value); });
    }
    if constexpr (i >= P1 && i < P1 + NS) {
      static_for<EPS>([&](auto uc) { pointwise(1, (i - P1) * EPS + uc.value); });
    }
    __builtin_amdgcn_sched_barrier(0);
  });
}

template <int D, bool MASKED, bool CHK>
__global__ void __launch_bounds__(256, 1) __attribute__((amdgpu_waves_per_eu(1, 1))) dkdv_bf16_kernel(BwdArgs a) {
  using Gm = DkdvGeom<D>;
  constexpr int NKS = D / 16, NDB = D / 32;
  constexpr int QC = Gm::QC, TE = Gm::TE, PW = Gm::PW;
  __shared__ __attribute__((aligned(1024))) bf16 sQ0[TE];
  __shared__ __attribute__((aligned(1024))) bf16 sG0[TE];
  __shared__ __attribute__((aligned(1024))) bf16 sQ1[TE];
  __shared__ __attribute__((aligned(1024))) bf16 sG1[TE];
  __shared__ __attribute__((aligned(1024))) bf16 sQ2[TE];
  __shared__ __attribute__((aligned(1024))) bf16 sG2[TE];
  // per-stage row terms: LSE*log2(e), delta, row limit (one array per stage so the
  // compiler can tell the stage being read from the ones being filled)
  __shared__ __attribute__((aligned(256))) float sL0[QC], sL1[QC], sL2[QC];
  __shared__ __attribute__((aligned(256))) float sD0[QC], sD1[QC], sD2[QC];
  __shared__ __attribute__((aligned(256))) int sM0[QC], sM1[QC], sM2[QC];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 31, h = lane >> 5;
  const SwLane<D> lo(lane);
  const int4 itv = ld_rec4(a.bwd_items, blockIdx.x);
  if (itv.x < 0) return;
  if (reject_record<CHK>(itv.x >= a.n_ktiles || itv.y < 0 || itv.y / a.hkv - 1 >= a.n_dkv_slots || itv.z < 0 ||
                    itv.z > itv.w))
    return;
  const int kvh = itv.y % a.hkv;
  const int slot = itv.y / a.hkv - 1;                   // partial slot of a split tile, or -1
  const KTile kt = load_ktile(a.ktiles, itv.x);
  if (CHK && reject_record<CHK>(!ktile_in_bounds(kt, a.tq, a.tk, a.n_canvq) ||
                                !ktile_canvq_in_bounds(kt, a.canvq, a.B, a.tq)))
    return;
  const bf16* __restrict__ Q = static_cast<const bf16*>(a.q);
  const bf16* __restrict__ K = static_cast<const bf16*>(a.k);
  const bf16* __restrict__ V = static_cast<const bf16*>(a.v);
  const bf16* __restrict__ dO = static_cast<const bf16*>(a.dout);
  const int G = a.G, B = a.B, Bc = a.grain;

  const int kidx = wave * 32 + j;
  const bool key_ok = kidx < kt.n_keys;
  const bool wave_live = wave * 32 < kt.n_keys;
  const int64_t krow = (int64_t)(kt.k_tok + min(kidx, kt.n_keys - 1)) * a.hkv + kvh;
  const bool canvas_keys = kt.p0 < 0;
  const int kpos = canvas_keys ? 0 : kt.p0 + kidx;
  const int wpos_lo = kt.p0 + wave * 32;
  // a clean query row at grid position x sees the wave's first key iff
  // wpos_lo < (x / Bc + 1) Bc, i.e. iff x >= (wpos_lo / Bc) Bc: one division per
  // kernel instead of two per chunk
  const int wpos_floor = canvas_keys ? 0 : (wpos_lo / Bc) * Bc;

  const int qct = QC / G;                               // tokens per chunk
  const int nc0 = (kt.cq_len + qct - 1) / qct;
  const int cpc = (B + qct - 1) / qct;
  const int nall = nc0 + kt.cv_count * cpc;             // chunks that may see the tile
  // this item's part of them, in visiting order: [c0, c0 + nchunks)
  const int c0 = min(itv.z, nall);
  const int nchunks = min(itv.w, nall) - c0;

  // Chunks are visited from the last one back: every key tile of a segment ends
  // its query range at the same place, so tiles running at the same time start on
  // the same chunks and share them in L2.
  // Row r of a chunk is the (token r / G, head r % G) pair, at element offset
  // ((r / G) * Hq + r % G) * D from the chunk's first row; the per-lane offsets
  // are the same for every chunk and are computed once.
  auto row_elems = [&](int r) { return ((r / G) * a.hq + (r - (r / G) * G)) * D; };
  const SwFetch<D> fetch(row_elems, wave, lane);
  const int lane_tok = lane / G;                        // token of chunk row `lane`
  const int lane_row = lane_tok * a.hq + (lane - lane_tok * G);  // its LSE/delta row

  // async fetch of chunk c: Q and dO rows (swizzled row-major tiles), log2-domain
  // LSE and delta per row, and (masked kernel) row limits. Rows past the chunk's
  // end read its last row. Waves 0 and 1 issue one load more than 2 and 3.
  auto issue = [&](int c, bf16* dQ_, bf16* dG_, float* dL_, float* dD_, int* dM_) {
    const ChunkGeom g = chunk_geom(kt, a.canvq, nall - 1 - (c0 + c), nc0, cpc, qct);
    const int nrows = g.ntok * G;                       // valid rows (<= qct*G <= 64)
    const int64_t row0 = (int64_t)g.tok0 * a.hq + kvh * G;
    const int last = (g.ntok - 1) * a.hq + (G - 1);     // row nrows - 1 (nrows = ntok G); uniform
    fetch.template issue<false>(dQ_, Q + row0 * D, nrows, last * D, wave);
    fetch.template issue<false>(dG_, dO + row0 * D, nrows, last * D, wave);
    if (wave < 2) {                                     // 64 rows x 4 bytes each
      const int64_t qr = row0 + (lane < nrows ? lane_row : last);
      const float* src = wave == 0 ? a.lse2 + qr : a.delta + qr;
      dma_b32(src, wave == 0 ? dL_ : dD_);
    } else if (MASKED && wave == 2) {
      int lim = -1;                                     // padding rows see nothing
      if (lane < nrows) lim = g.pos0 >= 0 ? ((g.pos0 + lane_tok) / Bc + 1) * Bc : g.lim;
      dM_[lane] = lim;
    }
  };

  bf16x8 kf[NKS], vf[NKS];
#pragma unroll
  for (int kk = 0; kk < NKS; ++kk) {
    kf[kk] = *reinterpret_cast<const bf16x8*>(K + krow * D + kk * 16 + h * 8);
    vf[kk] = *reinterpret_cast<const bf16x8*>(V + krow * D + kk * 16 + h * 8);
  }
  // the K/V rows must be in registers before the pipelined loads start, so that no
  // later wait for them has to drain the chunk loads in flight
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  // K/V fragments live in accumulation registers (MFMA reads its A/B operands from
  // either file), leaving the vector registers to the scores the ALU works on
#pragma unroll
  for (int kk = 0; kk < NKS; ++kk) asm volatile("" : "+a"(kf[kk]), "+a"(vf[kk]));
  f32x16 dkt[NDB], dvt[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) { dkt[db] = f32x16{}; dvt[db] = f32x16{}; }

  if (nchunks > 0) issue(0, sQ0, sG0, sL0, sD0, sM0);
  if (nchunks > 1) issue(1, sQ1, sG1, sL1, sD1, sM1);

  auto step = [&](int c, const bf16* cQ, const bf16* cG, const float* cL, const float* cD, const int* cM,
                  bf16* nQ, bf16* nG, float* nL, float* nD, int* nM) __attribute__((always_inline)) {
    // chunk c has landed once at most the loads of chunk c+1 are outstanding
    if (c + 1 < nchunks) {
      if (wave < 2) __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * PW + 1));
      else __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * PW));
    } else {
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    }
    lds_barrier();                                      // chunk c visible; stage of c-1 free
    const ChunkGeom g = chunk_geom(kt, a.canvq, nall - 1 - (c0 + c), nc0, cpc, qct);
    const int nrows = g.ntok * G;
    // row limits of the first and the last valid row (clean limits grow with the row)
    // skip when no valid row sees any of the wave's keys: for a clean chunk its last
    // row (grid position pos0 + ntok - 1) has the largest limit
    const bool unseen = g.pos0 >= 0 ? g.pos0 + g.ntok - 1 < wpos_floor : wpos_lo >= g.lim;
    if (wave_live && (canvas_keys || !unseen))
      dkdv_chunk<D, MASKED>(kf, vf, dkt, dvt, cQ, cG, cL, cD, cM, lo, h, kpos, a.scale_log2);
    // the copies of chunk c+2 (into the stage of c-1, free since the barrier) go out
    // after this chunk's products
    if (c + 2 < nchunks) issue(c + 2, nQ, nG, nL, nD, nM);
  };
  for (int c = 0; c < nchunks; c += kBwdStages) {
    step(c, sQ0, sG0, sL0, sD0, sM0, sQ2, sG2, sL2, sD2, sM2);
    if (c + 1 < nchunks) step(c + 1, sQ1, sG1, sL1, sD1, sM1, sQ0, sG0, sL0, sD0, sM0);
    if (c + 2 < nchunks) step(c + 2, sQ2, sG2, sL2, sD2, sM2, sQ1, sG1, sL1, sD1, sM1);
  }

  if (key_ok && slot >= 0) {                            // part of a split tile: fp32 partials
    float* pk = a.dkv_part + ((int64_t)slot * 2 * kKBlock + kidx) * D;
    float* pv = pk + (int64_t)kKBlock * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 kx, vx;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kx[e] = dkt[db][g4 * 4 + e];
          vx[e] = dvt[db][g4 * 4 + e];
        }
        const int d0 = db * 32 + g4 * 8 + h * 4;
        *reinterpret_cast<f32x4*>(pk + d0) = kx;
        *reinterpret_cast<f32x4*>(pv + d0) = vx;
      }
  } else if (key_ok) {
    bf16* dkp = static_cast<bf16*>(a.dk) + krow * D;
    bf16* dvp = static_cast<bf16*>(a.dv) + krow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        float kx[4], vx[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kx[e] = dkt[db][g4 * 4 + e] * a.scale;
          vx[e] = dvt[db][g4 * 4 + e];
        }
        const int d0 = db * 32 + g4 * 8 + h * 4;
        *reinterpret_cast<u32x2*>(dkp + d0) = u32x2{pack_bf16x2(kx[0], kx[1]), pack_bf16x2(kx[2], kx[3])};
        *reinterpret_cast<u32x2*>(dvp + d0) = u32x2{pack_bf16x2(vx[0], vx[1]), pack_bf16x2(vx[2], vx[3])};
      }
  }
}

// ---------------------------------------------------------------- dK/dV merge
// Sums the fp32 partial dK/dV of a split key tile in slot order, applies the
// softmax scale to dK and writes both in bf16. Workgroup: 256 threads, each four
// consecutive dimensions of one key; (kKBlock * D / 4) / 256 workgroups per tile.
template <int D, bool CHK>
__global__ void __launch_bounds__(256) dkdv_merge_kernel(BwdArgs a) {
  constexpr int Q4 = D / 4;
  constexpr int WG_PER = kKBlock * Q4 / 256;
  const int4 mv = ld_rec4(a.bmerge, blockIdx.x / WG_PER);
  if (reject_record<CHK>(mv.x < 0 || mv.x >= a.n_ktiles || mv.y < 0 || mv.y >= a.hkv || mv.z < 0 || mv.w < 1 ||
                    (int64_t)mv.z + mv.w > a.n_dkv_slots))
    return;
  const KTile kt = load_ktile(a.ktiles, mv.x);
  if (reject_record<CHK>(!ktile_in_bounds(kt, a.tq, a.tk, a.n_canvq))) return;
  const int idx = (blockIdx.x % WG_PER) * 256 + threadIdx.x;
  const int key = idx / Q4, d0 = (idx % Q4) * 4;
  if (key >= kt.n_keys) return;
  f32x4 sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < mv.w; ++i) {
    const float* pk = a.dkv_part + ((int64_t)(mv.z + i) * 2 * kKBlock + key) * D + d0;
    sk += *reinterpret_cast<const f32x4*>(pk);
    sv += *reinterpret_cast<const f32x4*>(pk + (int64_t)kKBlock * D);
  }
  const int64_t krow = (int64_t)(kt.k_tok + key) * a.hkv + mv.y;
  bf16* dkp = static_cast<bf16*>(a.dk) + krow * D + d0;
  bf16* dvp = static_cast<bf16*>(a.dv) + krow * D + d0;
  *reinterpret_cast<u32x2*>(dkp) = u32x2{pack_bf16x2(sk[0] * a.scale, sk[1] * a.scale),
                                         pack_bf16x2(sk[2] * a.scale, sk[3] * a.scale)};
  *reinterpret_cast<u32x2*>(dvp) = u32x2{pack_bf16x2(sv[0], sv[1]), pack_bf16x2(sv[2], sv[3])};
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

namespace {
template <int D, bool CHK>
void launch_dkdv_d(const BwdArgs& a, bool masked, int grid, hipStream_t s) {
  if (masked) hipLaunchKernelGGL((dkdv_bf16_kernel<D, true, CHK>), dim3(grid), dim3(256), 0, s, a);
  else hipLaunchKernelGGL((dkdv_bf16_kernel<D, false, CHK>), dim3(grid), dim3(256), 0, s, a);
}
}  // namespace

hipError_t launch_dkdv_bf16(const BwdArgs& a, int head_dim, bool masked, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (head_dim == 128) {
    if (a.checks) launch_dkdv_d<128, true>(a, masked, grid, s);
    else launch_dkdv_d<128, false>(a, masked, grid, s);
  } else {
    if (a.checks) launch_dkdv_d<64, true>(a, masked, grid, s);
    else launch_dkdv_d<64, false>(a, masked, grid, s);
  }
  return hipGetLastError();
}

hipError_t launch_dkdv_merge(const BwdArgs& a, int head_dim, int n_merge, hipStream_t s) {
  if (n_merge <= 0) return hipSuccess;
  const dim3 b(256);
  if (head_dim == 128) {
    const dim3 g(n_merge * (kKBlock * 32 / 256));
    if (a.checks) hipLaunchKernelGGL((dkdv_merge_kernel<128, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((dkdv_merge_kernel<128, false>), g, b, 0, s, a);
  } else {
    const dim3 g(n_merge * (kKBlock * 16 / 256));
    if (a.checks) hipLaunchKernelGGL((dkdv_merge_kernel<64, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((dkdv_merge_kernel<64, false>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

BD_ATTN_DEVICE_ERRORS_QUERY(device_errors_bwd)

}  // namespace bdattn
