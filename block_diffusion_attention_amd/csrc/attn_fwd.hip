// Forward staircase block-diffusion attention for gfx950 (bf16 in, fp32 accumulate).
//
// One workgroup (4 waves) handles one query tile of up to 128 rows (tokens x
// the query heads of one kv head, so the grouped heads share every K/V tile)
// over the key tiles of its visible ranges: the clean context below the tile's
// limit and, for a canvas, the canvas' own keys (ORL paper, section 3.2
// "Staircase attention kernel"; appendix D.2 paragraph on the kernel: ranges
// from per-document metadata, invisible tiles never visited, the predicate
// only inside boundary tiles).
//
// Per wave, 32 query rows. Scores are computed transposed, S^T = K Q^T, with
// the 32x32x16 MFMA so that each lane owns one query row: row maxima and sums
// need one cross-half exchange instead of a 32-lane reduction, and the
// probabilities feed the P V product straight from registers. K and V tiles go
// from global memory straight into swizzled row-major LDS tiles (two pipeline
// stages, no register staging); the V^T operand is read with the LDS transpose
// read.
#include "kcommon.h"
#include "kernels.h"

namespace bdattn {

namespace {

// LDS operand reads run this many products ahead of the MFMA that consumes them.
constexpr int kFwdAhead = 4;

// SPLIT: one part of a split key range (short query streams over long contexts):
// the item comes with its query tile in one record, the first two key tiles are
// requested together before anything else, and the result is a partial (bf16 O
// normalized by the part's own row sums, fp32 LSE) for the merge kernel.
template <int D, bool SPLIT, bool CHK>
__global__ void __launch_bounds__(256, 2) fwd_bf16_kernel(FwdArgs a) {
  constexpr int KT = kKTile;
  constexpr int NDB = D / 32;
  constexpr int NKS = D / 16;
  constexpr int TE = KT * D;                       // elements of one K or V tile
  // two pipeline stages of (K tile, V tile), filled asynchronously; separate
  // arrays so the compiler can tell a stage being read from the one being filled
  __shared__ __attribute__((aligned(1024))) bf16 sK0[TE];
  __shared__ __attribute__((aligned(1024))) bf16 sV0[TE];
  __shared__ __attribute__((aligned(1024))) bf16 sK1[TE];
  __shared__ __attribute__((aligned(1024))) bf16 sV1[TE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: copy targets in SGPRs
  const int j = lane & 31, h = lane >> 5;
  const SwLane<D> lo(lane);
  FwdWork w;
  if constexpr (SPLIT) {
    if (a.grid_parts > 0) grid_split_work(a.grid_qt, a.hkv, a.grid_parts, a.grid_tps, a.grid_tiles, blockIdx.x, &w);
    else if (!load_split_work(a.splits, blockIdx.x, &w)) return;   // empty launch slot
  } else {
    if (!load_fwd_work<CHK>(a.items, a.qtiles, blockIdx.x, &w, a.n_qtiles)) return;   // empty launch slot
  }
  if (reject_record<CHK>(!fwd_work_in_bounds(w, SPLIT, a.G, a.hkv, a.tq, a.tk, a.n_slots))) return;
  const int kvh = w.kvh, kt_begin = w.kt_begin, kt_end = w.kt_end;
  const QTile& qt = w.qt;
  const bf16* __restrict__ Q = static_cast<const bf16*>(a.q);
  const bf16* __restrict__ K = static_cast<const bf16*>(a.k);
  const bf16* __restrict__ V = static_cast<const bf16*>(a.v);

  const int G = a.G;
  const int row = wave * 32 + j;
  int t = row / G;
  const int gh = row - t * G;
  const bool row_ok = row < qt.n_tok * G;
  if (t >= qt.n_tok) t = qt.n_tok - 1;          // padding rows mirror the last token
  const int64_t qrow = (int64_t)(qt.q_tok + t) * a.hq + kvh * G + gh;

  const int L = row_limit(qt, t, a.grain);
  const int n1 = (qt.lim_max + KT - 1) / KT;
  const int64_t kv_stride = (int64_t)a.hkv * D;

  // K and V tiles: 64 key rows at stride Hkv*D, swizzled row-major in LDS
  const SwFetch<D> fetch([&](int r) { return r * (int)kv_stride; }, wave, lane);
  auto issue = [&](int kt, bf16* dK, bf16* dV) {
    int base, nvalid;
    if (kt < n1) { base = qt.k_ctx + kt * KT; nvalid = min(KT, qt.lim_max - kt * KT); }
    else { const int k2 = kt - n1; base = qt.k_own + k2 * KT; nvalid = min(KT, qt.n_own - k2 * KT); }
    const int64_t off0 = (int64_t)base * kv_stride + kvh * D;
    const int last = (nvalid - 1) * (int)kv_stride;
    fetch.issue(dK, K + off0, nvalid, last, wave);
    fetch.issue(dV, V + off0, nvalid, last, wave);
  };
  issue(kt_begin, sK0, sV0);
  // a split part is short: its second tile goes out at once too (one memory
  // round trip for the whole part instead of one per tile)
  if (SPLIT && kt_begin + 1 < kt_end) issue(kt_begin + 1, sK1, sV1);

  bf16x8 qf[NKS];
  {
    const bf16* qp = Q + qrow * D + h * 8;
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk) qf[kk] = *reinterpret_cast<const bf16x8*>(qp + kk * 16);
  }

  float m = -INFINITY, l = 0.f;
  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  auto step = [&](int kt, const bf16* sK, const bf16* sV, bf16* nK, bf16* nV) __attribute__((always_inline)) {
    wait_vmem();
    __syncthreads();                  // tile kt is in LDS; the other stage is free again
    const bool r1 = kt < n1;
    const int kpos0 = r1 ? kt * KT : (kt - n1) * KT;
    const int lim = r1 ? L : qt.n_own;
    const bool need_mask = kpos0 + KT > (r1 ? qt.lim_min : qt.n_own);

    // S^T = K Q^T : two 32-key blocks, each lane one query row. Fixed program of
    // 2 NKS products (the two blocks alternate) whose K operands are read from LDS
    // kFwdAhead products ahead; the reads of the first V^T operands are issued
    // under the last products, so they land during the softmax.
    constexpr int NSS = 2 * NKS, NPV = 4 * NDB;
    f32x16 s[2] = {f32x16{}, f32x16{}};
    bf16x8 opk[NSS], opv[NPV];
    auto fetch_k = [&](int i) { return sw_row8<D>(sK, lo, (i & 1) * 32, i >> 1); };
    auto fetch_v = [&](int i) { return sw_tr8<D>(sV, lo, (i / NDB) * 16, (i % NDB) * 32); };
    static_for<kFwdAhead>([&](auto ic) { opk[ic.value] = fetch_k(ic.value); });
    __builtin_amdgcn_sched_barrier(0);
    static_for<NSS>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      s[i & 1] = mfma32(opk[i], qf[i >> 1], s[i & 1]);
      if constexpr (i + kFwdAhead < NSS) opk[i + kFwdAhead] = fetch_k(i + kFwdAhead);
      else opv[i + kFwdAhead - NSS] = fetch_v(i + kFwdAhead - NSS);
      __builtin_amdgcn_sched_barrier(0);
    });
    // the next tile's copies go out after the S products, so their LDS writes do
    // not compete with this tile's K operand reads (the other stage is free since
    // the barrier; a split part's second tile is already on its way)
    // The softmax runs at raised wave priority: of the two waves that share a
    // SIMD, the one in its vector-ALU phase issues first, and the other one's
    // products fill the matrix unit meanwhile (measured 1-2 % faster than equal
    // priorities).
    __builtin_amdgcn_s_setprio(1);
    if (kt + 1 < kt_end && (!SPLIT || kt + 1 > kt_begin + 1)) issue(kt + 1, nK, nV);

    // masking only on tiles that cross a row limit or the end of a range
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (kpos0 + kb * 32 + c_row(r, h) >= lim) s[kb][r] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, swap_halves(mx)) * a.scale_log2;     // running max in the log2 domain
    const bool need = mx > m + kRescaleSlack;
    if (__any(need)) {
      const float mnew = need ? mx : m;
      const float alpha = need ? fast_exp2(m - mnew) : 1.f;
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
    }
    const float mref = (m == -INFINITY) ? 0.f : m;
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(__builtin_fmaf(s[kb][r], a.scale_log2, -mref));
        s[kb][r] = p;
        ls += p;
      }
    l += ls;

    bf16x8 pb[4];
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      float tmp[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) tmp[e] = s[kq >> 1][(kq & 1) * 8 + e];
      pb[kq] = pack8(tmp);
    }
    // O^T += V^T P^T, V^T read transposed out of the natural V tile; product
    // i = kq NDB + db, so consecutive products accumulate into different blocks
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    static_for<NPV>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      acc[i % NDB] = mfma32(opv[i], pb[i / NDB], acc[i % NDB]);
      if constexpr (i + kFwdAhead < NPV) opv[i + kFwdAhead] = fetch_v(i + kFwdAhead);
      __builtin_amdgcn_sched_barrier(0);
    });
  };
  for (int kt = kt_begin; kt < kt_end; kt += 2) {
    step(kt, sK0, sV0, sK1, sV1);
    if (kt + 1 < kt_end) step(kt + 1, sK1, sV1, sK0, sV0);
  }

  const float lt = l + swap_halves(l);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse = lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
  if constexpr (SPLIT) {
    store_partial<D>(a.part_o, a.part_lse, w.slot, wave, lane, acc, inv, lse);
  } else if (row_ok) {
    bf16* op = static_cast<bf16*>(a.o) + qrow * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        u32x2 v;
        v[0] = pack_bf16x2(acc[db][g4 * 4 + 0] * inv, acc[db][g4 * 4 + 1] * inv);
        v[1] = pack_bf16x2(acc[db][g4 * 4 + 2] * inv, acc[db][g4 * 4 + 3] * inv);
        *reinterpret_cast<u32x2*>(op + db * 32 + g4 * 8 + h * 4) = v;
      }
    if (h == 0) a.lse[qrow] = lse;
  }
}

// Merges the partial results of a split key range: for each row,
//   lse = log sum_i exp(lse_i),  O = sum_i exp(lse_i - lse) O_i
// over the parts i in key order. One wave per workgroup merges one block of the
// partials' register-order layout (32 rows x 16 columns; lane j + 32 h holds row
// 32 w + j, columns 32 db + 16 p + 4 h + {0..3} and + 8 + {0..3}): every load of
// a part is one contiguous 1 KiB. Parts are taken kMergeBatch at a time with all
// of a batch's loads issued before the first is used (one memory round trip per
// batch), folded into a running maximum.
constexpr int kMergeBatch = 32;

template <int D, bool CHK>
__global__ void __launch_bounds__(kMergeThreads) merge_kernel(MergeArgs a) {
  constexpr int NDB = D / 32;
  const int i = blockIdx.x;
  const int4 r0 = ld_rec4(a.items, 4 * i), r2 = ld_rec4(a.items, 4 * i + 2);
  const int kvh = r2.x, first = r2.y, count = r2.z, blk = r2.w;
  if (kvh < 0) return;                             // empty launch slot
  const int q_tok = r0.x, n_tok = r0.y;
  if (reject_record<CHK>(kvh >= a.hq / a.G || q_tok < 0 || n_tok < 1 || n_tok * a.G > kQRows ||
                    (int64_t)q_tok + n_tok > a.tq || first < 0 || count < 1 ||
                    (int64_t)first + count > a.n_slots || blk < 0 || blk >= 8 * NDB))
    return;
  const int w = blk / (2 * NDB), db = (blk / 2) % NDB, p = blk % 2;
  const int lane = threadIdx.x, j = lane & 31, h = lane >> 5;
  const int row = w * 32 + j;
  const float* pl = a.part_lse + (int64_t)first * kQRows + row;
  const bf16* po = static_cast<const bf16*>(a.part_o) + ((int64_t)(first * 4 + w) * NDB * 2 + blk % (2 * NDB)) * 512 +
                   8 * lane;
  constexpr int64_t kSlotElems = (int64_t)kQRows * D;
  float m = -INFINITY, wsum = 0.f;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int i0 = 0; i0 < count; i0 += kMergeBatch) {
    const int n = min(kMergeBatch, count - i0);
    float lv[kMergeBatch];
    u32x4 ov[kMergeBatch];
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      lv[k] = -INFINITY;
      ov[k] = u32x4{0u, 0u, 0u, 0u};
      if (k < n) {
        lv[k] = pl[(int64_t)(i0 + k) * kQRows];
        ov[k] = *reinterpret_cast<const u32x4*>(po + (int64_t)(i0 + k) * kSlotElems);
      }
    }
    float mx = m;
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) mx = fmaxf(mx, lv[k]);
    if (mx == -INFINITY) continue;                  // no part of this batch sees the row
    const float alpha = __expf(m - mx);             // 0 while m is -inf
    wsum *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
    m = mx;
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const float wk = __expf(lv[k] - m);           // 0 for the padding entries
      wsum += wk;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        acc[2 * u] += wk * __builtin_bit_cast(float, ov[k][u] << 16);
        acc[2 * u + 1] += wk * __builtin_bit_cast(float, ov[k][u] & 0xffff0000u);
      }
    }
  }
  if (row >= n_tok * a.G) return;                   // padding row of the query tile
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const int t = row / a.G, gh = row - t * a.G;
  const int64_t qrow = (int64_t)(q_tok + t) * a.hq + kvh * a.G + gh;
  bf16* op = static_cast<bf16*>(a.o) + qrow * D + db * 32 + p * 16 + h * 4;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    u32x2 v;
    v[0] = pack_bf16x2(acc[4 * half + 0] * inv, acc[4 * half + 1] * inv);
    v[1] = pack_bf16x2(acc[4 * half + 2] * inv, acc[4 * half + 3] * inv);
    *reinterpret_cast<u32x2*>(op + 8 * half) = v;
  }
  if (h == 0 && blk % (2 * NDB) == 0) a.lse[qrow] = wsum > 0.f ? m + __logf(wsum) : -INFINITY;
}

}  // namespace

namespace {
template <bool SPLIT>
hipError_t launch_fwd(const FwdArgs& a, int head_dim, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  const dim3 g(grid), b(256);
  if (head_dim == 128) {
    if (a.checks) hipLaunchKernelGGL((fwd_bf16_kernel<128, SPLIT, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((fwd_bf16_kernel<128, SPLIT, false>), g, b, 0, s, a);
  } else {
    if (a.checks) hipLaunchKernelGGL((fwd_bf16_kernel<64, SPLIT, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((fwd_bf16_kernel<64, SPLIT, false>), g, b, 0, s, a);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, int head_dim, int grid, hipStream_t s) {
  return launch_fwd<false>(a, head_dim, grid, s);
}

hipError_t launch_fwd_split_direct(const FwdArgs& a, int head_dim, int grid, hipStream_t s) {
  return launch_fwd<true>(a, head_dim, grid, s);
}

hipError_t launch_merge(const MergeArgs& a, int head_dim, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  const dim3 g(grid), b(kMergeThreads);
  if (head_dim == 128) {
    if (a.checks) hipLaunchKernelGGL((merge_kernel<128, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((merge_kernel<128, false>), g, b, 0, s, a);
  } else {
    if (a.checks) hipLaunchKernelGGL((merge_kernel<64, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((merge_kernel<64, false>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

BD_ATTN_DEVICE_ERRORS_QUERY(device_errors_fwd)

}  // namespace bdattn
