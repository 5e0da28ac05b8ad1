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

template <int D>
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
  const int idx = a.order ? ld_rec1(a.order, blockIdx.x) : (int)blockIdx.x;
  if (idx < 0) return;                              // empty slot of the split launch order
  const int4 itv = ld_rec4(a.items, idx);
  if (itv.x < 0) return;
  const int kvh = itv.y, kt_begin = itv.z, kt_end = itv.w;
  const QTile qt = load_qtile(a.qtiles, itv.x);
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
    // the barrier)
    if (kt + 1 < kt_end) issue(kt + 1, nK, nV);

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
  if (a.part_o) {
    float* po = a.part_o + ((int64_t)idx * kQRows + row) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[db][g4 * 4 + e] * inv;
        *reinterpret_cast<f32x4*>(po + db * 32 + g4 * 8 + h * 4) = v;
      }
    if (h == 0) a.part_lse[(int64_t)idx * kQRows + row] = lse;
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

// Merges the split partial results of one query tile: lse = log sum_i exp(lse_i),
// O = sum_i exp(lse_i - lse) O_i. Workgroup: kCombRows rows of one merge item,
// one thread per (row, 4 columns); blockIdx.x = item * (kQRows / rows) + group.
constexpr int kCombFast = 16;   // splits merged from registers in one round trip

template <int D, bool BF16>
__global__ void __launch_bounds__(256) combine_kernel(CombArgs a) {
  constexpr int C4 = D / 4;
  constexpr int RPW = 256 / C4;                    // rows per workgroup
  constexpr int GROUPS = kQRows / RPW;
  const int item = blockIdx.x / GROUPS;
  const int row = (blockIdx.x - item * GROUPS) * RPW + threadIdx.x / C4;
  const int c = threadIdx.x % C4;
  const int4 it = ld_rec4(a.items, item);
  const QTile qt = load_qtile(a.qtiles, it.x);
  const int kvh = it.y, first = it.z, count = it.w;
  if (row >= qt.n_tok * a.G) return;
  const float* pl = a.part_lse + (int64_t)first * kQRows + row;
  const float* po = a.part_o + ((int64_t)first * kQRows + row) * D + c * 4;
  float mx = -INFINITY;
  float wsum = 0.f;
  f32x4 accv = f32x4{};
  if (count <= kCombFast) {
    // every partial LSE and O of the row is requested before the first is used:
    // one memory round trip instead of one per loop iteration
    float lv[kCombFast];
    f32x4 ov[kCombFast];
#pragma unroll
    for (int i = 0; i < kCombFast; ++i) {
      lv[i] = -INFINITY;
      ov[i] = f32x4{};
      if (i < count) {
        lv[i] = pl[(int64_t)i * kQRows];
        ov[i] = *reinterpret_cast<const f32x4*>(po + (int64_t)i * kQRows * D);
      }
    }
#pragma unroll
    for (int i = 0; i < kCombFast; ++i) mx = fmaxf(mx, lv[i]);
    if (mx != -INFINITY) {
#pragma unroll
      for (int i = 0; i < kCombFast; ++i) {
        if (i < count) {
          const float w = __expf(lv[i] - mx);
          wsum += w;
          accv += w * ov[i];
        }
      }
    }
  } else {
    for (int i = 0; i < count; ++i) mx = fmaxf(mx, pl[(int64_t)i * kQRows]);
    if (mx != -INFINITY) {
#pragma unroll 4
      for (int i = 0; i < count; ++i) {
        const float w = __expf(pl[(int64_t)i * kQRows] - mx);
        wsum += w;
        accv += w * *reinterpret_cast<const f32x4*>(po + (int64_t)i * kQRows * D);
      }
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const int t = row / a.G, gh = row - t * a.G;
  const int64_t qrow = (int64_t)(qt.q_tok + t) * a.hq + kvh * a.G + gh;
  if (BF16) {
    u32x2 v;
    v[0] = pack_bf16x2(accv[0] * inv, accv[1] * inv);
    v[1] = pack_bf16x2(accv[2] * inv, accv[3] * inv);
    *reinterpret_cast<u32x2*>(static_cast<bf16*>(a.o) + qrow * D + c * 4) = v;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.o) + qrow * D + c * 4) = accv * inv;
  }
  if (c == 0) a.lse[qrow] = wsum > 0.f ? mx + __logf(wsum) : -INFINITY;
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, int head_dim, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  if (head_dim == 128) hipLaunchKernelGGL(fwd_bf16_kernel<128>, dim3(grid), dim3(256), 0, s, a);
  else hipLaunchKernelGGL(fwd_bf16_kernel<64>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombArgs& a, int head_dim, bool bf16_out, int items, hipStream_t s) {
  if (items <= 0) return hipSuccess;
  const int groups = kQRows / (256 / (head_dim / 4));
  const dim3 grid((unsigned)(items * groups));
  if (head_dim == 128) {
    if (bf16_out) hipLaunchKernelGGL((combine_kernel<128, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((combine_kernel<128, false>), grid, dim3(256), 0, s, a);
  } else {
    if (bf16_out) hipLaunchKernelGGL((combine_kernel<64, true>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((combine_kernel<64, false>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace bdattn
