// Forward staircase block-diffusion attention for gfx950, reading V through a
// transposed copy (bf16 in, fp32 accumulate).
//
// Same work lists and visibility as the direct forward kernel (ORL paper,
// section 3.2 "Staircase attention kernel"; appendix D.2 paragraph on the
// kernel: key ranges from per-document metadata, invisible tiles never visited,
// the predicate only inside boundary tiles), same per-tile loop. Two things differ:
//
//  * V^T. O^T = V^T P^T takes V^T as its A operand, i.e. 8 consecutive keys per
//    lane at one head dimension. A pre-pass writes VT[kv head][d][key] once per
//    call, so that operand is one 16-byte LDS read instead of two transposing
//    reads; the probabilities come out of the score accumulator in the MFMA
//    result's row order and two cross-half lane swaps per operand put them in
//    key order.
//
//  * Coalesced tiles. K and VT tiles are fetched with whole rows per
//    instruction into padded row-major LDS tiles (odd row stride in 16-byte
//    units), so operand reads stay free of bank conflicts.
//
// Requires every key range to start at a multiple of 8 keys (block size a
// multiple of 8), so VT rows are read in aligned 16-byte pieces.
#include "kcommon.h"
#include "kernels.h"

namespace bdattn {

namespace {

// VT[g][d][key] = V[key][g][d] for key < tk, 0 for tk <= key < tk_pad.
// Workgroup: 64 keys x one kv head.
template <int D>
__global__ void __launch_bounds__(256) transpose_v_kernel(const bf16* __restrict__ v, bf16* __restrict__ vt, int tk,
                                                          int tk_pad, int hkv) {
  constexpr int KB = 64;
  constexpr int CPR = D / 8;                       // 16-byte chunks per key row
  __shared__ bf16 tile[KB][D + 8];
  const int k0 = blockIdx.x * KB, g = blockIdx.y;
  for (int u = threadIdx.x; u < KB * CPR; u += 256) {
    const int r = u / CPR, c = u - r * CPR;
    u32x4 val = u32x4{0u, 0u, 0u, 0u};
    if (k0 + r < tk) val = *reinterpret_cast<const u32x4*>(v + ((int64_t)(k0 + r) * hkv + g) * D + c * 8);
    *reinterpret_cast<u32x4*>(&tile[r][c * 8]) = val;
  }
  __syncthreads();
  for (int u = threadIdx.x; u < D * (KB / 8); u += 256) {
    const int d = u / (KB / 8), c = u - d * (KB / 8);
    bf16x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = tile[c * 8 + e][d];
    *reinterpret_cast<bf16x8*>(vt + ((int64_t)g * D + d) * tk_pad + k0 + c * 8) = out;
  }
}

// Puts the P^T operand of 16 keys, packed from registers 8q..8q+7 of a score
// accumulator (keys {0-3, 8-11} + 4h of the group in lane half h), in key order
// (keys 0-7 in half 0, 8-15 in half 1) by swapping two dwords across the halves.
__device__ __forceinline__ bf16x8 ptr_operand(const float* p) {
  uint32_t u0 = pack_bf16x2(p[0], p[1]), u1 = pack_bf16x2(p[2], p[3]);
  uint32_t u2 = pack_bf16x2(p[4], p[5]), u3 = pack_bf16x2(p[6], p[7]);
  const auto s02 = __builtin_amdgcn_permlane32_swap(u0, u2, false, false);
  const auto s13 = __builtin_amdgcn_permlane32_swap(u1, u3, false, false);
  return __builtin_bit_cast(bf16x8, u32x4{(uint32_t)s02[0], (uint32_t)s13[0], (uint32_t)s02[1], (uint32_t)s13[1]});
}

// SPLIT: one part of a split key range, item from the split list (with its query
// tile), result written as a partial for the merge kernel.
template <int D, bool SPLIT, bool CHK>
__global__ void __launch_bounds__(256, 2) fwd_vt_kernel(FwdArgs a) {
  constexpr int KT = kKTile;
  constexpr int NDB = D / 32;
  constexpr int NKS = D / 16;
  using KTl = PadTile<KT, D / 8>;                  // K tile: 64 keys x D
  using VTl = PadTile<D, KT / 8>;                  // VT tile: D dimensions x 64 keys
  __shared__ __attribute__((aligned(1024))) bf16 sK0[KTl::kElems];
  __shared__ __attribute__((aligned(1024))) bf16 sK1[KTl::kElems];
  __shared__ __attribute__((aligned(1024))) bf16 sV0[VTl::kElems];
  __shared__ __attribute__((aligned(1024))) bf16 sV1[VTl::kElems];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 31, h = lane >> 5;
  const int kbase = pad_base<D / 8>(lane);        // K operand rows
  const int vbase = pad_base<KT / 8>(lane);       // VT operand dimensions
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
  const bf16* __restrict__ VT = static_cast<const bf16*>(a.vt) + (int64_t)kvh * D * a.tk_pad;

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
  const float cl2 = a.scale_log2;

  auto issue = [&](int kt, bf16* dK, bf16* dV) {
    int base, nvalid;
    if (kt < n1) { base = qt.k_ctx + kt * KT; nvalid = min(KT, qt.lim_max - kt * KT); }
    else { const int k2 = kt - n1; base = qt.k_own + k2 * KT; nvalid = min(KT, qt.n_own - k2 * KT); }
    pad_tile_fetch<KT, D / 8>(dK, K + (int64_t)base * kv_stride + kvh * D, (int)kv_stride, nvalid, wave, lane);
    // keys past the range read valid memory (the next keys, or the zero padding)
    pad_tile_fetch<D, KT / 8>(dV, VT + base, a.tk_pad, D, wave, lane);
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
    lds_barrier();                    // tile kt is in LDS; the other stage is free again
    if (kt + 1 < kt_end) issue(kt + 1, nK, nV);
    const bool r1 = kt < n1;
    const int kpos0 = r1 ? kt * KT : (kt - n1) * KT;
    const int lim = r1 ? L : qt.n_own;
    const bool need_mask = kpos0 + KT > (r1 ? qt.lim_min : qt.n_own);

    // S^T = K Q^T : two 32-key blocks, each lane one query row
    f32x16 s[2];
    s[0] = f32x16{}; s[1] = f32x16{};
    static_for<NKS>([&](auto kc) {
      static_for<2>([&](auto bc) {
        s[bc.value] = mfma32(pad_row8<D / 8>(sK, kbase, bc.value * 32, kc.value), qf[kc.value], s[bc.value]);
      });
    });
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
    mx = fmaxf(mx, swap_halves(mx)) * cl2;           // running max in the log2 domain
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
        const float p = fast_exp2(__builtin_fmaf(s[kb][r], cl2, -mref));
        s[kb][r] = p;
        ls += p;
      }
    l += ls;
    // P^T operands of the four 16-key groups, in key order
    bf16x8 pb[4];
    static_for<4>([&](auto qc) {
      float t8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) t8[e] = s[qc.value >> 1][(qc.value & 1) * 8 + e];
      pb[qc.value] = ptr_operand(t8);
    });
    // O^T += V^T P^T, V^T straight out of the transposed copy
    static_for<NDB>([&](auto dc) {
      static_for<4>([&](auto qc) {
        acc[dc.value] = mfma32(pad_row8<KT / 8>(sV, vbase, dc.value * 32, qc.value), pb[qc.value], acc[dc.value]);
      });
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

}  // namespace

hipError_t launch_transpose_v(const void* v, void* vt, int tk, int tk_pad, int hkv, int head_dim, hipStream_t s) {
  const dim3 grid((unsigned)(tk_pad / 64), (unsigned)hkv);
  if (head_dim == 128)
    hipLaunchKernelGGL(transpose_v_kernel<128>, grid, dim3(256), 0, s, static_cast<const bf16*>(v),
                       static_cast<bf16*>(vt), tk, tk_pad, hkv);
  else
    hipLaunchKernelGGL(transpose_v_kernel<64>, grid, dim3(256), 0, s, static_cast<const bf16*>(v),
                       static_cast<bf16*>(vt), tk, tk_pad, hkv);
  return hipGetLastError();
}

namespace {
template <bool SPLIT>
hipError_t launch_vt(const FwdArgs& a, int head_dim, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  const dim3 g(grid), b(256);
  if (head_dim == 128) {
    if (a.checks) hipLaunchKernelGGL((fwd_vt_kernel<128, SPLIT, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((fwd_vt_kernel<128, SPLIT, false>), g, b, 0, s, a);
  } else {
    if (a.checks) hipLaunchKernelGGL((fwd_vt_kernel<64, SPLIT, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((fwd_vt_kernel<64, SPLIT, false>), g, b, 0, s, a);
  }
  return hipGetLastError();
}
}  // namespace

hipError_t launch_fwd_vt(const FwdArgs& a, int head_dim, int grid, hipStream_t s) {
  return launch_vt<false>(a, head_dim, grid, s);
}

hipError_t launch_fwd_split_vt(const FwdArgs& a, int head_dim, int grid, hipStream_t s) {
  return launch_vt<true>(a, head_dim, grid, s);
}

BD_ATTN_DEVICE_ERRORS_QUERY(device_errors_fwd_vt)

}  // namespace bdattn
