// Backward staircase block-diffusion attention for gfx950: the dQ kernel (bf16 in,
// fp32 accumulate). It runs first in the backward pass and also writes the row
// terms delta = rowsum(dO * O) and LSE * log2(e) that the dK/dV kernel reads
// (attn_bwd.hip). Deterministic, no atomics (ORL paper, appendix D.2, the
// paragraph on the kernel: dQ follows the forward's traversal of each query
// tile's visible key ranges). dQ = scale ds K with dp = dO V^T and
// ds = p (dp - delta).
// Kept in a source file of its own so that it is compiled with the machine
// scheduler that suits it best (the build's per-file flags).
#include "kcommon.h"
#include "kernels.h"

namespace bdattn {

namespace {

// ---------------------------------------------------------------- dQ
// Workgroup: one query tile (up to 128 rows) and one kv head, over the same key
// tiles as the forward pass. It also computes and stores the row terms (delta,
// LSE * log2(e)) that the dK/dV kernel reads, so it runs first. Per wave 32 rows; scores transposed as in the
// forward pass. K and V tiles go straight into LDS (two stages); K^T for
// dQ^T = K^T dS^T is read with the LDS transpose read.
// dQ: LDS operand reads run this many products ahead of the MFMA that consumes them.
constexpr int kDqAhead = 3;   // (3 measured 0.6 % faster than 4 on the packed replay; 6 spills)

template <int D, bool CHK>
__global__ void __launch_bounds__(256, 2) dq_bf16_kernel(BwdArgs a) {
  constexpr int KT = kKTile;
  constexpr int NDB = D / 32, NKS = D / 16;
  constexpr int TE = KT * D;
  __shared__ __attribute__((aligned(1024))) bf16 sK0[TE];
  __shared__ __attribute__((aligned(1024))) bf16 sV0[TE];
  __shared__ __attribute__((aligned(1024))) bf16 sK1[TE];
  __shared__ __attribute__((aligned(1024))) bf16 sV1[TE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: copy targets in SGPRs
  const int j = lane & 31, h = lane >> 5;
  const SwLane<D> lo(lane);
  const int4 itv = ld_rec4(a.dq_items, blockIdx.x);
  if (itv.x < 0) return;
  if (reject_record<CHK>(itv.x >= a.n_qtiles)) return;
  const int kvh = itv.y, kt_begin = itv.z, kt_end = itv.w;
  const QTile qt = load_qtile(a.qtiles, itv.x);
  if (reject_record<CHK>(kvh < 0 || kvh >= a.hkv || !qtile_in_bounds(qt, a.G, a.tq, a.tk) ||
                    !key_range_in_bounds(qt, kt_begin, kt_end)))
    return;
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
  if (kt_begin < kt_end) issue(kt_begin, sK0, sV0);

  bf16x8 qf[NKS], df[NKS];
#pragma unroll
  for (int kk = 0; kk < NKS; ++kk) {
    qf[kk] = *reinterpret_cast<const bf16x8*>(Q + qrow * D + kk * 16 + h * 8);
    df[kk] = *reinterpret_cast<const bf16x8*>(dO + qrow * D + kk * 16 + h * 8);
  }
  // Row terms of the wave's rows: delta = rowsum(dO * O) (each lane half holds
  // half of the row) and LSE * log2(e). Stored for the dK/dV kernel, which runs
  // after this one; every row belongs to exactly one dQ item.
  float dl = 0.f;
  {
    const bf16* orow = static_cast<const bf16*>(a.o) + qrow * D + h * 8;
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk) {
      const u32x4 ov = *reinterpret_cast<const u32x4*>(orow + kk * 16);
      const u32x4 gv = __builtin_bit_cast(u32x4, df[kk]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        dl += __builtin_bit_cast(float, ov[w] << 16) * __builtin_bit_cast(float, gv[w] << 16);
        dl += __builtin_bit_cast(float, ov[w] & 0xffff0000u) * __builtin_bit_cast(float, gv[w] & 0xffff0000u);
      }
    }
    dl += swap_halves(dl);
  }
  const float lse2 = a.lse[qrow] * kLog2e;
  if (row_ok && h == 0) {
    a.delta[qrow] = dl;
    a.lse2[qrow] = lse2;
  }

  f32x16 acc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

  auto step = [&](int kt, const bf16* sK, const bf16* sV, bf16* nK, bf16* nV) __attribute__((always_inline)) {
    wait_vmem();
    __syncthreads();
    const bool r1 = kt < n1;
    const int kpos0 = r1 ? kt * KT : (kt - n1) * KT;
    const int lim = r1 ? L : qt.n_own;
    const bool need_mask = kpos0 + KT > (r1 ? qt.lim_min : qt.n_own);

    // S^T = K Q^T and dP^T = V dO^T as one fixed program of 4 NKS products
    // (product i: dimension step i / 4, key block i % 2, K/Q for even i % 4 / 2,
    // V/dO for odd), four accumulators in rotation, operands read from LDS
    // kDqAhead products ahead; the first K^T operands of dQ are requested under
    // the last products.
    constexpr int NSD = 4 * NKS, NQ = 4 * NDB;
    f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
    bf16x8 opa[NSD], opq[NQ];
    auto fetch_a = [&](int i) { return sw_row8<D>((i & 2) ? sV : sK, lo, (i & 1) * 32, i >> 2); };
    auto fetch_q = [&](int i) { return sw_tr8<D>(sK, lo, (i / NDB) * 16, (i % NDB) * 32); };
    static_for<kDqAhead>([&](auto ic) { opa[ic.value] = fetch_a(ic.value); });
    __builtin_amdgcn_sched_barrier(0);
    static_for<NSD>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i & 2) dp[i & 1] = mfma32(opa[i], df[i >> 2], dp[i & 1]);
      else s[i & 1] = mfma32(opa[i], qf[i >> 2], s[i & 1]);
      if constexpr (i + kDqAhead < NSD) opa[i + kDqAhead] = fetch_a(i + kDqAhead);
      else opq[i + kDqAhead - NSD] = fetch_q(i + kDqAhead - NSD);
      __builtin_amdgcn_sched_barrier(0);
    });
    // dS at raised wave priority, as the forward's softmax
    __builtin_amdgcn_s_setprio(1);
    // the next tile's copies go out after the S and dP products (as in the forward)
    if (kt + 1 < kt_end) issue(kt + 1, nK, nV);
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
    // dQ^T += K^T dS^T: product i = kq NDB + db, reads kDqAhead products ahead
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    static_for<NQ>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      acc[i % NDB] = mfma32(opq[i], sb[i / NDB], acc[i % NDB]);
      if constexpr (i + kDqAhead < NQ) opq[i + kDqAhead] = fetch_q(i + kDqAhead);
      __builtin_amdgcn_sched_barrier(0);
    });
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

hipError_t launch_dq_bf16(const BwdArgs& a, int head_dim, int grid, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  const dim3 g(grid), b(256);
  if (head_dim == 128) {
    if (a.checks) hipLaunchKernelGGL((dq_bf16_kernel<128, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((dq_bf16_kernel<128, false>), g, b, 0, s, a);
  } else {
    if (a.checks) hipLaunchKernelGGL((dq_bf16_kernel<64, true>), g, b, 0, s, a);
    else hipLaunchKernelGGL((dq_bf16_kernel<64, false>), g, b, 0, s, a);
  }
  return hipGetLastError();
}

BD_ATTN_DEVICE_ERRORS_QUERY(device_errors_dq)

}  // namespace bdattn
