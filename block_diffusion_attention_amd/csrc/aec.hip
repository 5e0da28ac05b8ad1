// Normalized entropy of vocabulary distributions and the adjacent-entropy-
// contraction (AEC) loss, for gfx950.
//
// ORL paper, paragraph "Learning how fast to refine": the normalized token
// entropy -sum_v p_v log p_v / log|V| of a softmax over the vocabulary, its mean
// over the unresolved positions of a state, and the hinge
// max(0, H_next - (1 - rho) H_source)^2 of an adjacent pair of states; the
// appendix paragraph on valid AEC pairs gives the pair weights w, fixed before
// the gate g, and the normalizer D = sum w g (loss 0 when D = 0). The natural-log
// normalizer of every row is written as well (appendix F.1 "Kernels": a later
// softmax over the same logits reuses it).
//
// The logits are read once. Each workgroup streams a contiguous part of one
// row with 16-byte loads, eight in flight per thread, and keeps per thread a
// running (max m, S = sum 2^d, U = sum 2^d d) over d = x log2(e) - m, so that
// log2 Z = m + log2 S and the entropy in bits is log2 S - U / S. Partial
// triples of several workgroups (short batches split each row; a single
// workgroup merges them before the state means) merge exactly:
// moving a triple to a larger max M scales S by 2^(m-M) and U to
// 2^(m-M) (U + (m-M) S). Every sum runs in a fixed order: no atomics.
#include "aec.h"

namespace bdattn {

namespace {

constexpr float kL2E = 1.4426950408889634f;
constexpr float kLN2 = 0.6931471805599453f;
constexpr int kThreads = 256;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct Acc {
  float m, s, u;
};

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void merge(Acc& a, const Acc& b) {
  if (b.s == 0.f) return;
  if (a.s == 0.f) { a = b; return; }
  const float m = fmaxf(a.m, b.m);
  const float da = a.m - m, db = b.m - m;
  const float fa = ex2(da), fb = ex2(db);
  a.u = fa * fmaf(da, a.s, a.u) + fb * fmaf(db, b.s, b.u);
  a.s = fa * a.s + fb * b.s;
  a.m = m;
}

// Adds K logits (natural units); the running max only moves up.
template <int K>
__device__ __forceinline__ void add(Acc& a, const float (&x)[K]) {
  float mx = x[0];
#pragma unroll
  for (int j = 1; j < K; ++j) mx = fmaxf(mx, x[j]);
  const float mv = mx * kL2E;
  if (mv > a.m) {
    if (a.s > 0.f) {
      const float d = a.m - mv, f = ex2(d);
      a.u = f * fmaf(d, a.s, a.u);
      a.s *= f;
    }
    a.m = mv;
  }
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const float d = fmaf(x[j], kL2E, -a.m);
    const float e = ex2(d);
    a.s += e;
    a.u = fmaf(e, d, a.u);
  }
}

template <bool BF16>
__device__ __forceinline__ void unpack(const u32x4& w, float (&x)[BF16 ? 8 : 4]) {
  if constexpr (BF16) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      x[2 * k] = __builtin_bit_cast(float, w[k] << 16);
      x[2 * k + 1] = __builtin_bit_cast(float, w[k] & 0xffff0000u);
    }
  } else {
    // whole-vector reinterpretation: a bit cast of one element of a vector
    // value is compiled here as a cast of element 0
    const f32x4 f = __builtin_bit_cast(f32x4, w);
#pragma unroll
    for (int k = 0; k < 4; ++k) x[k] = f[k];
  }
}

__device__ __forceinline__ float finish(const Acc& a, int vocab, float* lse, float* hbar) {
  const float l2s = log2f(a.s);
  *lse = (a.m + l2s) * kLN2;
  const float h = (l2s - a.u / a.s) / log2f((float)vocab);
  *hbar = h;
  return h;
}

template <bool BF16>
__global__ void __launch_bounds__(kThreads) aec_entropy_kernel(AecArgs a) {
  constexpr int EPV = BF16 ? 8 : 4;                   // elements per 16-byte load
  const int row = blockIdx.x / a.nsplit, split = blockIdx.x - row * a.nsplit;
  const int64_t c0 = (int64_t)split * a.chunk;
  const int64_t c1 = min((int64_t)a.vocab, c0 + a.chunk);
  const int64_t nvec = (c1 - c0) / EPV;               // whole vectors; c0 is a multiple of EPV
  const int tail = (int)((c1 - c0) - nvec * EPV);     // only the last split has one
  const char* rowp = static_cast<const char*>(a.logits) + (row * a.row_stride + c0) * (BF16 ? 2 : 4);
  const u32x4* vp = reinterpret_cast<const u32x4*>(rowp);

  Acc acc{-INFINITY, 0.f, 0.f};
  int64_t i = threadIdx.x;
  for (; i + 7 * kThreads < nvec; i += 8 * kThreads) {
    u32x4 w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = __builtin_nontemporal_load(vp + i + k * kThreads);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float x[EPV];
      unpack<BF16>(w[k], x);
      add<EPV>(acc, x);
    }
  }
  for (; i < nvec; i += kThreads) {
    float x[EPV];
    unpack<BF16>(__builtin_nontemporal_load(vp + i), x);
    add<EPV>(acc, x);
  }
  if (threadIdx.x < tail) {
    float x[1];
    if constexpr (BF16) {
      const uint16_t b = reinterpret_cast<const uint16_t*>(rowp)[nvec * EPV + threadIdx.x];
      x[0] = __builtin_bit_cast(float, (uint32_t)b << 16);
    } else {
      x[0] = reinterpret_cast<const float*>(rowp)[nvec * EPV + threadIdx.x];
    }
    add<1>(acc, x);
  }

  // workgroup reduction in a fixed order: lanes, then the four waves
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    Acc o{__shfl_xor(acc.m, off), __shfl_xor(acc.s, off), __shfl_xor(acc.u, off)};
    merge(acc, o);
  }
  __shared__ float red[3][kThreads / 64];
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) { red[0][wave] = acc.m; red[1][wave] = acc.s; red[2][wave] = acc.u; }
  __syncthreads();
  if (threadIdx.x == 0) {
    Acc t{red[0][0], red[1][0], red[2][0]};
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) merge(t, Acc{red[0][w], red[1][w], red[2][w]});
    if (a.nsplit == 1) {
      finish(t, a.vocab, a.lse + row, a.hbar + row);
    } else {
      float* p = a.part + (int64_t)blockIdx.x * 3;
      p[0] = t.m; p[1] = t.s; p[2] = t.u;
    }
  }
}

// Mean normalized entropy over the unresolved rows [lo, hi) of one state, by one
// wave: lanes take rows lo + lane, lo + lane + 64, ...; the sums meet in a fixed
// butterfly. NaN when the state has no unresolved row.
__device__ float wave_state_mean(const AecArgs& a, int s, int lane) {
  const int lo = min(max(a.state_rows[s], 0), a.n_rows);
  const int hi = min(max(a.state_rows[s + 1], lo), a.n_rows);
  float sum = 0.f, cnt = 0.f;
  for (int i = lo + lane; i < hi; i += 64)
    if (a.unresolved[i]) { sum += a.hbar[i]; cnt += 1.f; }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    sum += __shfl_xor(sum, off);
    cnt += __shfl_xor(cnt, off);
  }
  return cnt > 0.f ? sum / cnt : __builtin_nanf("");
}

// One workgroup, three phases separated by barriers (global writes of a phase
// are visible to the whole workgroup after the barrier):
//   1. split rows: merge each row's partial triples in split order -> lse, hbar;
//   2. per state, one wave: the mean over its unresolved rows -> h_state;
//   3. per pair, one thread: the gated, weighted hinge; a fixed-shape tree sums
//      numerators and weights. A pair is valid when its next state index lies
//      in [0, S), that state has an unresolved row and the source mean is finite.
__global__ void __launch_bounds__(kThreads) aec_reduce_kernel(AecArgs a) {
  if (a.nsplit > 1) {
    for (int row = threadIdx.x; row < a.n_rows; row += kThreads) {
      const float* p = a.part + (int64_t)row * a.nsplit * 3;
      Acc t{p[0], p[1], p[2]};
      for (int k = 1; k < a.nsplit; ++k) merge(t, Acc{p[3 * k], p[3 * k + 1], p[3 * k + 2]});
      finish(t, a.vocab, a.lse + row, a.hbar + row);
    }
    __threadfence_block();
    __syncthreads();
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int s = wave; s < a.n_states; s += kThreads / 64) {
    const float m = wave_state_mean(a, s, lane);
    if (lane == 0) a.h_state[s] = m;
  }
  __threadfence_block();
  __syncthreads();
  float num = 0.f, den = 0.f;
  for (int p = threadIdx.x; p < a.n_pairs; p += kThreads) {
    const int n = a.pair_next[p];
    const float hs = a.pair_h_source[p];
    if (n < 0 || n >= a.n_states || !__builtin_isfinite(hs) || !(hs <= a.gate_max)) continue;
    const float hn = a.h_state[n];
    if (!__builtin_isfinite(hn)) continue;
    const float w = a.pair_weight[p];
    const float h = fmaxf(0.f, hn - (1.f - a.rho) * hs);
    num = fmaf(w * h, h, num);
    den += w;
  }
  __shared__ float rn[kThreads], rd[kThreads];
  rn[threadIdx.x] = num;
  rd[threadIdx.x] = den;
  __syncthreads();
  for (int off = kThreads / 2; off > 0; off >>= 1) {
    if (threadIdx.x < off) {
      rn[threadIdx.x] += rn[threadIdx.x + off];
      rd[threadIdx.x] += rd[threadIdx.x + off];
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) a.loss[0] = rd[0] > 0.f ? rn[0] / rd[0] : 0.f;
}

// ------------------------------------------------------------------ backward
//
// dL/dx_iv = -c_i p_iv (log p_iv + H_i), with H_i = hbar_i ln V (nats),
// log p = x - lse and c_i = (dL/dHbar_i) / ln V. For an unresolved row of state
// s, dL/dHbar_i = dL/dH_s / |U_s|, and dL/dH_s is the sum over the kept valid
// pairs naming s as next state of 2 w_p hinge_p / D (times the upstream
// gradient). The captured source means are constants.

constexpr int kPairTile = 2048;

__device__ __forceinline__ bool pair_kept(const AecArgs& a, int p, float* w, float* hinge) {
  const int n = a.pair_next[p];
  const float hs = a.pair_h_source[p];
  if (n < 0 || n >= a.n_states || !__builtin_isfinite(hs) || !(hs <= a.gate_max)) return false;
  const float hn = a.h_state[n];
  if (!__builtin_isfinite(hn)) return false;
  *w = a.pair_weight[p];
  *hinge = fmaxf(0.f, hn - (1.f - a.rho) * hs);
  return true;
}

// One workgroup, four phases separated by barriers:
//   1. D = sum of the kept pairs' weights (fixed-shape tree); every row
//      coefficient and every state gradient set to 0 (state s by thread s % 256);
//   2. pairs staged through LDS in tiles; thread s % 256 adds, in pair order, the
//      contributions of the pairs naming state s;
//   3. one wave per state: its unresolved rows get dL/dH_s / (|U_s| ln V).
// Row ranges of the states must not overlap (state_rows non-decreasing) for the
// row coefficients to be well defined.
__global__ void __launch_bounds__(kThreads) aec_grad_coef_kernel(AecArgs a) {
  __shared__ float red[kThreads];
  __shared__ int tnext[kPairTile];
  __shared__ float tcontrib[kPairTile];
  float den = 0.f;
  for (int p = threadIdx.x; p < a.n_pairs; p += kThreads) {
    float w, h;
    if (pair_kept(a, p, &w, &h)) den += w;
  }
  red[threadIdx.x] = den;
  for (int i = threadIdx.x; i < a.n_rows; i += kThreads) a.row_coef[i] = 0.f;
  for (int s = threadIdx.x; s < a.n_states; s += kThreads) a.state_grad[s] = 0.f;
  __syncthreads();
  for (int off = kThreads / 2; off > 0; off >>= 1) {
    if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
    __syncthreads();
  }
  const float D = red[0];
  const float scale = D > 0.f ? 2.f * a.grad_loss[0] / D : 0.f;
  for (int p0 = 0; p0 < a.n_pairs; p0 += kPairTile) {
    const int np = min(kPairTile, a.n_pairs - p0);
    __syncthreads();                                  // the previous tile is consumed
    for (int q = threadIdx.x; q < np; q += kThreads) {
      float w = 0.f, h = 0.f;
      const bool kept = pair_kept(a, p0 + q, &w, &h);
      tnext[q] = kept ? a.pair_next[p0 + q] : -1;
      tcontrib[q] = scale * w * h;
    }
    __syncthreads();
    for (int q = 0; q < np; ++q) {
      const int n = tnext[q];
      if (n >= 0 && n % kThreads == (int)threadIdx.x) a.state_grad[n] += tcontrib[q];
    }
  }
  __threadfence_block();
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float inv_lnv = 1.f / logf((float)a.vocab);
  for (int s = wave; s < a.n_states; s += kThreads / 64) {
    const int lo = min(max(a.state_rows[s], 0), a.n_rows);
    const int hi = min(max(a.state_rows[s + 1], lo), a.n_rows);
    float cnt = 0.f;
    for (int i = lo + lane; i < hi; i += 64) cnt += a.unresolved[i] ? 1.f : 0.f;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
    const float c = cnt > 0.f ? a.state_grad[s] / cnt * inv_lnv : 0.f;
    for (int i = lo + lane; i < hi; i += 64)
      if (a.unresolved[i]) a.row_coef[i] = c;
  }
}

// ---------------------------------------------------------- LDS-resident forms
// The two single-workgroup kernels above chain several dependent memory round
// trips (partials -> entropies -> state means -> pairs; pairs -> D -> state
// gradients -> row coefficients), partly through values they have just written.
// For batches whose rows and states fit in LDS these forms request every input at
// the start (one round trip) and keep the intermediates in LDS; every sum runs in
// the same order as in the kernels above.
constexpr int kLdsRows = 8192;
constexpr int kLdsStates = 1024;

__device__ float lds_state_mean(const int* rows, const unsigned char* unres, const float* hbar, int n_rows, int s,
                                int lane) {
  const int lo = min(max(rows[s], 0), n_rows);
  const int hi = min(max(rows[s + 1], lo), n_rows);
  float sum = 0.f, cnt = 0.f;
  for (int i = lo + lane; i < hi; i += 64)
    if (unres[i]) { sum += hbar[i]; cnt += 1.f; }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    sum += __shfl_xor(sum, off);
    cnt += __shfl_xor(cnt, off);
  }
  return cnt > 0.f ? sum / cnt : __builtin_nanf("");
}

// States and the unresolved flags of the rows, into LDS (nothing when S = 0).
__device__ __forceinline__ void stage_states(const AecArgs& a, int* rows, unsigned char* unres) {
  if (a.n_states == 0) return;
  for (int s = threadIdx.x; s <= a.n_states; s += kThreads) rows[s] = a.state_rows[s];
  for (int r = threadIdx.x; r < a.n_rows; r += kThreads) unres[r] = a.unresolved[r];
}

__global__ void __launch_bounds__(kThreads) aec_reduce_lds_kernel(AecArgs a) {
  __shared__ float s_hbar[kLdsRows];
  __shared__ unsigned char s_unres[kLdsRows];
  __shared__ int s_rows[kLdsStates + 1];
  __shared__ float s_hstate[kLdsStates];
  __shared__ float rn[kThreads], rd[kThreads];
  const int tid = threadIdx.x;
  int n0 = -1;                                      // this thread's first pair
  float hs0 = 0.f, w0 = 0.f;
  if (tid < a.n_pairs) { n0 = a.pair_next[tid]; hs0 = a.pair_h_source[tid]; w0 = a.pair_weight[tid]; }
  stage_states(a, s_rows, s_unres);
  if (a.nsplit > 1) {
    for (int row = tid; row < a.n_rows; row += kThreads) {
      const float* p = a.part + (int64_t)row * a.nsplit * 3;
      Acc t{p[0], p[1], p[2]};
      for (int k = 1; k < a.nsplit; ++k) merge(t, Acc{p[3 * k], p[3 * k + 1], p[3 * k + 2]});
      s_hbar[row] = finish(t, a.vocab, a.lse + row, a.hbar + row);
    }
  } else {
    for (int row = tid; row < a.n_rows; row += kThreads) s_hbar[row] = a.hbar[row];
  }
  __syncthreads();
  const int lane = tid & 63, wave = tid >> 6;
  for (int s = wave; s < a.n_states; s += kThreads / 64) {
    const float m = lds_state_mean(s_rows, s_unres, s_hbar, a.n_rows, s, lane);
    if (lane == 0) { a.h_state[s] = m; s_hstate[s] = m; }
  }
  __syncthreads();
  float num = 0.f, den = 0.f;
  for (int p = tid; p < a.n_pairs; p += kThreads) {
    const int n = p == tid ? n0 : a.pair_next[p];
    const float hs = p == tid ? hs0 : a.pair_h_source[p];
    if (n < 0 || n >= a.n_states || !__builtin_isfinite(hs) || !(hs <= a.gate_max)) continue;
    const float hn = s_hstate[n];
    if (!__builtin_isfinite(hn)) continue;
    const float w = p == tid ? w0 : a.pair_weight[p];
    const float h = fmaxf(0.f, hn - (1.f - a.rho) * hs);
    num = fmaf(w * h, h, num);
    den += w;
  }
  rn[tid] = num;
  rd[tid] = den;
  __syncthreads();
  for (int off = kThreads / 2; off > 0; off >>= 1) {
    if (tid < off) {
      rn[tid] += rn[tid + off];
      rd[tid] += rd[tid + off];
    }
    __syncthreads();
  }
  if (tid == 0) a.loss[0] = rd[0] > 0.f ? rn[0] / rd[0] : 0.f;
}

// A pair's gate and hinge against state means in LDS (pair_kept's rule).
__device__ __forceinline__ bool lds_pair_kept(const AecArgs& a, const float* hstate, int n, float hs, float w_in,
                                              float* w, float* hinge) {
  if (n < 0 || n >= a.n_states || !__builtin_isfinite(hs) || !(hs <= a.gate_max)) return false;
  const float hn = hstate[n];
  if (!__builtin_isfinite(hn)) return false;
  *w = w_in;
  *hinge = fmaxf(0.f, hn - (1.f - a.rho) * hs);
  return true;
}

__global__ void __launch_bounds__(kThreads) aec_grad_coef_lds_kernel(AecArgs a) {
  __shared__ float red[kThreads];
  __shared__ int tnext[kPairTile];
  __shared__ float tcontrib[kPairTile];
  __shared__ float s_hstate[kLdsStates], s_sgrad[kLdsStates];
  __shared__ int s_rows[kLdsStates + 1];
  __shared__ unsigned char s_unres[kLdsRows];
  const int tid = threadIdx.x;
  int n0 = -1;
  float hs0 = 0.f, w0 = 0.f;
  if (tid < a.n_pairs) { n0 = a.pair_next[tid]; hs0 = a.pair_h_source[tid]; w0 = a.pair_weight[tid]; }
  for (int s = tid; s < a.n_states; s += kThreads) s_hstate[s] = a.h_state[s];
  stage_states(a, s_rows, s_unres);
  const float gl = a.grad_loss[0];
  __syncthreads();
  auto pair_at = [&](int p, int* n, float* hs, float* w) {
    if (p == tid) { *n = n0; *hs = hs0; *w = w0; }
    else { *n = a.pair_next[p]; *hs = a.pair_h_source[p]; *w = a.pair_weight[p]; }
  };
  float den = 0.f;
  for (int p = tid; p < a.n_pairs; p += kThreads) {
    int n;
    float hs, wi, w, h;
    pair_at(p, &n, &hs, &wi);
    if (lds_pair_kept(a, s_hstate, n, hs, wi, &w, &h)) den += w;
  }
  red[tid] = den;
  for (int i = tid; i < a.n_rows; i += kThreads) a.row_coef[i] = 0.f;
  for (int s = tid; s < a.n_states; s += kThreads) s_sgrad[s] = 0.f;
  __syncthreads();
  for (int off = kThreads / 2; off > 0; off >>= 1) {
    if (tid < off) red[tid] += red[tid + off];
    __syncthreads();
  }
  const float D = red[0];
  const float scale = D > 0.f ? 2.f * gl / D : 0.f;
  for (int p0 = 0; p0 < a.n_pairs; p0 += kPairTile) {
    const int np = min(kPairTile, a.n_pairs - p0);
    __syncthreads();                                  // the previous tile is consumed
    for (int q = tid; q < np; q += kThreads) {
      int n;
      float hs, wi, w = 0.f, h = 0.f;
      pair_at(p0 + q, &n, &hs, &wi);
      const bool kept = lds_pair_kept(a, s_hstate, n, hs, wi, &w, &h);
      tnext[q] = kept ? n : -1;
      tcontrib[q] = scale * w * h;
    }
    __syncthreads();
    for (int q = 0; q < np; ++q) {
      const int n = tnext[q];
      if (n >= 0 && n % kThreads == tid) s_sgrad[n] += tcontrib[q];
    }
  }
  __syncthreads();
  for (int s = tid; s < a.n_states; s += kThreads) a.state_grad[s] = s_sgrad[s];
  const int lane = tid & 63, wave = tid >> 6;
  const float inv_lnv = 1.f / logf((float)a.vocab);
  for (int s = wave; s < a.n_states; s += kThreads / 64) {
    const int lo = min(max(s_rows[s], 0), a.n_rows);
    const int hi = min(max(s_rows[s + 1], lo), a.n_rows);
    float cnt = 0.f;
    for (int i = lo + lane; i < hi; i += 64) cnt += s_unres[i] ? 1.f : 0.f;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) cnt += __shfl_xor(cnt, off);
    const float c = cnt > 0.f ? s_sgrad[s] / cnt * inv_lnv : 0.f;
    for (int i = lo + lane; i < hi; i += 64)
      if (s_unres[i]) a.row_coef[i] = c;
  }
}

__device__ __forceinline__ uint32_t pack_bf16x2(float x, float y) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v;
  v[0] = (__bf16)x;
  v[1] = (__bf16)y;
  return __builtin_bit_cast(uint32_t, v);
}

// dlogits of one row (or one part of it, as in the forward geometry); rows with
// a zero coefficient get zeros without reading their logits.
template <bool BF16>
__global__ void __launch_bounds__(kThreads) aec_grad_kernel(AecArgs a) {
  constexpr int EPV = BF16 ? 8 : 4;
  const int row = blockIdx.x / a.nsplit, split = blockIdx.x - row * a.nsplit;
  const int64_t c0 = (int64_t)split * a.chunk;
  const int64_t c1 = min((int64_t)a.vocab, c0 + a.chunk);
  const int64_t nvec = (c1 - c0) / EPV;
  const int tail = (int)((c1 - c0) - nvec * EPV);
  const int64_t off = (row * a.row_stride + c0) * (BF16 ? 2 : 4);
  const u32x4* vp = reinterpret_cast<const u32x4*>(static_cast<const char*>(a.logits) + off);
  u32x4* op = reinterpret_cast<u32x4*>(static_cast<char*>(a.dlogits) + off);
  const float c = a.row_coef[row];
  if (c == 0.f) {
    for (int64_t i = threadIdx.x; i < nvec; i += kThreads) op[i] = u32x4{0u, 0u, 0u, 0u};
    if (threadIdx.x < tail) {
      if constexpr (BF16) reinterpret_cast<uint16_t*>(op)[nvec * EPV + threadIdx.x] = 0;
      else reinterpret_cast<float*>(op)[nvec * EPV + threadIdx.x] = 0.f;
    }
    return;
  }
  const float lse = a.lse[row];
  const float H = a.hbar[row] * logf((float)a.vocab);
  auto grad = [&](float x) {
    const float lp = x - lse;
    return -c * ex2(lp * kL2E) * (lp + H);
  };
  auto grad_vec = [&](const u32x4& w) {
    float x[EPV];
    unpack<BF16>(w, x);
    u32x4 o;
    if constexpr (BF16) {
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = pack_bf16x2(grad(x[2 * k]), grad(x[2 * k + 1]));
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) o[k] = __builtin_bit_cast(uint32_t, grad(x[k]));
    }
    return o;
  };
  // eight 16-byte loads in flight per thread, all issued before the batch's stores
  // (each element is read and written by the same thread, so dlogits may be the
  // logits buffer itself)
  int64_t i = threadIdx.x;
  for (; i + 7 * kThreads < nvec; i += 8 * kThreads) {
    u32x4 w[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) w[k] = __builtin_nontemporal_load(vp + i + k * kThreads);
#pragma unroll
    for (int k = 0; k < 8; ++k) op[i + k * kThreads] = grad_vec(w[k]);
  }
  for (; i < nvec; i += kThreads) op[i] = grad_vec(__builtin_nontemporal_load(vp + i));
  if (threadIdx.x < tail) {
    const int64_t e = nvec * EPV + threadIdx.x;
    if constexpr (BF16) {
      const uint16_t b = reinterpret_cast<const uint16_t*>(vp)[e];
      const __bf16 r = (__bf16)grad(__builtin_bit_cast(float, (uint32_t)b << 16));
      reinterpret_cast<uint16_t*>(op)[e] = __builtin_bit_cast(uint16_t, r);
    } else {
      reinterpret_cast<float*>(op)[e] = grad(reinterpret_cast<const float*>(vp)[e]);
    }
  }
}

}  // namespace

hipError_t launch_aec_entropy(const AecArgs& a, bool bf16, hipStream_t s) {
  const int grid = a.n_rows * a.nsplit;
  if (bf16) hipLaunchKernelGGL(aec_entropy_kernel<true>, dim3(grid), dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(aec_entropy_kernel<false>, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_aec_reduce(const AecArgs& a, hipStream_t s) {
  if (a.n_rows <= kLdsRows && a.n_states <= kLdsStates)
    hipLaunchKernelGGL(aec_reduce_lds_kernel, dim3(1), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(aec_reduce_kernel, dim3(1), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_aec_grad_coef(const AecArgs& a, hipStream_t s) {
  if (a.n_rows <= kLdsRows && a.n_states <= kLdsStates)
    hipLaunchKernelGGL(aec_grad_coef_lds_kernel, dim3(1), dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL(aec_grad_coef_kernel, dim3(1), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_aec_grad(const AecArgs& a, bool bf16, hipStream_t s) {
  const int grid = a.n_rows * a.nsplit;
  if (bf16) hipLaunchKernelGGL(aec_grad_kernel<true>, dim3(grid), dim3(kThreads), 0, s, a);
  else hipLaunchKernelGGL(aec_grad_kernel<false>, dim3(grid), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace bdattn
