// Device helpers for the gfx950 kernels: vector types, MFMA wrappers, LDS tile
// layouts and the row-limit predicate.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bd_records.h"

namespace bdattn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Lazy rescaling: the running maximum (log2 domain) is only raised when a new
// score exceeds it by more than this, so unnormalised weights stay below 2^8.
constexpr float kRescaleSlack = 8.0f;

// 32x32x16 bf16 MFMA, fp32 accumulate. Lane l supplies A[l%32][8*(l/32)+e] and
// B[8*(l/32)+e][l%32] (e = 0..7); it receives C[8*(r/4)+4*(l/32)+r%4][l%32] in
// register r (r = 0..15).
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of a 32x32 MFMA result held by register r of a lane in half h (= lane/32).
__device__ __forceinline__ constexpr int c_row(int r, int h) { return 8 * (r >> 2) + 4 * h + (r & 3); }

// Column permutation of transposed LDS tiles. An MFMA result's column values in
// registers 8s..8s+7 of half h are the rows 16s + {0..3, 8..11} + 4h; packing
// them in register order gives the B operand of the next product, so the
// matching A operand must hold those rows at k slots 16s + 8h + 0..7. Storing
// index i of a transposed tile at column kperm(i) makes those 8 slots one
// contiguous 16-byte LDS read. kperm keeps aligned groups of 4 contiguous.
__device__ __forceinline__ constexpr int kperm(int i) {
  return (i & ~15) | (((i >> 2) & 1) << 3) | (((i >> 3) & 1) << 2) | (i & 3);
}

// Natural tile [rows][D + 8] (bf16): 16-byte row padding keeps 8 consecutive
// rows on distinct bank groups for 16-byte reads.
template <int D>
struct NatTile {
  static constexpr int kStride = D + 8;
  __device__ static __forceinline__ int off(int row, int col) { return row * kStride + col; }
};

// Transposed tile [D][NCOL] (bf16) with 16-byte chunks XOR-swizzled per row, so
// that 8 consecutive rows read at one column chunk hit distinct banks.
template <int NCOL>
struct TrTile {
  static constexpr int kChunks = NCOL / 8;
  __device__ static __forceinline__ int swz(int d) {
    if (kChunks == 8) return (d ^ (d >> 3)) & 7;
    return ((d >> 1) ^ (d >> 3)) & (kChunks - 1);
  }
  // element offset of (row d, column c)
  __device__ static __forceinline__ int off(int d, int c) {
    return d * NCOL + ((((c >> 3) ^ swz(d))) << 3) + (c & 7);
  }
};

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v;
  v[0] = (bf16)a;
  v[1] = (bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// Eight fp32 registers -> one bf16x8 MFMA operand.
__device__ __forceinline__ bf16x8 pack8(const float* x) {
  u32x4 u;
  u[0] = pack_bf16x2(x[0], x[1]);
  u[1] = pack_bf16x2(x[2], x[3]);
  u[2] = pack_bf16x2(x[4], x[5]);
  u[3] = pack_bf16x2(x[6], x[7]);
  return __builtin_bit_cast(bf16x8, u);
}

// bf16 element (odd ? high : low) of dword x, then of dword y, packed as one dword.
__device__ __forceinline__ uint32_t pick_pair(uint32_t x, uint32_t y, int odd) {
  return odd ? ((x >> 16) | (y & 0xffff0000u)) : ((x & 0xffffu) | (y << 16));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of x from lane l ^ 32 combined with the own one: returns (own, other).
__device__ __forceinline__ float swap_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x), false, false);
  // lanes < 32 receive the upper half's value in r[1], lanes >= 32 the lower half's in r[0]
  const int lane = threadIdx.x & 63;
  return __builtin_bit_cast(float, lane < 32 ? r[1] : r[0]);
}

// Limit on clean-key context positions visible to query token t of a tile.
__device__ __forceinline__ int row_limit(const QTile& qt, int t, int B) {
  return qt.pos0 >= 0 ? ((qt.pos0 + t) / B + 1) * B : qt.lim_min;
}

__device__ __forceinline__ QTile load_qtile(const int32_t* base, int i) {
  const int4* p = reinterpret_cast<const int4*>(base) + 2 * i;
  int4 a = p[0], b = p[1];
  QTile q;
  q.q_tok = a.x; q.n_tok = a.y; q.k_ctx = a.z; q.pos0 = a.w;
  q.lim_max = b.x; q.lim_min = b.y; q.k_own = b.z; q.n_own = b.w;
  return q;
}

__device__ __forceinline__ KTile load_ktile(const int32_t* base, int i) {
  const int4* p = reinterpret_cast<const int4*>(base) + 2 * i;
  int4 a = p[0], b = p[1];
  KTile k;
  k.k_tok = a.x; k.n_keys = a.y; k.p0 = a.z; k.cq_tok = a.w;
  k.cq_len = b.x; k.cq_pos = b.y; k.cv_begin = b.z; k.cv_count = b.w;
  return k;
}

}  // namespace bdattn
