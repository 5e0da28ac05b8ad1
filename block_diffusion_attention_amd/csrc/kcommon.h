// Device helpers for the gfx950 kernels: vector types, MFMA wrappers, LDS tile
// layouts and the row-limit predicate.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

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

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. N-1, fully
// expanded, so register arrays are only ever indexed with constants.
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

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

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------------------
// Global -> LDS copies and LDS reads shared by the tile layouts below.
typedef __attribute__((address_space(3))) void lds_void;

// Asynchronous copy global -> LDS of 16 (dma_b128) or 4 (dma_b32) bytes per lane:
// lane l writes LDS bytes dst + 16 l (4 l); dst is the same for the whole wave
// (it goes into M0). Written as inline assembly rather than the compiler builtin:
// the compiler counts a builtin copy in flight as a pending LDS access of the
// kind that completes out of order, and then turns every wait for an LDS read
// into a full drain (lgkmcnt(0)), which defeats any read-ahead of MFMA operands.
// The hardware tracks these copies with the vector memory counter only; callers
// wait for them with explicit vmcnt waits (or a barrier that waits vmcnt(0))
// before reading the destination.
// dst is a generic pointer into LDS: the low 32 bits of a flat LDS address are its
// LDS offset, so no address-space conversion (and its null check) is needed.
__device__ __forceinline__ uint32_t lds_offset(const void* dst) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)dst);
}
__device__ __forceinline__ void dma_b128(const void* src, void* dst) {
  const uint32_t m = lds_offset(dst);
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m) : "memory");
}
__device__ __forceinline__ void dma_b32(const void* src, void* dst) {
  const uint32_t m = lds_offset(dst);
  asm volatile("global_load_lds_dword %0, off" ::"v"(src), "{m0}"(m) : "memory");
}
// The same copy with a wave-uniform 64-bit base in scalar registers and a 32-bit
// per-lane byte offset (the instruction's scalar-base form): no per-lane 64-bit
// address arithmetic when the offsets are fixed.
__device__ __forceinline__ void dma_b128_sv(const void* sbase, uint32_t voff, void* dst) {
  const uint32_t m = lds_offset(dst);
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(m) : "memory");
}
typedef short v4i16 __attribute__((ext_vector_type(4)));

// ds_read_b64_tr_b16. Within each group of 16 lanes, lane s supplies the address
// of 4 consecutive bf16 M[s][0..3]; lane i of the group receives
// M[i/4 + 4e][i%4] for e = 0..3.
__device__ __forceinline__ v4i16 lds_tr4(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)((__attribute__((address_space(3))) char*)(lds_void*)(p)));
}

// ---------------------------------------------------------------------------
// Swizzled row-major tiles. A tile holds 64 rows of D bf16 (CH = D/8 16-byte
// chunks per row) with chunk c of row r in 16-byte slot
//   r * CH + (c ^ sw(r)),  sw(r) = 4 (r & 3) + ((r >> 2) & 3)            (D = 128)
//                          sw(r) = 4 ((r >> 1) & 1) + ((r >> 2) & 3)     (D = 64)
// One copy instruction (lane l to slot 64 m + l) covers 4 (8) whole rows, so it
// touches a few cache lines instead of 64. Reads with the 64-bank LDS:
//   - natural MFMA operands (16 rows at one chunk per 16-lane pass) hit 16
//     distinct 16-byte bank groups, since sw is a bijection on r mod 16 (for
//     D = 64 on each parity class);
//   - transposed reads (4 rows x 4 aligned chunks per 32-lane pass) too, since
//     the 4 rows differ in sw's high bits, which select the aligned chunk group.
// The XOR mixes lane-dependent bits with the compile-time chunk index, so each
// lane keeps one offset per operand variant (NKS natural, 2 NDB transposed).
template <int D>
__device__ __forceinline__ constexpr int swz(int r) {
  return D == 128 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

template <int D>
struct SwLane {
  static constexpr int CH = D / 8, NKS = D / 16, NDB = D / 32;
  int a[NKS];        // natural operand: row j = lane%32 of a 32-row block, chunk 2kk + lane/32
  int t[NDB][2];     // transposed operand: 32-column block db, 8-row half jj of a 16-row step
  __device__ explicit SwLane(int lane) {
    const int j = lane & 31, h = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < NKS; ++kk) a[kk] = 16 * (j * CH + ((2 * kk + h) ^ swz<D>(j)));
    const int g = lane >> 4, s = lane & 15;
    const int cl = 2 * (g & 1) + ((s & 3) >> 1);
    const int rl = 4 * (g >> 1) + (s >> 2);
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int w = swz<D>(rl + 8 * jj);
        t[db][jj] = 16 * ((rl + 8 * jj) * CH + 4 * (db ^ (w >> 2)) + (cl ^ (w & 3))) + 8 * (s & 1);
      }
  }
};

// Natural MFMA operand: row rbase + lane%32 (rbase a multiple of 32), elements
// 16kk + 8h .. +7 (h = lane/32).
template <int D>
__device__ __forceinline__ bf16x8 sw_row8(const bf16* tile, const SwLane<D>& o, int rbase, int kk) {
  const char* p = reinterpret_cast<const char*>(tile) + 16 * rbase * (D / 8) + o.a[kk];
  return *reinterpret_cast<const bf16x8*>(p);
}

// Transposed MFMA A operand: A[i][k] = T[row0 + r(k)][col0 + i] for output row
// i = lane%32, where slot 8h + 4jj + e reads row row0 + 8jj + 4h + e (jj = 0, 1;
// e = 0..3) -- the slot order of a 32x32 MFMA result's registers 0..7 (c_row),
// so a packed previous result is the matching B operand. row0 is a multiple of
// 16, col0 of 32.
template <int D>
__device__ __forceinline__ bf16x8 sw_tr8(const bf16* tile, const SwLane<D>& o, int row0, int col0) {
  const char* base = reinterpret_cast<const char*>(tile) + 16 * row0 * (D / 8);
  const u32x2 lo = __builtin_bit_cast(u32x2, lds_tr4(base + o.t[col0 >> 5][0]));
  const u32x2 hi = __builtin_bit_cast(u32x2, lds_tr4(base + o.t[col0 >> 5][1]));
  return __builtin_bit_cast(bf16x8, u32x4{lo[0], lo[1], hi[0], hi[1]});
}

// Async copy of 64-row swizzled tiles whose rows sit at fixed element offsets
// from a per-tile base pointer (offsets of rows 0..63 are the same for every
// tile). The per-lane parts (row, swizzled chunk and offset of each of the
// wave's D/32 copy instructions) are computed once; a fetch then only selects
// the last valid row for rows at or past nvalid.
template <int D>
struct SwFetch {
  static constexpr int CH = D / 8, RPI = 64 / CH, PER_WAVE = CH / 4;
  int row[PER_WAVE], col[PER_WAVE], off[PER_WAVE];
  template <class RowOff>
  __device__ SwFetch(RowOff row_off, int wave, int lane) {
#pragma unroll
    for (int n = 0; n < PER_WAVE; ++n) {
      const int r = (wave * PER_WAVE + n) * RPI + lane / CH;
      row[n] = r;
      col[n] = ((lane % CH) ^ swz<D>(r)) * 8;
      off[n] = row_off(r) + col[n];
    }
  }
  // base: wave-uniform (it goes into scalar registers); offsets are byte offsets
  // from it, below 2^32. last_off: element offset of row nvalid - 1 (any valid row
  // works for the rows past the end: their values are never used). A whole tile
  // takes the fixed offsets as they are.
  // SCALAR_BASE = false keeps 64-bit per-lane addresses (fewer scalar registers,
  // for kernels at their register limit).
  template <bool SCALAR_BASE = true>
  __device__ __forceinline__ void issue(bf16* tile, const bf16* base, int nvalid, int last_off, int wave) const {
    if constexpr (!SCALAR_BASE) {
#pragma unroll
      for (int n = 0; n < PER_WAVE; ++n) {
        const int o = row[n] < nvalid ? off[n] : last_off + col[n];
        dma_b128(base + o, tile + (wave * PER_WAVE + n) * 64 * 8);
      }
    } else if (nvalid >= 64) {
#pragma unroll
      for (int n = 0; n < PER_WAVE; ++n)
        dma_b128_sv(base, 2u * (uint32_t)off[n], tile + (wave * PER_WAVE + n) * 64 * 8);
    } else {
#pragma unroll
      for (int n = 0; n < PER_WAVE; ++n) {
        const int o = row[n] < nvalid ? off[n] : last_off + col[n];
        dma_b128_sv(base, 2u * (uint32_t)o, tile + (wave * PER_WAVE + n) * 64 * 8);
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Padded row-major tiles. A tile of ROWS rows x CH 16-byte chunks keeps each row
// in CH + 1 slots: chunk (r, c) sits in slot r * (CH + 1) + c (the last slot of a
// row is padding). One global_load_lds instruction (lane l writes slot 64 m + l)
// covers whole rows apart from the two ends, i.e. a few cache lines, and MFMA
// operand reads of 16 consecutive rows at one chunk land in 16 distinct 16-byte
// bank groups of the 64-bank LDS (the row stride is odd in 16-byte units), with
// addresses affine in the chunk index (one base register per lane).
template <int ROWS, int CH>
struct PadTile {
  static constexpr int kStride = CH + 1;                      // slots per row
  static constexpr int kSlots = ROWS * kStride;
  static constexpr int kInstr = kSlots / 64;                  // DMA instructions per tile
  static_assert(kSlots % 64 == 0, "tile must be whole DMA instructions");
  static constexpr int kElems = kSlots * 8;                   // bf16 elements of LDS
};

// Issues the async copy of one padded tile, instructions m = wave, wave + 4, ...
// Row r is read from base + min(r, nvalid - 1) * row_stride (elements; the offset
// of the last row fits in 31 bits) and padding slots read chunk 0 of their row,
// so every address is inside the tensor.
template <int ROWS, int CH>
__device__ __forceinline__ void pad_tile_fetch(bf16* tile, const bf16* base, int row_stride, int nvalid, int wave,
                                               int lane) {
  using T = PadTile<ROWS, CH>;
#pragma unroll
  for (int m0 = 0; m0 < T::kInstr; m0 += 4) {
    const int m = m0 + wave;
    if (m < T::kInstr) {
      const int s = m * 64 + lane;
      const int r = s / T::kStride, c = s - r * T::kStride;
      const uint32_t boff = 2u * (uint32_t)(min(r, nvalid - 1) * row_stride + (c < CH ? c : 0) * 8);
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const char*>(base) + boff,
                                       (lds_void*)(tile + m * 64 * 8), 16, 0, 0);
    }
  }
}

// Natural MFMA operand from a padded tile: row rbase + lane%32, chunk
// 2kk + lane/32; base = 16 * ((lane%32) * (CH + 1) + lane/32).
template <int CH>
__device__ __forceinline__ int pad_base(int lane) { return 16 * ((lane & 31) * (CH + 1) + (lane >> 5)); }

template <int CH>
__device__ __forceinline__ bf16x8 pad_row8(const bf16* tile, int base, int rbase, int kk) {
  const char* p = reinterpret_cast<const char*>(tile) + base + 16 * (rbase * (CH + 1) + 2 * kk);
  return *reinterpret_cast<const bf16x8*>(p);
}

// Waits for this wave's outstanding global loads (including those into LDS).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0); }

// s_waitcnt immediate that waits until at most n vector-memory operations of this
// wave are outstanding and leaves the LDS/scalar and export counters unconstrained
// (gfx9 encoding: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[15:14]).
__host__ __device__ constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
// ... and the one that waits for this wave's LDS operations only.
constexpr int kLgkm0Imm = 15 | (7 << 4) | (0 << 8) | (3 << 14);

// Workgroup barrier that orders LDS accesses only. Unlike __syncthreads() it does
// not wait for this wave's outstanding global loads (a memory fence would, since
// loads that write LDS asynchronously count as pending LDS writes), so loads
// issued for later pipeline stages stay in flight; the caller first waits (vmcnt)
// for the loads of the stage it is about to read. The empty asm statements keep
// the compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kLgkm0Imm);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Value of x from lane l ^ 32 combined with the own one: returns (own, other).
__device__ __forceinline__ float swap_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x), false, false);
  // lanes < 32 receive the upper half's value in r[1], lanes >= 32 the lower half's in r[0]
  const int lane = threadIdx.x & 63;
  return __builtin_bit_cast(float, lane < 32 ? r[1] : r[0]);
}

// Limit on clean-key context positions visible to query token t of a tile: the
// first row's limit, raised by the grain at every multiple of it that the grid
// position crosses from the first row to row t (constant for a canvas tile).
__device__ __forceinline__ int row_limit(const QTile& qt, int t, int grain) {
  return qt.pos0 >= 0 ? qt.lim_min + ((qt.pos0 + t) / grain - qt.pos0 / grain) * grain : qt.lim_min;
}

// Work-list records are read through the constant address space with a
// wave-uniform index, so they come in with scalar loads (counted by lgkmcnt, not
// by vmcnt: waiting for them never waits for the global loads in flight).
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(4))) const i32x4 ci32x4;

__device__ __forceinline__ int4 ld_rec4(const void* base, int i) {
  const int u = __builtin_amdgcn_readfirstlane(i);
  const i32x4 v = reinterpret_cast<ci32x4*>(reinterpret_cast<uintptr_t>(base))[u];
  return make_int4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ int ld_rec1(const void* base, int i) {
  const int u = __builtin_amdgcn_readfirstlane(i);
  return reinterpret_cast<__attribute__((address_space(4))) const int*>(reinterpret_cast<uintptr_t>(base))[u];
}

__device__ __forceinline__ QTile load_qtile(const int32_t* base, int i) {
  int4 a = ld_rec4(base, 2 * i), b = ld_rec4(base, 2 * i + 1);
  QTile q;
  q.q_tok = a.x; q.n_tok = a.y; q.k_ctx = a.z; q.pos0 = a.w;
  q.lim_max = b.x; q.lim_min = b.y; q.k_own = b.z; q.n_own = b.w;
  return q;
}

// Work of one forward workgroup: its query tile, kv head, key-tile range and, on
// the split path, the partial slot it writes.
struct FwdWork {
  QTile qt;
  int kvh, kt_begin, kt_end, slot;
};

// ---------------------------------------------------------------------------
// Device-side record checks (plans made with BD_ATTN_FLAG_DEBUG_CHECKS). Every
// kernel has a CHK template parameter; its CHK instantiation checks each work
// record a workgroup reads against the list and tensor sizes before it follows any
// index or token range in it. A record that fails is counted (one counter per
// source file and device, read and cleared from the host) and its workgroup does
// nothing. The values checked are wave-uniform and every wave of a workgroup reads
// the same records, so a rejected workgroup leaves as a whole, before its first
// barrier. In the instantiations without CHK every check folds away.
static __device__ unsigned long long g_bad_records;

// Host side of the counter: NAME(count, reset) waits for all work on the current
// device, adds the count of that device's copy to *count and clears it when asked.
// Each source file that launches checked kernels defines one with a name of its own.
#define BD_ATTN_DEVICE_ERRORS_QUERY(NAME)                                                  \
  hipError_t NAME(uint64_t* count, bool reset) {                                           \
    void* p = nullptr;                                                                     \
    hipError_t e = hipDeviceSynchronize();                                                 \
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_bad_records));           \
    if (e != hipSuccess) return e;                                                         \
    unsigned long long v = 0;                                                              \
    if ((e = hipMemcpy(&v, p, sizeof v, hipMemcpyDeviceToHost)) != hipSuccess) return e;   \
    *count += v;                                                                           \
    if (reset) {                                                                           \
      const unsigned long long zero = 0;                                                   \
      e = hipMemcpy(p, &zero, sizeof zero, hipMemcpyHostToDevice);                         \
    }                                                                                      \
    return e;                                                                              \
  }

// True (and the record counted, once per workgroup) when a checking instantiation
// finds `bad`; always false in the others.
template <bool CHK>
__device__ __forceinline__ bool reject_record(bool bad) {
  if constexpr (CHK) {
    if (bad) {
      if (threadIdx.x == 0) atomicAdd(&g_bad_records, 1ull);
      return true;
    }
  }
  (void)bad;
  return false;
}

// A query tile's rows lie in [0, Tq) and fill at most one tile; its clean and own
// key ranges lie in [0, Tk).
__device__ __forceinline__ bool qtile_in_bounds(const QTile& t, int G, int64_t tq, int64_t tk) {
  return t.q_tok >= 0 && t.n_tok >= 1 && t.n_tok * G <= kQRows && (int64_t)t.q_tok + t.n_tok <= tq &&
         t.lim_min >= 0 && t.lim_min <= t.lim_max && t.k_ctx >= 0 && (int64_t)t.k_ctx + t.lim_max <= tk &&
         t.n_own >= 0 && (t.n_own == 0 || (t.k_own >= 0 && (int64_t)t.k_own + t.n_own <= tk));
}

// A key-tile range [b, e) within a query tile's list (its clean tiles, then its own).
__device__ __forceinline__ bool key_range_in_bounds(const QTile& t, int b, int e) {
  const int n = (t.lim_max + kKTile - 1) / kKTile + (t.n_own + kKTile - 1) / kKTile;
  return b >= 0 && b <= e && e <= n;
}

// A key tile's keys lie in [0, Tk), its clean query range in [0, Tq) and its
// canvas-query entries in their list.
__device__ __forceinline__ bool ktile_in_bounds(const KTile& t, int64_t tq, int64_t tk, int n_canvq) {
  return t.k_tok >= 0 && t.n_keys >= 1 && t.n_keys <= kKBlock && (int64_t)t.k_tok + t.n_keys <= tk &&
         t.cq_len >= 0 && (t.cq_len == 0 || (t.cq_tok >= 0 && (int64_t)t.cq_tok + t.cq_len <= tq)) &&
         t.cv_begin >= 0 && t.cv_count >= 0 && (int64_t)t.cv_begin + t.cv_count <= n_canvq;
}

// A canvas-query entry holds one whole canvas (B rows) in [0, Tq).
__device__ __forceinline__ bool canvq_in_bounds(const int4& e, int B, int64_t tq) {
  return e.x >= 0 && e.y == B && (int64_t)e.x + e.y <= tq && e.z >= 0 && (e.w == 0 || e.w == 1);
}

// Every canvas-query entry a key tile lists (its range already checked).
__device__ __forceinline__ bool ktile_canvq_in_bounds(const KTile& t, const void* canvq, int B, int64_t tq) {
  bool ok = true;
  for (int e = 0; e < t.cv_count; ++e) ok &= canvq_in_bounds(ld_rec4(canvq, t.cv_begin + e), B, tq);
  return ok;
}

// Direct path: item i (launch order) and its query tile, two dependent scalar
// loads. Returns false for an empty launch slot (and, with CHK, for an item whose
// query tile index lies outside the n_qtiles tiles).
template <bool CHK>
__device__ __forceinline__ bool load_fwd_work(const void* items, const int32_t* qtiles, int i, FwdWork* w,
                                              int n_qtiles) {
  const int4 itv = ld_rec4(items, i);
  if (itv.x < 0) return false;
  if (reject_record<CHK>(itv.x >= n_qtiles)) return false;
  w->kvh = itv.y; w->kt_begin = itv.z; w->kt_end = itv.w; w->slot = -1;
  w->qt = load_qtile(qtiles, itv.x);
  return true;
}

// Split path: item i carries its query tile; its three 16-byte parts are
// independent scalar loads (one memory round trip).
__device__ __forceinline__ bool load_split_work(const void* splits, int i, FwdWork* w) {
  const int4 a = ld_rec4(splits, 4 * i), b = ld_rec4(splits, 4 * i + 1), c = ld_rec4(splits, 4 * i + 2);
  w->qt.q_tok = a.x; w->qt.n_tok = a.y; w->qt.k_ctx = a.z; w->qt.pos0 = a.w;
  w->qt.lim_max = b.x; w->qt.lim_min = b.y; w->qt.k_own = b.z; w->qt.n_own = b.w;
  w->kvh = c.x; w->kt_begin = c.y; w->kt_end = c.z; w->slot = c.w;
  return w->kvh >= 0;
}

// Split part i of a regular split grid (one query tile whose key range of ntiles
// tiles each kv head cuts into parts of tps tiles): kv head i % hkv, part i / hkv,
// slot kv head * parts + part. Computed from the index: no dependent record load.
__device__ __forceinline__ void grid_split_work(const QTile& qt, int hkv, int parts, int tps, int ntiles, int i,
                                                FwdWork* w) {
  const int kvh = i % hkv, part = i / hkv;
  w->qt = qt;
  w->kvh = kvh;
  w->kt_begin = part * tps;
  w->kt_end = min(ntiles, (part + 1) * tps);
  w->slot = kvh * parts + part;
}

// A forward work item (either path) whose kv head, query tile, key-tile range and
// partial slot (split path) are in bounds.
__device__ __forceinline__ bool fwd_work_in_bounds(const FwdWork& w, bool split, int G, int hkv, int64_t tq,
                                                   int64_t tk, int n_slots) {
  return w.kvh >= 0 && w.kvh < hkv && qtile_in_bounds(w.qt, G, tq, tk) &&
         key_range_in_bounds(w.qt, w.kt_begin, w.kt_end) && (!split || (w.slot >= 0 && w.slot < n_slots));
}

// Partial result of a split workgroup, in register order (see the layout next to
// kMergeThreads): wave w's acc[db][8 p .. 8 p + 7] times inv (the part's own row
// sum) as 8 bf16 per lane, one contiguous 1 KiB store per (db, p); the part's
// LSE of row 32 w + j from lane j.
template <int D>
__device__ __forceinline__ void store_partial(void* part_o, float* part_lse, int slot, int wave, int lane,
                                              const f32x16 (&acc)[D / 32], float inv, float lse) {
  constexpr int NDB = D / 32;
  bf16* po = static_cast<bf16*>(part_o) + ((int64_t)(slot * 4 + wave) * NDB * 2) * 512 + 8 * lane;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = acc[db][8 * p + e] * inv;
      *reinterpret_cast<bf16x8*>(po + (db * 2 + p) * 512) = pack8(x);
    }
  if (lane < 32) part_lse[(int64_t)slot * kQRows + wave * 32 + lane] = lse;
}

__device__ __forceinline__ KTile load_ktile(const int32_t* base, int i) {
  int4 a = ld_rec4(base, 2 * i), b = ld_rec4(base, 2 * i + 1);
  KTile k;
  k.k_tok = a.x; k.n_keys = a.y; k.p0 = a.z; k.cq_tok = a.w;
  k.cq_len = b.x; k.cq_pos = b.y; k.cv_begin = b.z; k.cv_count = b.w;
  return k;
}

}  // namespace bdattn
