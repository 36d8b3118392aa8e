// Device-side helpers shared by the gfx950 kernels of the paged chunk-attention
// library: element types, conversions, wavefront reductions, the attended-key
// address map and the XCD-aware workgroup order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace oomb {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---- scalar element access (raw bf16 bits or fp32) ---------------------------------
struct bf16_t { uint16_t bits; };

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
  __bf16 b = static_cast<__bf16>(x);  // v_cvt_pk_bf16_f32: round to nearest even
  bf16_t r;
  r.bits = __builtin_bit_cast(uint16_t, b);
  return r;
}

// Pack two fp32 into one dword of two bf16 (lo = a, hi = b), round to nearest even:
// a single v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// ---- wavefront reductions (butterfly: every lane ends with the full result) -------
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) x += __shfl_xor(x, s, kWave);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) x = fmaxf(x, __shfl_xor(x, s, kWave));
  return x;
}

// ---- attended keys of one chunk -------------------------------------------------------
// The keys a chunk attends, per KV head, are numbered a = 0, 1, ...: first the
// selected prior pages in list order (all prior pages when dense), then the local
// pages [first_local, last_local]. Key a sits in list entry a / P, slot a % P.
struct AttendMap {
  const int32_t* table;   // this head's page-table row
  const int32_t* sel;     // this head's selected logical pages, or nullptr (dense)
  int n_sel;              // entries taken from sel (or number of prior pages if dense)
  int prior0;             // dense: logical page of entry 0 (0, or a window's first page)
  int first_local;        // first local logical page
  int n_pages_att;        // n_sel + number of local pages
  int64_t num_pages;      // pool size, for the bounds check
  int log2p;              // log2(page size)

  // Logical page of list entry e.
  __device__ __forceinline__ int logical(int e) const {
    if (e < n_sel) return sel ? sel[e] : prior0 + e;
    return first_local + (e - n_sel);
  }
  // Physical page of list entry e, or -1 when the entry is out of range.
  __device__ __forceinline__ int64_t physical(int e, int lp) const {
    if (lp < 0) return -1;
    int64_t ph = table[lp];
    return (ph >= 0 && ph < num_pages) ? ph : -1;
  }
};

// Clamp a device-side selection count into [0, min(sel_stride, n_cand)].
__device__ __forceinline__ int clamp_count(const int32_t* count, int g, int64_t sel_stride,
                                           int n_cand) {
  int c = count[g];
  int hi = static_cast<int>(sel_stride < n_cand ? sel_stride : n_cand);
  return c < 0 ? 0 : (c > hi ? hi : c);
}

// ---- XCD-aware workgroup order ---------------------------------------------------------
// Workgroups are dispatched round-robin over the 8 XCDs (workgroup i runs on XCD
// i % 8), and within an XCD to whichever CU frees up first. A grid of n workgroups
// holds n / Hkv work units per KV head, each head's units numbered longest first.
// head_unit gives workgroup i its (head, unit): each head's units run on their own
// 8 / Hkv XCDs (the head's keys and queries share those XCDs' L2) and are dealt
// round-robin among them, so every XCD receives the same mix of long and short units
// in longest-first order and the greedy fill of its CUs ends evenly. When Hkv does not
// divide 8 (or n is not a multiple of 8) the units are taken head by head instead.
struct HeadUnit {
  int head, unit;
};
__device__ __forceinline__ HeadUnit head_unit(int i, int n, int n_heads) {
  constexpr int kXcd = 8;
  const int per = n / n_heads;
  if (kXcd % n_heads != 0 || n % kXcd != 0) return {i / per, i % per};
  const int x_per_head = kXcd / n_heads;
  const int x = i % kXcd, local = i / kXcd;
  return {x / x_per_head, local * x_per_head + x % x_per_head};
}

// Unit u of one KV head under a split plan: the head's first `whole` tiles (in its
// longest-first tile order) are one unit each; every later tile is n_ks consecutive
// units, one per key range.
struct TileRange {
  int tile, range, n_ranges;
};
__device__ __forceinline__ TileRange tile_range(int u, int whole, int n_ks) {
  if (u < whole) return {u, 0, 1};
  const int v = u - whole;
  return {whole + v / n_ks, v % n_ks, n_ks};
}

}  // namespace oomb
