// Shared pieces of the matrix-core paged chunk-attention kernels for gfx950 (bf16
// inputs, head_dim 128): MFMA wrappers, swizzled LDS tiles and their fragments, the
// attended-key map, and direct global->LDS staging of key blocks. The kernels live in
// attn_fwd_mfma.hip (forward), attn_dq_mfma.hip (dQ) and attn_dkdv_mfma.hip (dK/dV).
//
// Method (gist.science explainer of OOMB): 2.A chunk-recurrent training with
// recomputation (the backward recomputes P from the saved log-sum-exp); 2.B paged
// K/V and paged K/V gradients, accumulated in place; 2.D page-level top-k sparsity
// (the attended page list is the selected pages followed by the chunk's own pages).
//
// Design (every product is v_mfma_f32_32x32x16_bf16 on 64-lane wavefronts):
//  * Tiles are staged in LDS row-major, 128 bf16 (256 B) per row, with the 16-byte
//    chunks of row r XOR-swizzled by f(r) = 4(r%4) + (r/4)%4. Row fragments (a lane
//    reads 8 consecutive columns of one row) and transposed fragments (a lane reads
//    one column of 8 rows, through ds_read_b64_tr_b16) are then both free of bank
//    conflicts, and no tile is ever stored transposed.
//  * The physical page ids a workgroup attends are copied into LDS once, so a key
//    block's rows are addressed without a dependent table walk.
//  * Forward and dQ compute S^T = K Q^T so that a lane owns one query column: the
//    row max, row sum, LSE and Delta are lane scalars, and the C layout of S^T is
//    directly the B operand of the next product (P^T or dS^T). The forward rescales
//    its output only when a row maximum grows by more than 2^8 (exact: P and the
//    running sum always share one reference), which removes almost every rescale.
//  * The dK/dV pass owns 128 keys per workgroup (32 per wavefront, K and V held in
//    registers), streams the query tiles of all heads of its KV group through
//    double-buffered LDS, and does one read-modify-write of its gradient rows. When
//    that grid would under-fill the GPU the query stream is split across workgroups;
//    each split writes fp32 partials and a merge kernel adds them in split order.
//    No two workgroups ever write the same gradient row: no atomics, no races, and
//    bit-reproducible results.
//  * Workgroup ids are remapped so that each XCD works on one contiguous range (one
//    KV head's queries and pages share that XCD's L2).
#pragma once

#include "device_common.hpp"
#include "launch.hpp"
#include "profiling.hpp"

namespace oomb {
namespace mf {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int D = 128;
constexpr int KB = 64;        // keys per block (forward / dQ)
constexpr int PCAP = 2048;    // attended page ids held in LDS at a time
constexpr float kTau = 8.0f;  // lazy-rescale threshold (log2 units)
constexpr int KPW = 128;      // keys per workgroup in the dK/dV pass (32 per wavefront)
constexpr int QTB = 64;       // queries per staged tile in the dK/dV pass

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// ---- swizzled row-major tiles -----------------------------------------------------------
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// Element offset of (row r, column c) with c a multiple of 4.
__device__ __forceinline__ int toff(int r, int c) {
  return r * D + ((((c >> 3) ^ swz(r))) << 3) + (c & 7);
}
__device__ __forceinline__ u32x4 lds16(const uint16_t* t, int off) {
  return *reinterpret_cast<const u32x4*>(t + off);
}
__device__ __forceinline__ void sts16(uint16_t* t, int off, u32x4 v) {
  *reinterpret_cast<u32x4*>(t + off) = v;
}

// Row fragment: lane l reads row r0 + (l%32), columns 16kk + 8(l/32) .. +7.
// Used as the A operand (rows = M) or the B operand (rows = N) of a product over d.
__device__ __forceinline__ bf16x8 row_frag(const uint16_t* t, int r0, int kk, int lane) {
  return as_bf16x8(lds16(t, toff(r0 + (lane & 31), 16 * kk + 8 * (lane >> 5))));
}

// Transposed fragment for k-step s of a 32-row sub-tile starting at row r0: lane l
// gets column c0 + (l%32) of rows r0 + 16s + 8(j/4) + 4(l/32) + (j%4), j = 0..7 - the
// same row order in which a lane holds the k-step of a 32x32 C-layout accumulator.
// ds_read_b64_tr_b16: within a 16-lane group, destination lane d, element k is
// source lane 4k + d/4's element d%4; each source lane reads 4 columns of one row.
__device__ __forceinline__ bf16x8 tr_frag(const uint16_t* t, int r0, int c0, int s, int lane) {
  const int s16 = lane & 15;
  const int row = r0 + 16 * s + 4 * (lane >> 5) + (s16 >> 2);
  const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (s16 & 3);
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + toff(row, col)));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(t + toff(row + 8, col)));
  // a shuffle (not an element-wise rebuild) lets both loads land in one register quad
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Pack 8 fp32 (registers 8s..8s+7 of a C-layout accumulator) into a bf16 operand.
__device__ __forceinline__ bf16x8 pack8(const float* p) {
  u32x4 w;
  w[0] = pack_bf16x2(p[0], p[1]);
  w[1] = pack_bf16x2(p[2], p[3]);
  w[2] = pack_bf16x2(p[4], p[5]);
  w[3] = pack_bf16x2(p[6], p[7]);
  return as_bf16x8(w);
}

__device__ __forceinline__ u32x4 gld16(const void* base, int64_t elem) {
  return *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + elem);
}

// ---- attended keys ------------------------------------------------------------------------
// Attended key index a: list entry a / P, slot a % P; entries are the selected prior
// pages (all prior pages when dense) followed by the local pages. Positions of the
// local keys are linear in a: first_local * P + (a - local0).
struct Keys {
  const int32_t* table;
  const int32_t* sel;
  int n_sel, first_local, n_keys, local0, kv_end, log2p, n_entries;
  int64_t num_pages;

  // Physical page of entry e (bounds-checked), or -1.
  __device__ __forceinline__ int phys(int e) const {
    int lp;
    if (e < n_sel) {
      lp = sel ? sel[e] : e;
      if (sel && (lp < 0 || lp >= first_local)) return -1;
    } else {
      lp = first_local + (e - n_sel);
    }
    const int64_t ph = table[lp];
    return (ph >= 0 && ph < num_pages) ? static_cast<int>(ph) : -1;
  }
  __device__ __forceinline__ int logical(int e) const {
    return e < n_sel ? (sel ? sel[e] : e) : first_local + (e - n_sel);
  }
  // Last attended index visible to a query at position qpos (mask: a > klim).
  __device__ __forceinline__ int klim(int qpos) const {
    const int l = qpos - (first_local << log2p) + local0;
    return l < n_keys - 1 ? l : n_keys - 1;
  }
  // Does attended key a exist and lie before the end of the sequence?
  __device__ __forceinline__ bool in_seq(int a) const {
    return a < n_keys && (a < local0 || (first_local << log2p) + (a - local0) < kv_end);
  }
};

__device__ __forceinline__ Keys make_keys(const AttnArgs& a, int g) {
  Keys k;
  k.table = a.table + g * a.tstride;
  k.sel = a.sel ? a.sel + g * a.sel_stride : nullptr;
  k.n_sel = a.sel ? clamp_count(a.count, g, a.sel_stride, a.n_cand) : a.n_cand;
  k.first_local = a.first_local;
  k.n_entries = k.n_sel + a.n_local;
  k.n_keys = k.n_entries << a.pool.log2p;
  k.local0 = k.n_sel << a.pool.log2p;
  k.kv_end = a.t0 + a.n_q;
  k.log2p = a.pool.log2p;
  k.num_pages = a.pool.N;
  return k;
}

// Blocks of KB keys that queries up to position qmax_pos must visit.
__device__ __forceinline__ int n_blocks(const Keys& k, int qmax_pos) {
  const int last = k.klim(qmax_pos);
  return last < 0 ? 0 : last / KB + 1;
}

// ---- direct global -> LDS staging ---------------------------------------------------------
// global_load_lds_dwordx4 writes lane L's 16 bytes at a wave-uniform LDS base + 16 L.
// A [64 rows][128 bf16] swizzled tile (16 KiB) is filled by 16 such wave-instructions:
// wave w issues i = 0..3, covering LDS rows 16i + 4w .. +3; lane L fills physical
// chunk L%16 of row r = 16i + 4w + L/16, whose logical chunk is (L%16) ^ swz(r). With
// this row order swz(r) = 4(L/16) + w is the same for all four instructions of a lane,
// so one column offset serves them all.
// Rows that are not loaded keep their previous (finite) contents; every consumer
// masks them (P = 0), so stale values never reach a result.
__device__ __forceinline__ void lds_dma16(const uint16_t* gsrc, uint16_t* ldst) {
  __builtin_amdgcn_global_load_lds(gsrc, ldst, 16, 0, 0);
}
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0); }
// Global column (in elements) that lane L of wave w fetches for its row: 8 * logical chunk.
// The empty asm makes the value opaque at each use, so that the compiler recomputes the
// per-lane 64-bit addresses near the loads instead of hoisting (and spilling) them.
__device__ __forceinline__ int dma_col(int wave, int lane) {
  int c = 8 * ((lane & 15) ^ (((lane >> 4) << 2) | wave));
  asm volatile("" : "+v"(c));
  return c;
}

// Zero a [64][128] bf16 tile (once, before the first DMA into it).
__device__ __forceinline__ void zero_tile(uint16_t* t, int tid) {
#pragma unroll
  for (int i = 0; i < 4; ++i) sts16(t, (tid + 256 * i) * 8, u32x4{0u, 0u, 0u, 0u});
}

// Key blocks for the forward and dQ kernels, through the LDS page-id window.
struct KeyStream {
  const Keys& k;
  const int* spage;  // LDS page ids of entries [win, win + PCAP)
  int win;
  const uint16_t* kp;
  const uint16_t* vp;

  __device__ __forceinline__ void issue(int b, uint16_t* kt, uint16_t* vt, int wave, int lane) const {
    const int c8 = dma_col(wave, lane);
    const int a0 = b * KB;
    if (k.log2p >= 6) {
      // Pages of 64+ keys: the whole block lies in one page, so one (broadcast) page-id
      // read and a uniform page base serve all rows; only the sequence tail is per row.
      const int e = a0 >> k.log2p;
      const int ph = e < k.n_entries ? __builtin_amdgcn_readfirstlane(spage[e - win]) : -1;
      if (ph < 0) return;
      const int64_t base = (static_cast<int64_t>(ph) << k.log2p) * D;
      const int slot0 = a0 & ((1 << k.log2p) - 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r0 = 16 * i + 4 * wave;
        const int r = r0 + (lane >> 4);
        if (k.in_seq(a0 + r)) {
          const int off = (slot0 + r) * D + c8;
          lds_dma16(kp + base + off, kt + r0 * D);
          lds_dma16(vp + base + off, vt + r0 * D);
        }
      }
      return;
    }
    // Smaller pages: each row looks up its own page id (all four reads issued together).
    int ph[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int a = a0 + 16 * i + 4 * wave + (lane >> 4);
      const int e = a >> k.log2p;
      ph[i] = k.in_seq(a) ? spage[e - win] : -1;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r0 = 16 * i + 4 * wave;
      const int a = a0 + r0 + (lane >> 4);
      if (ph[i] >= 0) {
        const int64_t off = ((static_cast<int64_t>(ph[i]) << k.log2p) + (a & ((1 << k.log2p) - 1))) * D + c8;
        lds_dma16(kp + off, kt + r0 * D);
        lds_dma16(vp + off, vt + r0 * D);
      }
    }
  }
};

// Fill spage with the page ids of entries [win, win + PCAP).
__device__ __forceinline__ void fill_pages(const Keys& k, int* spage, int win, int tid) {
  const int end = min(k.n_entries, win + PCAP);
  for (int e = win + tid; e < end; e += 256) spage[e - win] = k.phys(e);
}

// Issue the loads of block b + 1 into (kn, vn), sliding the page-id window first when
// needed. The two K/V buffers are distinct __shared__ objects and every call site
// names them at compile time, so the compiler can see that a DMA into one buffer does
// not alias reads of the other and does not wait for it.
__device__ __forceinline__ void prefetch_next(KeyStream& ks, int* spage, const Keys& km, int b,
                                              int nblk, int tid, int wave, int lane,
                                              uint16_t* kn, uint16_t* vn) {
  if (b + 1 >= nblk) return;
  const int last_e = ((b + 1) * KB + KB - 1) >> km.log2p;
  if (last_e >= ks.win + PCAP) {  // uniform over the workgroup
    ks.win = ((b + 1) * KB) >> km.log2p;
    fill_pages(km, spage, ks.win, tid);
    // Retire every table load here: a load the compiler cannot prove consumed would
    // otherwise make it wait for all loads (the DMA included) at later register reuse.
    wait_dma();
    __syncthreads();
  }
  ks.issue(b + 1, kn, vn, wave, lane);
}

// Start a key stream: page window, zeroed tiles, block 0 loaded and visible.
__device__ __forceinline__ void start_stream(KeyStream& ks, int* spage, const Keys& km, int nblk,
                                             int tid, int wave, int lane, uint16_t* k0,
                                             uint16_t* v0, uint16_t* k1, uint16_t* v1) {
  fill_pages(km, spage, 0, tid);
  zero_tile(k0, tid);
  zero_tile(v0, tid);
  zero_tile(k1, tid);
  zero_tile(v1, tid);
  wait_dma();
  __syncthreads();
  if (nblk > 0) ks.issue(0, k0, v0, wave, lane);
  wait_dma();
  __syncthreads();
}

#define OOMB_KV_BUFFERS                                  \
  __shared__ __attribute__((aligned(16))) uint16_t s_k0[KB * D]; \
  __shared__ __attribute__((aligned(16))) uint16_t s_v0[KB * D]; \
  __shared__ __attribute__((aligned(16))) uint16_t s_k1[KB * D]; \
  __shared__ __attribute__((aligned(16))) uint16_t s_v1[KB * D]; \
  __shared__ int s_page[PCAP];

}  // namespace mf
}  // namespace oomb
