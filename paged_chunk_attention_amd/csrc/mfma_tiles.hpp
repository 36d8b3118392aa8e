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
//  * The dK/dV pass owns 128 keys per workgroup (32 per pair of wavefronts: one holds
//    K and dV, the other V and dK, and P passes between them through LDS), streams the
//    query tiles of all heads of its KV group through triple-buffered LDS, and does one
//    read-modify-write of its gradient rows. When the work would not spread evenly
//    over the CUs, the query stream is split across workgroups; each split writes fp32
//    partials and a merge kernel adds them in split order. No two workgroups ever
//    write the same gradient row: no atomics, no races, and bit-reproducible results.
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
constexpr int DS_REC = 4 * 64 * 8;  // bf16 of spilled dS per (64-query tile, 32 keys)

// Whether attention row `row` (= h * n_q + i) belongs to a query tile (of `tileq`
// queries) that a split plan cut into key ranges: its tile index in the KV head's
// longest-first order is at least `whole`.
__device__ __forceinline__ bool row_was_split(const AttnArgs& a, int64_t row, int tileq, int whole) {
  if (whole <= 0) return true;
  const int G = a.pool.Hq / a.pool.Hkv;
  const int h = static_cast<int>(row / a.n_q), i = static_cast<int>(row % a.n_q);
  const int n_qt = (a.n_q + tileq - 1) / tileq;
  return (n_qt - 1 - i / tileq) * G + h % G >= whole;
}

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// max(x[l], x[l ^ 32]) in every lane l, by one v_permlane32_swap (no LDS traffic).
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

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

// Per-lane element offsets of every fragment of a [rows][128] tile: row fragments of k-step
// kk (rows r0 + 32j share them, the swizzle repeating every 16 rows) and the two halves of
// the transposed fragment of column block db (rows r0 + 16j share them). Keeping these
// 16 values, rather than one address per fragment per buffer, keeps register use flat
// however many LDS buffers a kernel reads; opaque() makes the compiler re-add the buffer
// base at each use instead of keeping one address register per buffer and fragment.
// Kernels apply it to their one copy in place (a copy made opaque costs 16 moves per use).
struct FragOffsets {
  int rf[8];  // row fragment, k-step kk
  int tr[8];  // transposed fragment, column block db: [2 db] rows +0, [2 db + 1] rows +8
  __device__ __forceinline__ void init(int lane) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) rf[kk] = toff(lane & 31, 16 * kk + 8 * (lane >> 5));
    const int s16 = lane & 15;
    const int row = 4 * (lane >> 5) + (s16 >> 2);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int col = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (s16 & 3);
      tr[2 * db] = toff(row, col);
      tr[2 * db + 1] = toff(row + 8, col);
    }
  }
  __device__ __forceinline__ void opaque() {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      asm volatile("" : "+v"(rf[i]));
      asm volatile("" : "+v"(tr[i]));
    }
  }
};
// row_frag(t, r0, kk, lane) for r0 a multiple of 16 (of 32 for the swizzle to repeat:
// swz depends on r % 16 only, so any multiple of 16 works).
__device__ __forceinline__ bf16x8 row_frag_at(const uint16_t* t, int r0, const FragOffsets& o, int kk) {
  return as_bf16x8(lds16(t + r0 * D, o.rf[kk]));
}
// tr_frag(t, r0, 32 db, s, lane) for r0 a multiple of 16.
__device__ __forceinline__ bf16x8 tr_frag_at(const uint16_t* t, int r0, int s, const FragOffsets& o, int db) {
  const uint16_t* b = t + (r0 + 16 * s) * D;
  const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b + o.tr[2 * db]));
  const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(b + o.tr[2 * db + 1]));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
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
// pages (when dense, the prior pages from prior0 on) followed by the local pages.
// Positions of the local keys are linear in a: first_local * P + (a - local0); when
// dense, so are all of them (prior0 * P + a). With a window W (dense calls only) a
// query at position p sees the keys with p - W < position <= p.
struct Keys {
  const int32_t* table;
  const int32_t* sel;
  int n_sel, prior0, first_local, n_keys, local0, kv_end, log2p, n_entries, window;
  int64_t num_pages;

  // Physical page of entry e (bounds-checked), or -1.
  __device__ __forceinline__ int phys(int e) const {
    int lp;
    if (e < n_sel) {
      lp = sel ? sel[e] : prior0 + e;
      if (sel && (lp < 0 || lp >= first_local)) return -1;
    } else {
      lp = first_local + (e - n_sel);
    }
    const int64_t ph = table[lp];
    return (ph >= 0 && ph < num_pages) ? static_cast<int>(ph) : -1;
  }
  __device__ __forceinline__ int logical(int e) const {
    return e < n_sel ? (sel ? sel[e] : prior0 + e) : first_local + (e - n_sel);
  }
  // Last attended index visible to a query at position qpos (mask: a > klim).
  __device__ __forceinline__ int klim(int qpos) const {
    const int l = qpos - (first_local << log2p) + local0;
    return l < n_keys - 1 ? l : n_keys - 1;
  }
  // First attended index visible to a query at position qpos (mask: a < klo); may be
  // negative, and is far below every index without a window.
  __device__ __forceinline__ int klo(int qpos) const {
    return window > 0 ? qpos - window + 1 - (prior0 << log2p) : -(1 << 30);
  }
  // Position of attended index a (dense calls: every key; else local keys only).
  __device__ __forceinline__ int pos_linear(int a) const {
    return (first_local << log2p) + (a - local0);
  }
  // Does attended key a exist and lie before the end of the sequence? (Bitwise, so that
  // per-lane uses compile to compares and selects, not branches.)
  __device__ __forceinline__ bool in_seq(int a) const {
    return (a < n_keys) & ((a < local0) | ((first_local << log2p) + (a - local0) < kv_end));
  }
};

__device__ __forceinline__ Keys make_keys(const AttnArgs& a, int g) {
  Keys k;
  k.table = a.table + g * a.tstride;
  k.sel = a.sel ? a.sel + g * a.sel_stride : nullptr;
  k.n_sel = a.sel ? clamp_count(a.count, g, a.sel_stride, a.n_cand) : a.n_cand;
  k.prior0 = a.prior0;
  k.window = a.window;
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
// First block a query at position qpos (or any later one) sees.
__device__ __forceinline__ int first_block(const Keys& k, int qpos) {
  const int lo = k.klo(qpos);
  return lo > 0 ? lo / KB : 0;
}

// ---- direct global -> LDS staging ---------------------------------------------------------
// global_load_lds_dwordx4 writes lane L's 16 bytes at a wave-uniform LDS base + 16 L.
// A [64 rows][128 bf16] swizzled tile (16 KiB) is filled by 16 such wave-instructions:
// wave w issues i = 0..3, covering LDS rows 16i + 4w .. +3; lane L fills physical
// chunk L%16 of row r = 16i + 4w + L/16, whose logical chunk is (L%16) ^ swz(r). With
// this row order swz(r) = 4(L/16) + w is the same for all four instructions of a lane,
// so one column offset serves them all.
//
// The instruction is issued from inline assembly rather than through the compiler's
// builtin. The compiler models the builtin as a flat access that may touch LDS, and while
// one is outstanding it waits for every pending LDS read (lgkmcnt(0)) wherever a single
// fragment is needed; issued from assembly, the LDS reads keep their exact in-order
// counts. The compiler then does not know of the DMA at all, which is sound because every
// caller waits for its DMAs explicitly (vmcnt, then a barrier) before anything reads the
// buffer, and no code touches a buffer while it is being filled. The compiler's own
// vmcnt waits stay correct: loads retire in issue order, so untracked DMAs can only make
// them wait longer. M0 (the LDS base) is an input operand, so the compiler knows it is
// set; the nop is the one wait state an LDS DMA needs after an M0 write. (Measured: 1-2%
// faster than the builtin in the dQ and dK/dV passes.)
__device__ __forceinline__ void lds_dma16(const uint16_t* gsrc, uint16_t* ldst) {
  const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) uint16_t*)ldst));
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "{m0}"(base));
}
// As lds_dma16, in the instruction's scalar-base form: a wave-uniform 64-bit base
// in scalar registers plus a per-lane 32-bit byte offset. A wave whose rows share one base
// then needs no per-lane 64-bit address arithmetic (vector ALU work that the forward's
// softmax phases compete for). gbase must be the same in every lane of the wave: the
// operand is bound to scalar registers, so a per-lane value would silently be read from
// one lane. Every caller derives it from wave-uniform indices and readfirstlane'd ids.
__device__ __forceinline__ void lds_dma16_s(const uint16_t* gbase, uint32_t off_bytes, uint16_t* ldst) {
  const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) uint16_t*)ldst));
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off_bytes), "s"(gbase), "{m0}"(base));
}
__device__ __forceinline__ void wait_dma() { __builtin_amdgcn_s_waitcnt(0); }

// Workgroup barrier without the release/acquire fences of __syncthreads(). Those fences
// make the compiler wait for every outstanding global->LDS DMA of the wave, which would
// defeat prefetching several phases ahead. Callers order the LDS data themselves: DMA
// data by explicit vmcnt waits before the barrier, and a wave's own LDS reads are all
// consumed (so complete) before it reaches the barrier. The empty asm statements keep
// the compiler from moving memory accesses across it.
__device__ __forceinline__ void phase_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until at most N vector-memory operations of this wave are outstanding (they
// complete in issue order), leaving the LDS and export counters alone.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Global column (in elements) that lane L of wave w fetches when a DMA instruction of the
// wave fills four rows r with swz(r) = 4 (L/16) + w: 8 * the logical chunk of its slot.
// The empty asm makes the value opaque at each use, so that the compiler recomputes the
// per-lane 64-bit addresses near the loads instead of hoisting (and spilling) them.
__device__ __forceinline__ int dma_col(int wave, int lane) {
  int c = 8 * ((lane & 15) ^ (((lane >> 4) << 2) | wave));
  asm volatile("" : "+v"(c));
  return c;
}

// Zero a [ROWS][128] bf16 tile with NT threads (once, before the first DMA into it).
template <int ROWS, int NT>
__device__ __forceinline__ void zero_tile(uint16_t* t, int tid) {
#pragma unroll
  for (int c = tid; c < ROWS * 16; c += NT) sts16(t, c * 8, u32x4{0u, 0u, 0u, 0u});
}

// Fill spage with the page ids of entries [win, win + CAP), NT threads.
template <int NT, int CAP = PCAP>
__device__ __forceinline__ void fill_pages(const Keys& k, int* spage, int win, int tid) {
  const int end = min(k.n_entries, win + CAP);
  for (int e = win + tid; e < end; e += NT) spage[e - win] = k.phys(e);
}

// Four zero rows of keys in global memory: the source of every staged row that is not
// an attended key (lane offsets stay below 4 rows). One copy per code object.
static __device__ __attribute__((aligned(16))) uint16_t g_zero_rows[4 * D] = {};

// Direct staging of a stage of ROWS attended keys (K and V rows) by NW wavefronts.
// Instruction i of wave w fills LDS rows r0 = 4 (NW i + w) .. r0 + 3. Those four rows are
// 4-aligned, so they lie in one page (pages hold >= 16 tokens): one broadcast page-id read
// gives a uniform page base, and lane L adds a fixed offset, row L/16 of the four plus
// the logical column whose 16 bytes land in its physical slot. With NW a multiple of 4,
// swz(r) = 4 (L/16) + (w % 4) for every instruction, so that offset is one register.
template <int ROWS, int NW, int CAP = PCAP>
struct KeyStage {
  static_assert(NW % 4 == 0 && ROWS % (4 * NW) == 0, "rows per wave must tile the stage");
  static constexpr int NI = ROWS / (4 * NW);
  const Keys& k;
  const int* spage;  // LDS page ids of entries [win, win + CAP)
  int win;
  int lane_off;      // (L/16) D + 8 ((L%16) ^ swz)

  __device__ static int lane_offset(int wave, int lane) {
    return (lane >> 4) * D + 8 * ((lane & 15) ^ (((lane >> 4) << 2) | (wave & 3)));
  }

  // With pages of at least ROWS tokens every stage (ROWS-aligned) lies in one page: one
  // page id, one validity test and one base then serve all NI instructions. A wave issues
  // its instructions one at a time, so this per-stage work (about 30 scalar instructions
  // per DMA instruction otherwise) is time the wave's softmax waits behind. (Stage sizes
  // other than 64, 128 and 256 rows always take the per-instruction path.)
  static constexpr int LOG2_ROWS = ROWS == 64 ? 6 : ROWS == 128 ? 7 : ROWS == 256 ? 8 : 30;
  __device__ __forceinline__ bool one_page() const { return k.log2p >= LOG2_ROWS; }

  // DMA the rows of stage st (attended keys st*ROWS ..) of one pool (K or V) into t.
  // Every wave issues exactly NI DMA instructions with all lanes active, whatever the
  // rows: a lane whose row does not exist, lies past the end of the sequence or has an
  // invalid page copies a zero row instead (such rows are masked; zeros keep them
  // finite, since a masked P of 0 still multiplies them). A fixed count per call lets
  // the caller wait for all but its most recent batches with vmcnt(n). Split in two so
  // that the page-id reads (LDS) can be issued well before the DMA needs them.
  __device__ __forceinline__ void read_pages(int st, int wave, int (&ph)[NI]) const {
    if (one_page()) {  // uniform; dma_fixed then reads ph[0] only
      const int e = min((st * ROWS) >> k.log2p, k.n_entries - 1) - win;
      ph[0] = spage[max(0, min(e, CAP - 1))];
      return;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      // branch-free: the read index is clamped into the window; for rows past the
      // attended keys the id is read but never used (in_seq fails for them)
      const int a = st * ROWS + 4 * (NW * i + wave);
      const int e = min(a >> k.log2p, k.n_entries - 1) - win;
      ph[i] = spage[max(0, min(e, CAP - 1))];
    }
  }
  __device__ __forceinline__ void dma_fixed(int st, const uint16_t* pool, uint16_t* t, int wave,
                                            int lane, const int (&ph)[NI]) const {
    const uint32_t lob = 2u * static_cast<uint32_t>(lane_off);
    if (one_page()) {
      const int a0 = st * ROWS;
      const int p = __builtin_amdgcn_readfirstlane(ph[0]);
      const uint16_t* base =
          pool + ((static_cast<int64_t>(p) << k.log2p) + (a0 & ((1 << k.log2p) - 1))) * D;
      // The rows of the sequence are a prefix of the attended keys (in_seq(x) implies
      // in_seq(y) for y < x), so the whole stage exists exactly when its last row does:
      // then every instruction takes the uniform base. Otherwise (the sequence's last
      // stage, an invalid page) each lane picks its row or a zero row.
      if ((p >= 0) & k.in_seq(a0 + ROWS - 1)) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int r0 = 4 * (NW * i + wave);
          lds_dma16_s(base + r0 * D, lob, t + r0 * D);
        }
      } else {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const int r0 = 4 * (NW * i + wave);
          int lo = lane_off, row = lane >> 4;
          asm volatile("" : "+v"(lo), "+v"(row));  // keep the per-lane work in this branch
          const bool ok = (p >= 0) & k.in_seq(a0 + r0 + row);
          lds_dma16((ok ? base + r0 * D : g_zero_rows) + lo, t + r0 * D);
        }
      }
      return;
    }
    // Smaller pages: each instruction's four rows (4-aligned) still share a page.
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r0 = 4 * (NW * i + wave);
      const int a = st * ROWS + r0;
      const int p = __builtin_amdgcn_readfirstlane(ph[i]);
      const int64_t base = ((static_cast<int64_t>(p) << k.log2p) + (a & ((1 << k.log2p) - 1))) * D;
      // Rows a .. a + 3 all exist exactly when row a + 3 does (the prefix rule above).
      if ((p >= 0) & k.in_seq(a + 3)) {
        lds_dma16_s(pool + base, lob, t + r0 * D);
      } else {
        int lo = lane_off, row = lane >> 4;
        asm volatile("" : "+v"(lo), "+v"(row));  // keep the per-lane work in this branch
        const bool ok = (p >= 0) & k.in_seq(a + row);
        lds_dma16((ok ? pool + base : g_zero_rows) + lo, t + r0 * D);
      }
    }
  }
  __device__ __forceinline__ void issue_fixed(int st, const uint16_t* pool, uint16_t* t, int wave,
                                              int lane) const {
    int ph[NI];
    read_pages(st, wave, ph);
    dma_fixed(st, pool, t, wave, lane, ph);
  }
};

}  // namespace mf
}  // namespace oomb
