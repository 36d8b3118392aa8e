// Matrix-core paged chunk attention for gfx950 (bf16 inputs, head_dim 128):
// forward with online softmax, and the recomputing backward (dQ pass and a
// race-free dK/dV pass into the paged fp32 gradient pool).
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

// ---- key-block streaming shared by the forward and dQ kernels ---------------------------
// 256 threads stage one 64-key block: thread = (rows tid/16 + 16i, 16-byte chunk tid%16).
struct KeyStream {
  const Keys& k;
  const int* spage;  // LDS page ids of entries [win, win + PCAP)
  int win;
  const void* kp;
  const void* vp;
  u32x4 kr[4], vr[4];

  __device__ __forceinline__ void load(int b, int tid) {
    const int c = tid & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int a = b * KB + (tid >> 4) + 16 * i;
      u32x4 x = u32x4{0u, 0u, 0u, 0u}, y = x;
      if (k.in_seq(a)) {
        const int ph = spage[(a >> k.log2p) - win];
        if (ph >= 0) {
          const int64_t row = (static_cast<int64_t>(ph) << k.log2p) + (a & ((1 << k.log2p) - 1));
          x = gld16(kp, row * D + 8 * c);
          y = gld16(vp, row * D + 8 * c);
        }
      }
      kr[i] = x;
      vr[i] = y;
    }
  }
  __device__ __forceinline__ void store(uint16_t* kt, uint16_t* vt, int tid) const {
    const int c = tid & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 4) + 16 * i;
      sts16(kt, toff(r, 8 * c), kr[i]);
      sts16(vt, toff(r, 8 * c), vr[i]);
    }
  }
};

// Fill spage with the page ids of entries [win, win + PCAP).
__device__ __forceinline__ void fill_pages(const Keys& k, int* spage, int win, int tid) {
  const int end = min(k.n_entries, win + PCAP);
  for (int e = win + tid; e < end; e += 256) spage[e - win] = k.phys(e);
}

struct BlockSmem {
  uint16_t k[2][KB * D];
  uint16_t v[2][KB * D];
  int page[PCAP];
};

// Advance the key stream to block b + 1 (sliding the page-id window when needed).
__device__ __forceinline__ void prefetch_next(KeyStream& ks, BlockSmem& sm, const Keys& km,
                                              int b, int nblk, int tid) {
  if (b + 1 >= nblk) return;
  const int last_e = ((b + 1) * KB + KB - 1) >> km.log2p;
  if (last_e >= ks.win + PCAP) {  // uniform over the workgroup
    ks.win = ((b + 1) * KB) >> km.log2p;
    fill_pages(km, sm.page, ks.win, tid);
    __syncthreads();
  }
  ks.load(b + 1, tid);
}

// ============================================================================ forward
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_mfma_kernel(AttnArgs a) {
  __shared__ BlockSmem sm;
  constexpr int QT = 128;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h2 = lane >> 5, col = lane & 31;
  const int G = a.pool.Hq / a.pool.Hkv;
  const int n_qt = (a.n_q + QT - 1) / QT;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int hh = L % G, rest = L / G;
  const int qt = rest % n_qt, g = rest / n_qt;
  const int h = g * G + hh;
  const Keys km = make_keys(a, g);
  const int q0 = qt * QT;
  const int klim_tile = km.klim(a.t0 + q0);
  const int nblk = n_blocks(km, a.t0 + min(a.n_q, q0 + QT) - 1);
  const float c2 = a.scale * kLog2e;

  // This lane's query (column of S^T) and its Q fragments (B operand over d).
  const int i = q0 + wave * 32 + col;
  const int klim = km.klim(a.t0 + i);
  bf16x8 qf[8];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + h * a.q_hs + static_cast<int64_t>(i) * a.q_ts;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      qf[kk] = as_bf16x8(i < a.n_q ? *reinterpret_cast<const u32x4*>(qrow + 16 * kk + 8 * h2)
                                   : u32x4{0u, 0u, 0u, 0u});
  }

  f32x16 ot[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) ot[db] = f32x16{};
  float m_run = -__builtin_inff(), l_run = 0.0f;

  fill_pages(km, sm.page, 0, tid);
  __syncthreads();
  KeyStream ks{km, sm.page, 0, a.pool.k_pool, a.pool.v_pool};
  if (nblk > 0) {
    ks.load(0, tid);
    ks.store(sm.k[0], sm.v[0], tid);
  }
  __syncthreads();
  for (int b = 0; b < nblk; ++b) {
    const int buf = b & 1;
    prefetch_next(ks, sm, km, b, nblk, tid);
    const uint16_t* kt = sm.k[buf];
    const uint16_t* vt = sm.v[buf];

    // S^T = K Q^T for the block's two 32-key halves (raw dot products).
    f32x16 st[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      bf16x8 ka[8];  // all fragments first, so the MFMA chain does not wait per step
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) ka[kk] = row_frag(kt, 32 * sub, kk, lane);
      __builtin_amdgcn_sched_barrier(0);
      st[sub] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) st[sub] = mfma(ka[kk], qf[kk], st[sub]);
    }
    // Causal / tail mask, only in blocks that reach past the tile's first query.
    if (b * KB + KB - 1 > klim_tile) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (b * KB + 32 * sub + 8 * (r >> 2) + 4 * h2 + (r & 3) > klim) st[sub][r] = -__builtin_inff();
    }
    float mx = -__builtin_inff();
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, st[sub][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64)) * c2;
    // Lazy rescale: move the reference only when the maximum grew by more than 2^kTau.
    const bool grow = mx > m_run + kTau;
    if (__any(grow)) {
      const float alpha = grow ? fast_exp2(m_run - mx) : 1.0f;
      if (grow) m_run = mx;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) ot[db] *= alpha;
    }
    const float mref = m_run == -__builtin_inff() ? 0.0f : m_run;
    bf16x8 pb[2][2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          p[j] = fast_exp2(__builtin_fmaf(st[sub][8 * s + j], c2, -mref));
          l_run += p[j];
        }
        pb[sub][s] = pack8(p);
      }
    // O^T += V^T P^T, four transposed fragments in flight per step.
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8 va[4];
#pragma unroll
        for (int db = 0; db < 4; ++db) va[db] = tr_frag(vt, 32 * sub, 32 * db, s, lane);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < 4; ++db) ot[db] = mfma(va[db], pb[sub][s], ot[db]);
      }

    if (b + 1 < nblk) ks.store(sm.k[buf ^ 1], sm.v[buf ^ 1], tid);
    __syncthreads();
  }

  // Epilogue: O = O^T / l, LSE = (m + log2 l) ln 2.
  const float lt = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / lt;
  if (i < a.n_q) {
    uint16_t* orow = static_cast<uint16_t*>(a.o) + h * a.o_hs + static_cast<int64_t>(i) * a.o_ts;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int ga = 0; ga < 4; ++ga) {
        u32x2 w;
        w[0] = pack_bf16x2(ot[db][4 * ga + 0] * inv, ot[db][4 * ga + 1] * inv);
        w[1] = pack_bf16x2(ot[db][4 * ga + 2] * inv, ot[db][4 * ga + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * ga + 4 * h2) = w;
      }
    if (h2 == 0) a.lse[static_cast<int64_t>(h) * a.n_q + i] = (m_run + __log2f(lt)) * kLn2;
  }
}

// ============================================================================ dQ
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void dq_mfma_kernel(AttnArgs a) {
  __shared__ BlockSmem sm;
  constexpr int QT = 128;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h2 = lane >> 5, col = lane & 31;
  const int G = a.pool.Hq / a.pool.Hkv;
  const int n_qt = (a.n_q + QT - 1) / QT;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int hh = L % G, rest = L / G;
  const int qt = rest % n_qt, g = rest / n_qt;
  const int h = g * G + hh;
  const Keys km = make_keys(a, g);
  const int q0 = qt * QT;
  const int klim_tile = km.klim(a.t0 + q0);
  const int nblk = n_blocks(km, a.t0 + min(a.n_q, q0 + QT) - 1);
  const float c2 = a.scale * kLog2e;

  const int i = q0 + wave * 32 + col;
  const int klim = km.klim(a.t0 + i);
  bf16x8 qf[8], df[8];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + h * a.q_hs + static_cast<int64_t>(i) * a.q_ts;
    const uint16_t* drow = static_cast<const uint16_t*>(a.dout) + h * a.do_hs + static_cast<int64_t>(i) * a.do_ts;
    const bool ok = i < a.n_q;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      qf[kk] = as_bf16x8(ok ? *reinterpret_cast<const u32x4*>(qrow + 16 * kk + 8 * h2) : u32x4{0u, 0u, 0u, 0u});
      df[kk] = as_bf16x8(ok ? *reinterpret_cast<const u32x4*>(drow + 16 * kk + 8 * h2) : u32x4{0u, 0u, 0u, 0u});
    }
  }
  const int64_t rid = static_cast<int64_t>(h) * a.n_q + i;
  const float lse2 = i < a.n_q ? a.lse_in[rid] * kLog2e : __builtin_inff();
  const float delta = i < a.n_q ? a.delta[rid] : 0.0f;

  f32x16 dqt[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) dqt[db] = f32x16{};

  fill_pages(km, sm.page, 0, tid);
  __syncthreads();
  KeyStream ks{km, sm.page, 0, a.pool.k_pool, a.pool.v_pool};
  if (nblk > 0) {
    ks.load(0, tid);
    ks.store(sm.k[0], sm.v[0], tid);
  }
  __syncthreads();
  for (int b = 0; b < nblk; ++b) {
    const int buf = b & 1;
    prefetch_next(ks, sm, km, b, nblk, tid);
    const uint16_t* kt = sm.k[buf];
    const uint16_t* vt = sm.v[buf];
    const bool mask = b * KB + KB - 1 > klim_tile;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      f32x16 st = f32x16{}, dpt = f32x16{};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        st = mfma(row_frag(kt, 32 * sub, kk, lane), qf[kk], st);
        dpt = mfma(row_frag(vt, 32 * sub, kk, lane), df[kk], dpt);
      }
      bf16x8 dsb[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        float ds[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = 8 * s + j;
          float p = fast_exp2(__builtin_fmaf(st[r], c2, -lse2));
          if (mask && b * KB + 32 * sub + 8 * (r >> 2) + 4 * h2 + (r & 3) > klim) p = 0.0f;
          ds[j] = p * (dpt[r] - delta);
        }
        dsb[s] = pack8(ds);
      }
      // dQ^T += K^T dS^T.
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8 ta[4];
#pragma unroll
        for (int db = 0; db < 4; ++db) ta[db] = tr_frag(kt, 32 * sub, 32 * db, s, lane);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int db = 0; db < 4; ++db) dqt[db] = mfma(ta[db], dsb[s], dqt[db]);
      }
    }
    if (b + 1 < nblk) ks.store(sm.k[buf ^ 1], sm.v[buf ^ 1], tid);
    __syncthreads();
  }

  if (i < a.n_q) {
    float* drow = a.dq + h * a.dq_hs + static_cast<int64_t>(i) * a.dq_ts;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int ga = 0; ga < 4; ++ga) {
        f32x4 w;
#pragma unroll
        for (int b2 = 0; b2 < 4; ++b2) w[b2] = dqt[db][4 * ga + b2] * a.scale;
        *reinterpret_cast<f32x4*>(drow + 32 * db + 8 * ga + 4 * h2) = w;
      }
  }
}

// ============================================================================ dK / dV
struct DkvSmem {
  uint16_t q[2][QTB * D];
  uint16_t d[2][QTB * D];
  float lse2[2][QTB];
  float delta[2][QTB];
  int64_t grow[KPW];  // output row of each key (gradient pool row, or -1 to skip)
};

// Grid: Hkv * (key blocks of 128) * n_split. With n_split > 1, split s writes its
// partial dK/dV rows to part[((s * Hkv + g) * part_keys + key) * 2D + {0: dK, D: dV}].
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void dkdv_mfma_kernel(AttnArgs a, int n_split, float* part, int part_keys) {
  __shared__ DkvSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h2 = lane >> 5, col = lane & 31;
  const int G = a.pool.Hq / a.pool.Hkv;
  const int nkb = (a.max_att_pages * a.pool.P + KPW - 1) / KPW;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int split = L % n_split, kb = (L / n_split) % nkb, g = L / (n_split * nkb);
  const Keys km = make_keys(a, g);
  const int k0 = kb * KPW;
  if (k0 >= km.n_keys) return;  // uniform: block past this head's attended keys
  const float c2 = a.scale * kLog2e;

  // This lane's key (column of S = Q K^T) and its K / V fragments (B operands over d).
  const int kidx = k0 + 32 * wave + col;
  int64_t krow = -1;
  int kpos = 0x7FFFFFFF;
  if (km.in_seq(kidx)) {
    const int e = kidx >> km.log2p;
    const int ph = km.phys(e);
    if (ph >= 0) {
      const int slot = kidx & ((1 << km.log2p) - 1);
      krow = (static_cast<int64_t>(ph) << km.log2p) + slot;
      kpos = (km.logical(e) << km.log2p) + slot;
    }
  }
  if (h2 == 0) {
    int64_t out = -1;
    if (krow >= 0) {
      if (n_split > 1) {
        out = kidx;  // partial row index
      } else {
        const int64_t gp = a.gtable[g * a.gtstride + (kpos >> km.log2p)];
        if (gp >= 0 && gp < a.pool.Ng) out = (gp << km.log2p) + (kpos & ((1 << km.log2p) - 1));
      }
    }
    sm.grow[32 * wave + col] = out;
  }
  bf16x8 kf[8], vf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const u32x4 z = u32x4{0u, 0u, 0u, 0u};
    kf[kk] = as_bf16x8(krow >= 0 ? gld16(a.pool.k_pool, krow * D + 16 * kk + 8 * h2) : z);
    vf[kk] = as_bf16x8(krow >= 0 ? gld16(a.pool.v_pool, krow * D + 16 * kk + 8 * h2) : z);
  }

  // Query tiles that can see some key of this block: every head of the group, from
  // the first query at or after the block's first key; cut into n_split parts.
  const int n_qt = (a.n_q + QTB - 1) / QTB;
  int qt0 = 0;
  if (!km.in_seq(k0)) {
    qt0 = n_qt;
  } else if (k0 >= km.local0) {
    const int first_pos = (km.first_local << km.log2p) + (k0 - km.local0);
    qt0 = first_pos > a.t0 ? (first_pos - a.t0) / QTB : 0;
  }
  const int tph = n_qt - qt0;
  const int n_tiles = G * tph;
  const int u_begin = static_cast<int>((static_cast<int64_t>(n_tiles) * split) / n_split);
  const int u_end = static_cast<int>((static_cast<int64_t>(n_tiles) * (split + 1)) / n_split);

  f32x16 dv[4], dk[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    dv[nb] = f32x16{};
    dk[nb] = f32x16{};
  }

  // Staging: 64 rows x 16 chunks per tensor; thread rows tid/16 + 16i, chunk tid%16.
  u32x4 rq[4], rd[4];
  float r_lse2 = 0.0f, r_delta = 0.0f;
  auto load_tile = [&](int u) {
    const int hq = g * G + u / tph, q0 = (qt0 + u % tph) * QTB;
    const int c = tid & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int qi = q0 + (tid >> 4) + 16 * i;
      u32x4 x = u32x4{0u, 0u, 0u, 0u}, y = x;
      if (qi < a.n_q) {
        x = gld16(a.q, hq * a.q_hs + static_cast<int64_t>(qi) * a.q_ts + 8 * c);
        y = gld16(a.dout, hq * a.do_hs + static_cast<int64_t>(qi) * a.do_ts + 8 * c);
      }
      rq[i] = x;
      rd[i] = y;
    }
    if (tid < QTB) {
      // raw loads only: any arithmetic on them here would wait for the whole prefetch
      const int qi = q0 + tid;
      const int64_t rid = static_cast<int64_t>(hq) * a.n_q + qi;
      r_lse2 = qi < a.n_q ? a.lse_in[rid] : __builtin_inff();
      r_delta = qi < a.n_q ? a.delta[rid] : 0.0f;
    }
  };
  auto store_tile = [&](int buf) {
    const int c = tid & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = (tid >> 4) + 16 * i;
      sts16(sm.q[buf], toff(r, 8 * c), rq[i]);
      sts16(sm.d[buf], toff(r, 8 * c), rd[i]);
    }
    if (tid < QTB) {
      sm.lse2[buf][tid] = r_lse2 * kLog2e;
      sm.delta[buf][tid] = r_delta;
    }
  };

  if (u_begin < u_end) {
    load_tile(u_begin);
    store_tile(0);
  }
  __syncthreads();
  for (int u = u_begin; u < u_end; ++u) {
    const int buf = (u - u_begin) & 1;
    if (u + 1 < u_end) load_tile(u + 1);
    const int q0 = (qt0 + u % tph) * QTB;
    const uint16_t* qt = sm.q[buf];
    const uint16_t* dt = sm.d[buf];
    // Some (key, query) pair of this tile is hidden for this lane's key?
    const bool wmask = __any(kpos > a.t0 + q0);
#pragma unroll
    for (int us = 0; us < QTB / 32; ++us) {
      // Phase 1: all row fragments of Q and dO in registers, then S = Q K^T and
      // dP = dO V^T (two independent chains) for 32 queries x this wave's 32 keys.
      bf16x8 qa[8], da[8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        qa[kk] = row_frag(qt, 32 * us, kk, lane);
        da[kk] = row_frag(dt, 32 * us, kk, lane);
      }
      __builtin_amdgcn_sched_barrier(0);
      f32x16 s_acc = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        s_acc = mfma(qa[kk], kf[kk], s_acc);
        dp = mfma(da[kk], vf[kk], dp);
      }
      // Phase 2: transposed fragments of dO and Q for dV / dK, issued before the
      // softmax arithmetic so that their latency hides behind it.
      bf16x8 tdo[2][4], tq[2][4];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          tdo[s][nb] = tr_frag(dt, 32 * us, 32 * nb, s, lane);
          tq[s][nb] = tr_frag(qt, 32 * us, 32 * nb, s, lane);
        }
      __builtin_amdgcn_sched_barrier(0);
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        // query rows rA + 8(j/4) + (j%4), j = 0..7, rA = 32us + 16s + 4h2
        const int rA = 32 * us + 16 * s + 4 * h2;
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(&sm.lse2[buf][rA]);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(&sm.lse2[buf][rA + 8]);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(&sm.delta[buf][rA]);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(&sm.delta[buf][rA + 8]);
        float p[8], ds[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = 8 * s + j;
          const float lse_r = j < 4 ? l0[j] : l1[j - 4];
          const float del_r = j < 4 ? d0[j] : d1[j - 4];
          float pv = fast_exp2(__builtin_fmaf(s_acc[r], c2, -lse_r));
          if (wmask && kpos > a.t0 + q0 + rA + 8 * (j >> 2) + (j & 3)) pv = 0.0f;
          p[j] = pv;
          ds[j] = pv * (dp[r] - del_r);
        }
        pb[s] = pack8(p);
        dsb[s] = pack8(ds);
      }
      __builtin_amdgcn_sched_barrier(0);
      // Phase 3: dV += P^T dO, dK += dS^T Q (the scale is applied once, at the end).
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          dv[nb] = mfma(pb[s], tdo[s][nb], dv[nb]);
          dk[nb] = mfma(dsb[s], tq[s][nb], dk[nb]);
        }
    }
    if (u + 1 < u_end) store_tile(buf ^ 1);
    __syncthreads();
  }

  // Write out: register r holds key row m = 8(r/4) + 4h2 + r%4 of this wave, column
  // 32nb + col of d.
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = 8 * (r >> 2) + 4 * h2 + (r & 3);
    const int64_t out = sm.grow[32 * wave + m];
    if (out < 0) continue;
    if (n_split == 1) {
      float* dkr = a.pool.dk_pool + out * D;
      float* dvr = a.pool.dv_pool + out * D;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        dkr[32 * nb + col] += dk[nb][r] * a.scale;
        dvr[32 * nb + col] += dv[nb][r];
      }
    } else {
      float* pk = part + ((static_cast<int64_t>(split) * a.pool.Hkv + g) * part_keys + out) * (2 * D);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        pk[32 * nb + col] = dk[nb][r] * a.scale;
        pk[D + 32 * nb + col] = dv[nb][r];
      }
    }
  }
}

// Adds the split partials of every attended key row, in split order, into the
// gradient pool. One wavefront per (key, KV head); lanes over d.
__global__ __launch_bounds__(256) void dkdv_merge_kernel(AttnArgs a, int n_split, const float* part,
                                                         int part_keys) {
  const int lane = threadIdx.x & 63;
  const int kidx = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int g = blockIdx.y;
  const Keys km = make_keys(a, g);
  if (kidx >= part_keys || !km.in_seq(kidx)) return;
  const int e = kidx >> km.log2p;
  if (km.phys(e) < 0) return;
  const int slot = kidx & ((1 << km.log2p) - 1);
  const int64_t gp = a.gtable[g * a.gtstride + km.logical(e)];
  if (gp < 0 || gp >= a.pool.Ng) return;
  const int64_t grow = (gp << km.log2p) + slot;
  float sk0 = 0.0f, sk1 = 0.0f, sv0 = 0.0f, sv1 = 0.0f;
  for (int s = 0; s < n_split; ++s) {
    const float* pk = part + ((static_cast<int64_t>(s) * a.pool.Hkv + g) * part_keys + kidx) * (2 * D);
    sk0 += pk[lane];
    sk1 += pk[64 + lane];
    sv0 += pk[D + lane];
    sv1 += pk[D + 64 + lane];
  }
  float* dkr = a.pool.dk_pool + grow * D;
  float* dvr = a.pool.dv_pool + grow * D;
  dkr[lane] += sk0;
  dkr[64 + lane] += sk1;
  dvr[lane] += sv0;
  dvr[64 + lane] += sv1;
}

}  // namespace mf

hipError_t launch_fwd_mfma(const AttnArgs& a, hipStream_t s) {
  const int n_qt = (a.n_q + 127) / 128;
  OOMB_LAUNCH("fwd_mfma", mf::fwd_mfma_kernel, dim3(a.pool.Hq * n_qt), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Query-stream splits of the dK/dV pass: double until the grid has two workgroups
// per CU of a 256-CU MI355X (at most 4 splits). A fixed CU count keeps the choice,
// and so the result bits and the workspace size, independent of the device queried.
int dkdv_splits(const AttnArgs& a) {
  const int nkb = (a.max_att_pages * a.pool.P + mf::KPW - 1) / mf::KPW;
  const int blocks = a.pool.Hkv * nkb;
  int ns = 1;
  while (ns < 4 && blocks * ns < 2 * 256) ns *= 2;
  return ns;
}

size_t dkdv_partial_bytes(const AttnArgs& a, int n_split) {
  if (n_split <= 1) return 0;
  const size_t keys = static_cast<size_t>(a.max_att_pages) * a.pool.P;
  return static_cast<size_t>(n_split) * a.pool.Hkv * keys * 2 * mf::D * sizeof(float);
}

hipError_t launch_bwd_mfma(const AttnArgs& a, int n_split, float* part, hipStream_t s) {
  hipError_t err = launch_delta(a, s);
  if (err != hipSuccess) return err;
  const int n_qt = (a.n_q + 127) / 128;
  OOMB_LAUNCH("dq_mfma", mf::dq_mfma_kernel, dim3(a.pool.Hq * n_qt), dim3(256), 0, s, a);
  const int nkb = (a.max_att_pages * a.pool.P + mf::KPW - 1) / mf::KPW;
  const int part_keys = a.max_att_pages * a.pool.P;
  OOMB_LAUNCH("dkdv_mfma", mf::dkdv_mfma_kernel, dim3(a.pool.Hkv * nkb * n_split), dim3(256), 0, s,
              a, n_split, part, part_keys);
  if (n_split > 1) {
    dim3 grid((part_keys + 3) / 4, a.pool.Hkv);
    OOMB_LAUNCH("dkdv_merge", mf::dkdv_merge_kernel, grid, dim3(256), 0, s, a, n_split, part,
                part_keys);
  }
  return hipGetLastError();
}

}  // namespace oomb
