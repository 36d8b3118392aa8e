// Matrix-core paged chunk attention for gfx950 (bf16 inputs, head_dim 128):
// forward with online softmax, and the recomputing backward (dQ pass and a
// race-free dK/dV pass into the paged fp32 gradient pool).
//
// Method (gist.science explainer of OOMB): 2.A chunk-recurrent training with
// recomputation (the backward recomputes P from the saved log-sum-exp); 2.B paged
// K/V and paged K/V gradients, accumulated in place; 2.D page-level top-k sparsity
// (the attended page list is the selected pages plus the chunk's own pages).
//
// Design (all tiles are v_mfma_f32_32x32x16_bf16, 64-lane wavefronts):
//  * Keys stream through LDS in blocks of 64, gathered row by row through the page
//    table (a 128-token page is two contiguous 16 KiB blocks per tensor).
//  * Forward and dQ compute S^T = K Q^T so that every lane owns one query column:
//    row max, row sum, LSE and Delta are per-lane scalars, and the C layout of S^T
//    feeds the next product directly as its B operand (P^T or dS^T), with the keys
//    permuted inside each 16-key step. The other operand (V^T or K^T) is staged in
//    LDS transposed in exactly that permuted key order, so every fragment is one
//    16-byte LDS read.
//  * The dK/dV pass owns 64 keys per workgroup (32 per wavefront, two wavefronts
//    splitting the query stream); it computes S = Q K^T so lanes own key columns,
//    accumulates dV and dK in C layout [key][d], merges the two query streams
//    in LDS and does one read-modify-write of its rows of the gradient pool. No
//    other workgroup touches those rows, so there are no atomics and no races.
//  * Workgroup ids are remapped so that each XCD works on one contiguous range
//    (one KV head's queries and pages share that XCD's L2).
#include "device_common.hpp"
#include "launch.hpp"

namespace oomb {
namespace mf {

constexpr int D = 128;
constexpr int KB = 64;      // keys per block
constexpr int KROW = 136;   // row-major tile row stride in elements (256 B + 16 B pad)

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// v_exp_f32: 2^x, exact 0 for -inf.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ u32x4 lds16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Position (within a 16-key group) at which key k is stored in a transposed tile:
// bits 2 and 3 swapped. A lane of half h (lanes 0-31 / 32-63) holds, for k-step s,
// the S^T rows 16s + 8(j/4) + 4h + (j%4), j = 0..7, i.e. positions 16s + 8h + j.
__device__ __forceinline__ int quad_pos(int kq) {  // key quad -> position quad
  return (kq & ~3) | ((kq & 1) << 1) | ((kq >> 1) & 1);
}

// XOR swizzles of the 16-byte units of transposed rows (conflict-free fragment reads).
__device__ __forceinline__ int sw8(int d) { return (d ^ (d >> 3)) & 7; }  // 64-key rows
__device__ __forceinline__ int sw4(int d) { return (d >> 2) & 3; }        // 32-query rows

// Element offset of (row d, position p) in a transposed tile with 64 positions per row.
__device__ __forceinline__ int t64(int d, int p) {
  return d * 64 + ((((p >> 3) ^ sw8(d))) << 3) + (p & 7);
}
// ... with 32 positions per row.
__device__ __forceinline__ int t32(int d, int p) {
  return d * 32 + ((((p >> 3) ^ sw4(d))) << 3) + (p & 7);
}

// Transpose a quad of 4 rows x 8 columns (bf16) into 8 column vectors of 4 rows and
// store them at the transposed positions of the quad (4 consecutive positions).
template <int W>
__device__ __forceinline__ void store_transposed(uint16_t* tile, const u32x4 (&rows)[4], int c,
                                                 int pq) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int w = j >> 1;
    u32x2 out;
    if (j & 1) {
      out[0] = (rows[0][w] >> 16) | (rows[1][w] & 0xFFFF0000u);
      out[1] = (rows[2][w] >> 16) | (rows[3][w] & 0xFFFF0000u);
    } else {
      out[0] = (rows[0][w] & 0xFFFFu) | (rows[1][w] << 16);
      out[1] = (rows[2][w] & 0xFFFFu) | (rows[3][w] << 16);
    }
    const int d = 8 * c + j;
    const int off = W == 64 ? t64(d, 4 * pq) : t32(d, 4 * pq);
    *reinterpret_cast<u32x2*>(tile + off) = out;
  }
}

struct KeyBlockMap {
  AttendMap m;
  int n_keys;     // attended keys of this head
  int kv_end;     // t0 + n_q: first position not in the sequence
  int local0;     // attended index of the first local key

  // Physical row (page * P + slot) and position of attended key `kidx`, or row -1.
  __device__ __forceinline__ int64_t row(int kidx, int* pos) const {
    *pos = 0x7FFFFFFF;
    if (kidx >= n_keys) return -1;
    const int e = kidx >> m.log2p;
    const int lp = m.logical(e);
    if (e < m.n_sel && m.sel && (lp < 0 || lp >= m.first_local)) return -1;
    const int64_t ph = m.physical(e, lp);
    if (ph < 0) return -1;
    const int slot = kidx & ((1 << m.log2p) - 1);
    const int p = (lp << m.log2p) + slot;
    if (p >= kv_end) return -1;
    *pos = p;
    return (ph << m.log2p) + slot;
  }
  // Largest position among attended keys [k0, k0 + 64) that may be visible, for the
  // mask decision: blocks before the local region only hold positions < t0.
  __device__ __forceinline__ bool needs_mask(int k0, int qmin_pos) const {
    const int last = k0 + KB - 1;
    if (last >= n_keys) return true;  // padding rows
    if (last < local0) return false;  // only prior keys
    const int p = (m.first_local << m.log2p) + (last - local0);
    return p > qmin_pos || p >= kv_end;
  }
};

__device__ __forceinline__ KeyBlockMap make_kmap(const AttnArgs& a, int g) {
  KeyBlockMap k;
  k.m.table = a.table + g * a.tstride;
  k.m.sel = a.sel ? a.sel + g * a.sel_stride : nullptr;
  k.m.n_sel = a.sel ? clamp_count(a.count, g, a.sel_stride, a.n_cand) : a.n_cand;
  k.m.first_local = a.first_local;
  k.m.n_pages_att = k.m.n_sel + a.n_local;
  k.m.num_pages = a.pool.N;
  k.m.log2p = a.pool.log2p;
  k.n_keys = k.m.n_pages_att << a.pool.log2p;
  k.kv_end = a.t0 + a.n_q;
  k.local0 = k.m.n_sel << a.pool.log2p;
  return k;
}

// Number of 64-key blocks a query tile whose last query sits at qmax_pos must visit.
__device__ __forceinline__ int blocks_for(const KeyBlockMap& k, int qmax_pos) {
  int last = k.local0 + (qmax_pos - (k.m.first_local << k.m.log2p));
  if (last > k.n_keys - 1) last = k.n_keys - 1;
  return last < 0 ? 0 : last / KB + 1;
}

__device__ __forceinline__ u32x4 ld_row16(const void* base, int64_t row, int c) {
  if (row < 0) return u32x4{0u, 0u, 0u, 0u};
  return *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(base) + row * D + 8 * c);
}

// ============================================================================ forward
struct FwdSmem {
  uint16_t k[2][KB * KROW];
  uint16_t vt[2][D * KB];
  int kpos[2][KB];
};

template <int QW>
__global__ __launch_bounds__(256) void fwd_mfma_kernel(AttnArgs a) {
  __shared__ FwdSmem sm;
  constexpr int QT = 128 * QW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, col = lane & 31;
  const int G = a.pool.Hq / a.pool.Hkv;
  const int n_qt = (a.n_q + QT - 1) / QT;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int hh = L % G, rest = L / G;
  const int qt = rest % n_qt, g = rest / n_qt;
  const int h = g * G + hh;
  const KeyBlockMap km = make_kmap(a, g);
  const int q0 = qt * QT;
  const int qmin_pos = a.t0 + q0;
  const int qmax_pos = a.t0 + min(a.n_q, q0 + QT) - 1;
  const int nblk = blocks_for(km, qmax_pos);
  const float c2 = a.scale * kLog2e;

  // Q fragments (B operand of S^T = K Q^T): lane holds query col, d = 16kk + 8hl + j.
  bf16x8 qf[QW][8];
  int qpos[QW];
#pragma unroll
  for (int qi = 0; qi < QW; ++qi) {
    const int i = q0 + wave * 32 * QW + qi * 32 + col;
    qpos[qi] = a.t0 + i;
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + h * a.q_hs + static_cast<int64_t>(i) * a.q_ts;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (i < a.n_q) v = *reinterpret_cast<const u32x4*>(qrow + 16 * kk + 8 * hl);
      qf[qi][kk] = as_bf16x8(v);
    }
  }

  f32x16 ot[QW][4];
  float mrow[QW], lrow[QW];
#pragma unroll
  for (int qi = 0; qi < QW; ++qi) {
    mrow[qi] = -__builtin_inff();
    lrow[qi] = 0.0f;
#pragma unroll
    for (int db = 0; db < 4; ++db) ot[qi][db] = f32x16{};
  }

  // Staging: thread = (key quad kq, 16-byte column chunk c).
  const int kq = tid >> 4, cc = tid & 15;
  u32x4 kreg[4], vreg[4];
  int rpos[4];
  auto load_block = [&](int b) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = km.row(b * KB + 4 * kq + r, &rpos[r]);
      kreg[r] = ld_row16(a.pool.k_pool, row, cc);
      vreg[r] = ld_row16(a.pool.v_pool, row, cc);
    }
  };
  auto store_block = [&](int buf) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      *reinterpret_cast<u32x4*>(&sm.k[buf][(4 * kq + r) * KROW + 8 * cc]) = kreg[r];
    store_transposed<64>(sm.vt[buf], vreg, cc, quad_pos(kq));
    if (cc == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.kpos[buf][4 * kq + r] = rpos[r];
    }
  };

  if (nblk > 0) {
    load_block(0);
    store_block(0);
  }
  __syncthreads();
  for (int b = 0; b < nblk; ++b) {
    const int buf = b & 1;
    if (b + 1 < nblk) load_block(b + 1);
    const bool mask = km.needs_mask(b * KB, qmin_pos);

    // S^T for both 32-key halves.
    f32x16 st[QW][2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int qi = 0; qi < QW; ++qi) st[qi][sub] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const bf16x8 ka = as_bf16x8(lds16(&sm.k[buf][(32 * sub + col) * KROW + 16 * kk + 8 * hl]));
#pragma unroll
        for (int qi = 0; qi < QW; ++qi) st[qi][sub] = mfma(ka, qf[qi][kk], st[qi][sub]);
      }
    }

    // Online softmax (log2 domain); each lane owns one query, the partner lane
    // (lane ^ 32) holds the other 16 keys of each half.
    bf16x8 pb[QW][2][2];
#pragma unroll
    for (int qi = 0; qi < QW; ++qi) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float s = st[qi][sub][r] * c2;
          if (mask) {
            const int kp = sm.kpos[buf][32 * sub + 8 * (r >> 2) + 4 * hl + (r & 3)];
            if (kp > qpos[qi]) s = -__builtin_inff();
          }
          st[qi][sub][r] = s;
          mx = fmaxf(mx, s);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = fmaxf(mrow[qi], mx);
      const float base = mnew == -__builtin_inff() ? 0.0f : mnew;
      const float alpha = fast_exp2(mrow[qi] - base);
      float psum = 0.0f;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          float p[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            p[j] = fast_exp2(st[qi][sub][8 * s + j] - base);
            psum += p[j];
          }
          u32x4 w;
          w[0] = pack_bf16x2(p[0], p[1]);
          w[1] = pack_bf16x2(p[2], p[3]);
          w[2] = pack_bf16x2(p[4], p[5]);
          w[3] = pack_bf16x2(p[6], p[7]);
          pb[qi][sub][s] = as_bf16x8(w);
        }
      }
      lrow[qi] = lrow[qi] * alpha + psum;
      mrow[qi] = mnew;
#pragma unroll
      for (int db = 0; db < 4; ++db) ot[qi][db] *= alpha;
    }

    // O^T += V^T P^T.
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = 32 * db + col;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8 va = as_bf16x8(lds16(&sm.vt[buf][t64(d, 32 * sub + 16 * s + 8 * hl)]));
#pragma unroll
          for (int qi = 0; qi < QW; ++qi) ot[qi][db] = mfma(va, pb[qi][sub][s], ot[qi][db]);
        }
      }
    }

    if (b + 1 < nblk) store_block(buf ^ 1);
    __syncthreads();
  }

  // Epilogue: O = O^T / l, LSE = (m + log2 l) ln 2.
#pragma unroll
  for (int qi = 0; qi < QW; ++qi) {
    const float lt = lrow[qi] + __shfl_xor(lrow[qi], 32, 64);
    const float inv = 1.0f / lt;
    const int i = q0 + wave * 32 * QW + qi * 32 + col;
    if (i < a.n_q) {
      uint16_t* orow = static_cast<uint16_t*>(a.o) + h * a.o_hs + static_cast<int64_t>(i) * a.o_ts;
#pragma unroll
      for (int db = 0; db < 4; ++db) {
#pragma unroll
        for (int ga = 0; ga < 4; ++ga) {
          u32x2 w;
          w[0] = pack_bf16x2(ot[qi][db][4 * ga + 0] * inv, ot[qi][db][4 * ga + 1] * inv);
          w[1] = pack_bf16x2(ot[qi][db][4 * ga + 2] * inv, ot[qi][db][4 * ga + 3] * inv);
          *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * ga + 4 * hl) = w;
        }
      }
      if (hl == 0) a.lse[static_cast<int64_t>(h) * a.n_q + i] = (mrow[qi] + __log2f(lt)) * kLn2;
    }
  }
}

// ============================================================================ dQ
struct DqSmem {
  uint16_t k[2][KB * KROW];
  uint16_t v[2][KB * KROW];
  uint16_t kt[2][D * KB];
  int kpos[2][KB];
};

__global__ __launch_bounds__(256) void dq_mfma_kernel(AttnArgs a) {
  __shared__ DqSmem sm;
  constexpr int QT = 128;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, col = lane & 31;
  const int G = a.pool.Hq / a.pool.Hkv;
  const int n_qt = (a.n_q + QT - 1) / QT;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int hh = L % G, rest = L / G;
  const int qt = rest % n_qt, g = rest / n_qt;
  const int h = g * G + hh;
  const KeyBlockMap km = make_kmap(a, g);
  const int q0 = qt * QT;
  const int qmin_pos = a.t0 + q0;
  const int qmax_pos = a.t0 + min(a.n_q, q0 + QT) - 1;
  const int nblk = blocks_for(km, qmax_pos);
  const float c2 = a.scale * kLog2e;

  const int i = q0 + wave * 32 + col;
  const int qpos = a.t0 + i;
  bf16x8 qf[8], df[8];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + h * a.q_hs + static_cast<int64_t>(i) * a.q_ts;
    const uint16_t* drow = static_cast<const uint16_t*>(a.dout) + h * a.do_hs + static_cast<int64_t>(i) * a.do_ts;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      u32x4 v = u32x4{0u, 0u, 0u, 0u}, w = v;
      if (i < a.n_q) {
        v = *reinterpret_cast<const u32x4*>(qrow + 16 * kk + 8 * hl);
        w = *reinterpret_cast<const u32x4*>(drow + 16 * kk + 8 * hl);
      }
      qf[kk] = as_bf16x8(v);
      df[kk] = as_bf16x8(w);
    }
  }
  const int64_t rid = static_cast<int64_t>(h) * a.n_q + i;
  const float lse2 = i < a.n_q ? a.lse_in[rid] * kLog2e : __builtin_inff();
  const float delta = i < a.n_q ? a.delta[rid] : 0.0f;

  f32x16 dqt[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) dqt[db] = f32x16{};

  const int kq = tid >> 4, cc = tid & 15;
  u32x4 kreg[4], vreg[4];
  int rpos[4];
  auto load_block = [&](int b) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = km.row(b * KB + 4 * kq + r, &rpos[r]);
      kreg[r] = ld_row16(a.pool.k_pool, row, cc);
      vreg[r] = ld_row16(a.pool.v_pool, row, cc);
    }
  };
  auto store_block = [&](int buf) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      *reinterpret_cast<u32x4*>(&sm.k[buf][(4 * kq + r) * KROW + 8 * cc]) = kreg[r];
      *reinterpret_cast<u32x4*>(&sm.v[buf][(4 * kq + r) * KROW + 8 * cc]) = vreg[r];
    }
    store_transposed<64>(sm.kt[buf], kreg, cc, quad_pos(kq));
    if (cc == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.kpos[buf][4 * kq + r] = rpos[r];
    }
  };

  if (nblk > 0) {
    load_block(0);
    store_block(0);
  }
  __syncthreads();
  for (int b = 0; b < nblk; ++b) {
    const int buf = b & 1;
    if (b + 1 < nblk) load_block(b + 1);
    const bool mask = km.needs_mask(b * KB, qmin_pos);
    bf16x8 dsb[2][2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      f32x16 st = f32x16{}, dpt = f32x16{};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int off = (32 * sub + col) * KROW + 16 * kk + 8 * hl;
        st = mfma(as_bf16x8(lds16(&sm.k[buf][off])), qf[kk], st);
        dpt = mfma(as_bf16x8(lds16(&sm.v[buf][off])), df[kk], dpt);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        float ds[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = 8 * s + j;
          float p = fast_exp2(st[r] * c2 - lse2);
          if (mask) {
            const int kp = sm.kpos[buf][32 * sub + 8 * (r >> 2) + 4 * hl + (r & 3)];
            if (kp > qpos) p = 0.0f;
          }
          ds[j] = p * (dpt[r] - delta);
        }
        u32x4 w;
        w[0] = pack_bf16x2(ds[0], ds[1]);
        w[1] = pack_bf16x2(ds[2], ds[3]);
        w[2] = pack_bf16x2(ds[4], ds[5]);
        w[3] = pack_bf16x2(ds[6], ds[7]);
        dsb[sub][s] = as_bf16x8(w);
      }
    }
    // dQ^T += K^T dS^T.
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = 32 * db + col;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8 ka = as_bf16x8(lds16(&sm.kt[buf][t64(d, 32 * sub + 16 * s + 8 * hl)]));
          dqt[db] = mfma(ka, dsb[sub][s], dqt[db]);
        }
      }
    }
    if (b + 1 < nblk) store_block(buf ^ 1);
    __syncthreads();
  }

  if (i < a.n_q) {
    float* drow = a.dq + h * a.dq_hs + static_cast<int64_t>(i) * a.dq_ts;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
#pragma unroll
      for (int ga = 0; ga < 4; ++ga) {
        f32x4 w;
#pragma unroll
        for (int b2 = 0; b2 < 4; ++b2) w[b2] = dqt[db][4 * ga + b2] * a.scale;
        *reinterpret_cast<f32x4*>(drow + 32 * db + 8 * ga + 4 * hl) = w;
      }
    }
  }
}

// ============================================================================ dK / dV
constexpr int QTB = 32;  // queries per staged tile in the dK/dV pass

struct DkvTile {
  uint16_t q[QTB * KROW];
  uint16_t d[QTB * KROW];
  uint16_t qt[D * QTB];
  uint16_t dt[D * QTB];
  float lse2[QTB];
  float delta[QTB];
};
union DkvSmem {
  DkvTile tile[2];                   // one per query stream
  float red[2][2][16][64 * 4];       // [key group][dK|dV][reg][lane x 4 n-blocks]
};

__global__ __launch_bounds__(256) void dkdv_mfma_kernel(AttnArgs a) {
  __shared__ DkvSmem sm;
  __shared__ int64_t s_grow[KB];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, col = lane & 31;
  const int kg = wave & 1, qs = wave >> 1;
  const int G = a.pool.Hq / a.pool.Hkv;
  const int nkb = (a.max_att_pages * a.pool.P + KB - 1) / KB;
  const int L = xcd_remap(blockIdx.x, gridDim.x);
  const int kb = L % nkb, g = L / nkb;
  const KeyBlockMap km = make_kmap(a, g);
  const int k0 = kb * KB;
  if (k0 >= km.n_keys) return;  // whole workgroup: this block is past the attended keys
  const float c2 = a.scale * kLog2e;

  // This lane's key (column of S = Q K^T).
  int kpos;
  const int64_t krow = km.row(k0 + 32 * kg + col, &kpos);
  if (qs == 0 && hl == 0) {
    int64_t grow = -1;
    if (krow >= 0) {
      const int e = (k0 + 32 * kg + col) >> km.m.log2p;
      const int lp = km.m.logical(e);
      const int64_t gp = a.gtable[g * a.gtstride + lp];
      if (gp >= 0 && gp < a.pool.Ng) grow = (gp << km.m.log2p) + (kpos & (a.pool.P - 1));
    }
    s_grow[32 * kg + col] = grow;
  }
  bf16x8 kf[8], vf[8];
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    u32x4 x = u32x4{0u, 0u, 0u, 0u}, y = x;
    if (krow >= 0) {
      x = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.pool.k_pool) + krow * D + 16 * kk + 8 * hl);
      y = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.pool.v_pool) + krow * D + 16 * kk + 8 * hl);
    }
    kf[kk] = as_bf16x8(x);
    vf[kk] = as_bf16x8(y);
  }

  // Queries that can see any key of this block.
  int first_pos;
  km.row(k0, &first_pos);
  const int i_start = first_pos > a.t0 ? first_pos - a.t0 : 0;
  const int n_qt = (a.n_q + QTB - 1) / QTB;
  const int qt0 = i_start >= a.n_q ? n_qt : i_start / QTB;
  const int tph = n_qt - qt0;  // tiles per head
  const int n_tiles = G * tph;
  const int n_iter = (n_tiles + 1) / 2;

  f32x16 dv[4], dk[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    dv[nb] = f32x16{};
    dk[nb] = f32x16{};
  }

  // Staging: item j in {0: Q, 1: dO}; thread = (stream tile st, query quad, chunk).
  const int st_tile = tid >> 7, sq = (tid >> 4) & 7, sc = tid & 15;
  u32x4 reg[2][4];
  float r_lse2 = 0.0f, r_delta = 0.0f;
  auto tile_of = [&](int u, int* hq, int* q0) {
    *hq = g * G + u / tph;
    *q0 = (qt0 + u % tph) * QTB;
  };
  auto load_tiles = [&](int it) {
    const int u = 2 * it + st_tile;
    int hq = 0, q0 = 0;
    const bool ok = u < n_tiles;
    if (ok) tile_of(u, &hq, &q0);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = q0 + 4 * sq + r;
      u32x4 x = u32x4{0u, 0u, 0u, 0u}, y = x;
      if (ok && i < a.n_q) {
        x = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.q) + hq * a.q_hs + static_cast<int64_t>(i) * a.q_ts + 8 * sc);
        y = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.dout) + hq * a.do_hs + static_cast<int64_t>(i) * a.do_ts + 8 * sc);
      }
      reg[0][r] = x;
      reg[1][r] = y;
    }
    if ((tid & 127) < QTB) {
      const int i = q0 + (tid & 127);
      const int64_t rid = static_cast<int64_t>(hq) * a.n_q + i;
      const bool v = ok && i < a.n_q;
      r_lse2 = v ? a.lse_in[rid] * kLog2e : __builtin_inff();
      r_delta = v ? a.delta[rid] : 0.0f;
    }
  };
  auto store_tiles = [&]() {
    DkvTile& t = sm.tile[st_tile];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      *reinterpret_cast<u32x4*>(&t.q[(4 * sq + r) * KROW + 8 * sc]) = reg[0][r];
      *reinterpret_cast<u32x4*>(&t.d[(4 * sq + r) * KROW + 8 * sc]) = reg[1][r];
    }
    store_transposed<32>(t.qt, reg[0], sc, quad_pos(sq));
    store_transposed<32>(t.dt, reg[1], sc, quad_pos(sq));
    if ((tid & 127) < QTB) {
      t.lse2[tid & 127] = r_lse2;
      t.delta[tid & 127] = r_delta;
    }
  };

  if (n_iter > 0) load_tiles(0);
  for (int it = 0; it < n_iter; ++it) {
    __syncthreads();  // previous iteration's readers are done with the tiles
    store_tiles();
    __syncthreads();
    if (it + 1 < n_iter) load_tiles(it + 1);
    const int u = 2 * it + qs;
    if (u < n_tiles) {
      int hq, q0;
      tile_of(u, &hq, &q0);
      const DkvTile& t = sm.tile[qs];
      const bool mask = km.needs_mask(k0, a.t0 + q0);
      // S = Q K^T and dP = dO V^T for this wave's 32 keys.
      f32x16 s_acc = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        const int off = col * KROW + 16 * kk + 8 * hl;
        s_acc = mfma(as_bf16x8(lds16(&t.q[off])), kf[kk], s_acc);
        dp = mfma(as_bf16x8(lds16(&t.d[off])), vf[kk], dp);
      }
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        float p[8], ds[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = 8 * s + j;
          const int qr = 8 * (r >> 2) + 4 * hl + (r & 3);
          float pv = fast_exp2(s_acc[r] * c2 - t.lse2[qr]);
          if (mask && kpos > a.t0 + q0 + qr) pv = 0.0f;
          p[j] = pv;
          ds[j] = pv * (dp[r] - t.delta[qr]);
        }
        u32x4 w, z;
        w[0] = pack_bf16x2(p[0], p[1]);
        w[1] = pack_bf16x2(p[2], p[3]);
        w[2] = pack_bf16x2(p[4], p[5]);
        w[3] = pack_bf16x2(p[6], p[7]);
        z[0] = pack_bf16x2(ds[0], ds[1]);
        z[1] = pack_bf16x2(ds[2], ds[3]);
        z[2] = pack_bf16x2(ds[4], ds[5]);
        z[3] = pack_bf16x2(ds[6], ds[7]);
        pb[s] = as_bf16x8(w);
        dsb[s] = as_bf16x8(z);
      }
      // dV += P^T dO, dK += dS^T Q (scale applied at the end).
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int d = 32 * nb + col;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int off = t32(d, 16 * s + 8 * hl);
          dv[nb] = mfma(pb[s], as_bf16x8(lds16(&t.dt[off])), dv[nb]);
          dk[nb] = mfma(dsb[s], as_bf16x8(lds16(&t.qt[off])), dk[nb]);
        }
      }
    }
  }

  // Merge the two query streams, then one read-modify-write per key row.
  __syncthreads();
  if (qs == 1) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        sm.red[kg][0][r][lane * 4 + nb] = dk[nb][r];
        sm.red[kg][1][r][lane * 4 + nb] = dv[nb][r];
      }
    }
  }
  __syncthreads();
  if (qs == 0) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 8 * (r >> 2) + 4 * hl + (r & 3);
      const int64_t grow = s_grow[32 * kg + m];
      if (grow < 0) continue;
      float* dkr = a.pool.dk_pool + grow * D;
      float* dvr = a.pool.dv_pool + grow * D;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const float kval = (dk[nb][r] + sm.red[kg][0][r][lane * 4 + nb]) * a.scale;
        const float vval = dv[nb][r] + sm.red[kg][1][r][lane * 4 + nb];
        dkr[32 * nb + col] += kval;
        dvr[32 * nb + col] += vval;
      }
    }
  }
}

}  // namespace mf

hipError_t launch_fwd_mfma(const AttnArgs& a, hipStream_t s) {
  constexpr int QW = 1;
  const int n_qt = (a.n_q + 128 * QW - 1) / (128 * QW);
  const int grid = a.pool.Hq * n_qt;
  hipLaunchKernelGGL(mf::fwd_mfma_kernel<QW>, dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_bwd_mfma(const AttnArgs& a, hipStream_t s) {
  hipError_t err = launch_delta(a, s);
  if (err != hipSuccess) return err;
  const int n_qt = (a.n_q + 127) / 128;
  hipLaunchKernelGGL(mf::dq_mfma_kernel, dim3(a.pool.Hq * n_qt), dim3(256), 0, s, a);
  const int nkb = (a.max_att_pages * a.pool.P + mf::KB - 1) / mf::KB;
  hipLaunchKernelGGL(mf::dkdv_mfma_kernel, dim3(a.pool.Hkv * nkb), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace oomb
