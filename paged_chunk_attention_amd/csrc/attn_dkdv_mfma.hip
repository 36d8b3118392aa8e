// Matrix-core backward of paged chunk attention, dK/dV pass (race-free, one owner per
// gradient row) and the launcher of the whole backward (Delta, dQ, dK/dV, merge).
#include "mfma_tiles.hpp"

namespace oomb {
namespace mf {

// ============================================================================ dK / dV
// Grid: Hkv * (key blocks of 128) * n_split. With n_split > 1, split s writes its
// partial dK/dV rows to part[((s * Hkv + g) * part_keys + key) * 2D + {0: dK, D: dV}].
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1)))
void dkdv_mfma_kernel(AttnArgs a, int n_split, float* part, int part_keys) {
  // Double-buffered Q / dO tiles and their rows' LSE (x log2 e) and Delta, each buffer
  // its own object (see prefetch_next), and the output row of each key.
  __shared__ __attribute__((aligned(16))) uint16_t s_q0[QTB * D];
  __shared__ __attribute__((aligned(16))) uint16_t s_d0[QTB * D];
  __shared__ __attribute__((aligned(16))) uint16_t s_q1[QTB * D];
  __shared__ __attribute__((aligned(16))) uint16_t s_d1[QTB * D];
  __shared__ __attribute__((aligned(16))) float s_lse0[QTB], s_lse1[QTB], s_del0[QTB], s_del1[QTB];
  __shared__ int64_t s_grow[KPW];  // gradient pool row (or partial row) of each key, -1 = skip
  // the wave index is uniform: keep it (and the LDS addresses built from it) scalar
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    s_grow[32 * wave + col] = out;
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

  // Query tiles go straight from global memory into LDS (DMA); the LSE and Delta of
  // the tile's rows take a small register path.
  float r_lse = 0.0f, r_delta = 0.0f;
  auto issue_tile = [&](int u, uint16_t* qd, uint16_t* dd) {
    const int hq = g * G + u / tph, q0 = (qt0 + u % tph) * QTB;
    const int c8 = dma_col(wave, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r0 = 16 * i + 4 * wave;
      const int qi = q0 + r0 + (lane >> 4);
      if (qi < a.n_q) {
        lds_dma16(static_cast<const uint16_t*>(a.q) + hq * a.q_hs + static_cast<int64_t>(qi) * a.q_ts + c8, qd + r0 * D);
        lds_dma16(static_cast<const uint16_t*>(a.dout) + hq * a.do_hs + static_cast<int64_t>(qi) * a.do_ts + c8, dd + r0 * D);
      }
    }
    if (tid < QTB) {  // raw loads: arithmetic here would wait for the whole prefetch
      const int qi = q0 + tid;
      const int64_t rid = static_cast<int64_t>(hq) * a.n_q + qi;
      r_lse = qi < a.n_q ? a.lse_in[rid] : __builtin_inff();
      r_delta = qi < a.n_q ? a.delta[rid] : 0.0f;
    }
  };
  auto store_rows = [&](float* lse, float* del) {
    if (tid < QTB) {
      lse[tid] = r_lse * kLog2e;
      del[tid] = r_delta;
    }
  };

  zero_tile<QTB, 256>(s_q0, tid);
  zero_tile<QTB, 256>(s_d0, tid);
  zero_tile<QTB, 256>(s_q1, tid);
  zero_tile<QTB, 256>(s_d1, tid);
  __syncthreads();
  if (u_begin < u_end) issue_tile(u_begin, s_q0, s_d0);
  wait_dma();
  store_rows(s_lse0, s_del0);
  __syncthreads();
  // One query tile: prefetch tile u + 1 into (qn, dn, lsen, deln), compute tile u.
  auto step = [&](int u, const uint16_t* qt, const uint16_t* dt, const float* lse,
                  const float* del, uint16_t* qn, uint16_t* dn, float* lsen,
                  float* deln) __attribute__((always_inline)) {
    if (u + 1 < u_end) issue_tile(u + 1, qn, dn);
    const int q0 = (qt0 + u % tph) * QTB;
    // Some (key, query) pair of this tile is hidden for this lane's key?
    const bool wmask = __any(kpos > a.t0 + q0);
    // S = Q K^T and dP = dO V^T over d for both 32-query halves (four MFMA chains),
    // so that the softmax arithmetic of one half can overlap the other's products.
    f32x16 sa[2], dpa[2];
#pragma unroll
    for (int us = 0; us < 2; ++us) {
      bf16x8 qa[8], da[8];
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        qa[kk] = row_frag(qt, 32 * us, kk, lane);
        da[kk] = row_frag(dt, 32 * us, kk, lane);
      }
      sa[us] = f32x16{};
      dpa[us] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < 8; ++kk) {
        sa[us] = mfma(qa[kk], kf[kk], sa[us]);
        dpa[us] = mfma(da[kk], vf[kk], dpa[us]);
      }
    }
#pragma unroll
    for (int us = 0; us < 2; ++us) {
      bf16x8 tdo[2][4], tq[2][4];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          tdo[s][nb] = tr_frag(dt, 32 * us, 32 * nb, s, lane);
          tq[s][nb] = tr_frag(qt, 32 * us, 32 * nb, s, lane);
        }
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        // query rows rA + 8(j/4) + (j%4), j = 0..7, rA = 32us + 16s + 4h2
        const int rA = 32 * us + 16 * s + 4 * h2;
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(lse + rA);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(lse + rA + 8);
        const f32x4 d0 = *reinterpret_cast<const f32x4*>(del + rA);
        const f32x4 d1 = *reinterpret_cast<const f32x4*>(del + rA + 8);
        float p[8], ds[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int r = 8 * s + j;
          const float lse_r = j < 4 ? l0[j] : l1[j - 4];
          const float del_r = j < 4 ? d0[j] : d1[j - 4];
          float pv = fast_exp2(__builtin_fmaf(sa[us][r], c2, -lse_r));
          if (wmask && kpos > a.t0 + q0 + rA + 8 * (j >> 2) + (j & 3)) pv = 0.0f;
          p[j] = pv;
          ds[j] = pv * (dpa[us][r] - del_r);
        }
        pb[s] = pack8(p);
        dsb[s] = pack8(ds);
      }
      // dV += P^T dO, dK += dS^T Q (the scale is applied once, at the end).
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          dv[nb] = mfma(pb[s], tdo[s][nb], dv[nb]);
          dk[nb] = mfma(dsb[s], tq[s][nb], dk[nb]);
        }
    }
    wait_dma();  // the next tile has landed (this wave's part)
    if (u + 1 < u_end) store_rows(lsen, deln);
    __syncthreads();
  };
  for (int u = u_begin; u < u_end; u += 2) {
    step(u, s_q0, s_d0, s_lse0, s_del0, s_q1, s_d1, s_lse1, s_del1);
    if (u + 1 < u_end) step(u + 1, s_q1, s_d1, s_lse1, s_del1, s_q0, s_d0, s_lse0, s_del0);
  }

  // Write out: register r holds key row m = 8(r/4) + 4h2 + r%4 of this wave, column
  // 32nb + col of d.
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = 8 * (r >> 2) + 4 * h2 + (r & 3);
    const int64_t out = s_grow[32 * wave + m];
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
  err = launch_dq_mfma(a, s);
  if (err != hipSuccess) return err;
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
