// Matrix-core backward of paged chunk attention, dK/dV pass (race-free, one owner per
// gradient row) and the launcher of the whole backward (dQ with Delta, dK/dV, merges).
#include "mfma_tiles.hpp"

namespace oomb {
namespace mf {

// ============================================================================ dK / dV
// Grid: Hkv * units; per KV head, the first `whole` key blocks of 128 (in block order)
// are one unit each and add into the gradient pool directly, every later block is
// n_split units over its query stream. Split s of such a block writes its partial
// dK/dV rows to part[((s * Hkv + g) * part_keys + key) * 2D + {0: dK, D: dV}], and a
// merge kernel adds them into the pool in split order.
//
// A workgroup is 8 wavefronts that own 128 keys, 32 per key group kg = wave % 4. The
// two wavefronts of a key group share a SIMD and split its work by role:
//  * the P wave holds K (B operand over d) and dV: per 64-query tile it computes
//    S = Q K^T, P = exp(S - LSE) (masked), hands P (fp16) to its partner through LDS,
//    and adds P^T dO into dV;
//  * the D wave holds V and dK: it computes dP = dO V^T of a tile, and one tile later,
//    once that tile's P has arrived, dS = P (dP - Delta) and dK += dS^T Q.
// Each wave carries half of the state of one owner of 32 keys, so two fit on a SIMD,
// and the hardware overlaps one wave's softmax arithmetic with the other's products.
// The D wave's order (dS and dK of the previous tile, then dP of this one) puts its
// 32 products under the P wave's softmax. Without SPILL it runs its tile at raised wave
// priority, so that the SIMD's arbiter feeds the matrix core first whenever both waves
// are ready (measured 4-5% faster than equal priorities; raising the P wave's products
// too gained less). With SPILL the waves keep equal priorities: there the raised D wave
// measured 3-4% slower, its products delaying the P wave's S chain, which the softmax
// and dV wait for. Query tiles arrive by DMA one tile ahead: Q in three buffers (the
// D wave still reads the previous tile's), dO in two; the buffers' roles are static in
// each sixth of the unrolled loop. P has to be exactly 0 for masked pairs and at most
// about 1 elsewhere (it is exp(S - LSE) with the forward's LSE), which fp16 holds.
//
// With SPILL the D wave also writes every dS tile it forms to ds, for the dQ pass to use
// instead of recomputing S and dP: its bf16 dS^T operands as they are, per (query head,
// key block, 64-query tile, key group) one record block of DS_REC values, [pack p =
// 2 us + s][lane][8], where lane (h2, col) holds key 32 kg + col and element j of pack
// (us, s) is query row 32 us + 16 s + 4 h2 + 8 (j / 4) + j % 4 of the tile. Four 16-byte
// stores per lane and tile, each a contiguous 1 KiB. The dQ product contracts over keys
// and so wants the transpose; the dQ pass forms it with transposing LDS reads, which
// costs it less than the two extra products a tile would cost here (measured: this pass
// 2.4% faster at dense 128K, the dQ pass 4% slower, the backward 0.8% faster). Masked
// pairs store exact zeros (P = 0); the tiles the pass never visits (query tiles wholly
// before a chunk key block) are never read.
//
// The D wave never waits for its stores: with SPILL the P waves stage both the Q and
// the dO tiles (and load the rows' LSE and Delta), so a D wave issues no load in the
// loop, and the loop's barrier carries no memory fence (every wave that staged or wrote
// LDS waits for that itself before it). Waiting at each barrier for the stores cost the
// pass up to half its time.
constexpr int DKV_WAVES = 8;

template <bool SPILL>
__global__ __launch_bounds__(64 * DKV_WAVES) __attribute__((amdgpu_waves_per_eu(2)))
void dkdv_mfma_kernel(AttnArgs a, int n_split, int whole, float* part, int part_keys,
                      uint16_t* ds) {
  __shared__ __attribute__((aligned(16))) uint16_t s_q0[QTB * D];
  __shared__ __attribute__((aligned(16))) uint16_t s_q1[QTB * D];
  __shared__ __attribute__((aligned(16))) uint16_t s_q2[QTB * D];
  __shared__ __attribute__((aligned(16))) uint16_t s_d0[QTB * D];
  __shared__ __attribute__((aligned(16))) uint16_t s_d1[QTB * D];
  // LSE (x log2 e) and Delta of the rows of the tile in the Q buffer of the same index
  __shared__ __attribute__((aligned(16))) float s_lse0[QTB], s_lse1[QTB], s_lse2[QTB];
  __shared__ __attribute__((aligned(16))) float s_del0[QTB], s_del1[QTB], s_del2[QTB];
  // P (fp16) of one tile for each key group: [tile parity][kg][2us + s][lane], eight
  // values (j = 0..7) per lane. fp16 keeps 11 significant bits for P in [0, 1] (bf16
  // keeps 8): the dS that the D wave forms from it is rounded to bf16 anyway, so the
  // exchange adds a small fraction of that rounding, at half the LDS traffic of fp32.
  // (A bf16 exchange doubled dS's rounding and failed the dK bar.)
  __shared__ __attribute__((aligned(16))) h16x8 s_p[2 * 4 * 4 * 64];
  __shared__ int64_t s_grow[KPW];  // gradient pool row (or partial row) of each key, -1 = skip
  // the wave index is uniform: keep it (and the LDS addresses built from it) scalar
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = wave & 3;
  const bool pwave = wave < 4;
  const int h2 = lane >> 5, col = lane & 31;
  const int G = a.pool.Hq / a.pool.Hkv;
  const int nkb = (a.max_att_pages * a.pool.P + KPW - 1) / KPW;
  // A head's units in key-block order (the splits of a block consecutive): the work per
  // block only falls with the index (local blocks see fewer query tiles), so this is
  // longest first.
  const HeadUnit hu = head_unit(blockIdx.x, gridDim.x, a.pool.Hkv);
  const TileRange tr = tile_range(hu.unit, whole, n_split);
  const int g = hu.head, split = tr.range, n_parts = tr.n_ranges, kb = tr.tile;
  const Keys km = make_keys(a, g);
  const int k0 = kb * KPW;
  if (kb >= nkb || k0 >= km.n_keys) return;  // uniform: block past this head's attended keys
  const float c2 = a.scale * kLog2e;
  // Pairs with q - k >= wlim lie outside the window (none without one).
  const int wlim = km.window > 0 ? km.window : 0x7FFFFFFF;

  // This lane's key (column of S = Q K^T) and its K (P wave) or V (D wave) fragments.
  const int kidx = k0 + 32 * kg + col;
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
  if (pwave && h2 == 0) {
    int64_t out = -1;
    if (krow >= 0) {
      if (n_parts > 1) {
        out = kidx;  // partial row index
      } else {
        const int64_t gp = a.gtable[g * a.gtstride + (kpos >> km.log2p)];
        if (gp >= 0 && gp < a.pool.Ng) out = (gp << km.log2p) + (kpos & ((1 << km.log2p) - 1));
      }
    }
    s_grow[32 * kg + col] = out;
  }
  bf16x8 kvf[8];
  {
    const void* src = pwave ? a.pool.k_pool : a.pool.v_pool;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk)
      kvf[kk] = as_bf16x8(krow >= 0 ? gld16(src, krow * D + 16 * kk + 8 * h2) : u32x4{0u, 0u, 0u, 0u});
  }

  // Query tiles that can see some key of this block: every head of the group, from
  // the first query at or after the block's first key (with a window, up to the last
  // query whose window still reaches the block's last key); cut into n_parts parts.
  const int n_qt = (a.n_q + QTB - 1) / QTB;
  int qt0 = 0, qt_end = n_qt;
  if (!km.in_seq(k0)) {
    qt0 = n_qt;
  } else if (k0 >= km.local0 || km.window > 0) {  // positions linear (window calls are dense)
    const int first_pos = km.pos_linear(k0);
    qt0 = first_pos > a.t0 ? (first_pos - a.t0) / QTB : 0;
  }
  if (km.window > 0) {
    const int lim = km.pos_linear(min(k0 + KPW, km.n_keys) - 1) + km.window - 1 - a.t0;
    qt_end = lim < 0 ? 0 : min(n_qt, lim / QTB + 1);
  }
  const int tph = max(0, qt_end - qt0);
  const int n_tiles = G * tph;
  const int u_begin = static_cast<int>((static_cast<int64_t>(n_tiles) * split) / n_parts);
  const int u_end = static_cast<int>((static_cast<int64_t>(n_tiles) * (split + 1)) / n_parts);
  const int n_it = u_end - u_begin;

  f32x16 acc[4];  // dV (P wave) or dK (D wave): register r = key row, lane column = d
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x16{};
  f32x16 dpa[2] = {f32x16{}, f32x16{}};  // D wave: dP of the tile in flight

  // Query tiles go straight from global memory into LDS (DMA): Q by the P waves, dO by
  // the D waves. The LSE (wave 0) and Delta (wave 4) of the tile's rows take a small
  // register path, stored once the tile has landed.
  float r_row = 0.0f;
  // Rows 16 i + 4 kg .. +3 (i = 0..3) of one tile of `src` into dst.
  auto stage_rows = [&](const uint16_t* src, int64_t ts, int q0, uint16_t* dst) {
    const int c8 = dma_col(kg, lane);
    if (q0 + QTB <= a.n_q) {  // uniform: the whole tile is in range
      const int64_t lo = static_cast<int64_t>(lane >> 4) * ts + c8;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r0 = 16 * i + 4 * kg;
        lds_dma16(src + static_cast<int64_t>(q0 + r0) * ts + lo, dst + r0 * D);
      }
    } else {
      // The last, partial tile: rows past the end reload the last row. Their data is
      // finite and their LSE +inf, so their P (and dS) is exactly zero.
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r0 = 16 * i + 4 * kg;
        const int qi = min(q0 + r0 + (lane >> 4), a.n_q - 1);
        lds_dma16(src + static_cast<int64_t>(qi) * ts + c8, dst + r0 * D);
      }
    }
  };
  // Wave kg of each role stages its rows of the tile (SPILL: the P waves stage both);
  // the LSE (P wave 0) and Delta (wave 4, or P wave 1 with SPILL) take a small register
  // path, stored once the tile has landed.
  const bool lse_wave = pwave && kg == 0;
  const bool del_wave = SPILL ? (pwave && kg == 1) : (!pwave && kg == 0);
  auto issue_tile = [&](int u, uint16_t* qd, uint16_t* dd) {
    const int hq = g * G + u / tph, q0 = (qt0 + u % tph) * QTB;
    const uint16_t* qsrc = static_cast<const uint16_t*>(a.q) + hq * a.q_hs;
    const uint16_t* dsrc = static_cast<const uint16_t*>(a.dout) + hq * a.do_hs;
    if (pwave) stage_rows(qsrc, a.q_ts, q0, qd);
    if (SPILL ? pwave : !pwave) stage_rows(dsrc, a.do_ts, q0, dd);
    if (lse_wave || del_wave) {  // raw loads: arithmetic here would wait for the whole prefetch
      const int qi = q0 + lane;
      const int64_t rid = static_cast<int64_t>(hq) * a.n_q + qi;
      if (lse_wave) r_row = qi < a.n_q ? a.lse_in[rid] : __builtin_inff();
      else r_row = qi < a.n_q ? a.delta[rid] : 0.0f;
    }
  };
  auto store_rows = [&](float* lse, float* del) {
    if (lse_wave) lse[lane] = r_row * kLog2e;
    else if (del_wave) del[lane] = r_row;
  };

  FragOffsets fo;
  fo.init(lane);
  zero_tile<QTB, 64 * DKV_WAVES>(s_q0, tid);
  zero_tile<QTB, 64 * DKV_WAVES>(s_q1, tid);
  zero_tile<QTB, 64 * DKV_WAVES>(s_q2, tid);
  zero_tile<QTB, 64 * DKV_WAVES>(s_d0, tid);
  zero_tile<QTB, 64 * DKV_WAVES>(s_d1, tid);
  __syncthreads();
  if (n_it > 0) issue_tile(u_begin, s_q0, s_d0);
  wait_dma();
  store_rows(s_lse0, s_del0);
  __syncthreads();

  // P wave, tile u from (qt, dt, lse); writes P into s_p parity xp.
  auto p_tile = [&](int u, const uint16_t* qt, const uint16_t* dt, const float* lse, int xp)
      __attribute__((always_inline)) {
    const int q0 = (qt0 + u % tph) * QTB;
    // Some pair of this tile hidden for this lane's key (in its future, or past the end
    // of a window: q - kpos >= window, written so that kpos = INT_MAX cannot overflow)?
    const bool wmask = __any(kpos > a.t0 + q0 || a.t0 + q0 + QTB - 1 - kpos >= wlim);
    fo.opaque();
    const FragOffsets& o = fo;
    // S = Q K^T for both 32-query halves, the two chains interleaved, fragments read one
    // step ahead.
    f32x16 sa[2] = {f32x16{}, f32x16{}};
    bf16x8 fq = row_frag_at(qt, 0, o, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int us = i & 1, kk = i >> 1;
      bf16x8 nq = fq;
      if (i + 1 < 16) nq = row_frag_at(qt, 32 * ((i + 1) & 1), o, (i + 1) >> 1);
      sa[us] = mfma(fq, kvf[kk], sa[us]);
      fq = nq;
    }
    // P = exp2(S c - LSE log2 e) in place; register 8s + j of half us holds query row
    // rA + 8(j/4) + (j%4), j = 0..7, rA = 32us + 16s + 4h2.
#pragma unroll
    for (int us = 0; us < 2; ++us)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int rA = 32 * us + 16 * s + 4 * h2;
        const f32x4 l0 = *reinterpret_cast<const f32x4*>(lse + rA);
        const f32x4 l1 = *reinterpret_cast<const f32x4*>(lse + rA + 8);
#pragma unroll
        for (int j = 0; j < 8; ++j)
          sa[us][8 * s + j] = fast_exp2(__builtin_fmaf(sa[us][8 * s + j], c2, -(j < 4 ? l0[j] : l1[j - 4])));
      }
    // One uniform branch per tile, branch-free inside: the masked pairs of tiles on the
    // block's diagonal (or window edge) get P = 0.
    if (wmask) {
#pragma unroll
      for (int us = 0; us < 2; ++us)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int qpos = a.t0 + q0 + 32 * us + 16 * (r >> 3) + 4 * h2 + 8 * ((r >> 2) & 1) + (r & 3);
          const bool hide = (kpos > qpos) | (qpos - kpos >= wlim);
          sa[us][r] = hide ? 0.0f : sa[us][r];
        }
    }
    bf16x8 pb[2][2];
#pragma unroll
    for (int us = 0; us < 2; ++us)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = sa[us][8 * s + j];
        pb[us][s] = pack8(p);
        h16x8 ph;
#pragma unroll
        for (int j = 0; j < 8; ++j) ph[j] = static_cast<_Float16>(p[j]);
        s_p[((xp * 4 + kg) * 4 + 2 * us + s) * 64 + lane] = ph;
      }
    // dV += P^T dO, transposed dO fragments read one step ahead.
    bf16x8 ft = tr_frag_at(dt, 0, 0, o, 0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int nb = i & 3, s = (i >> 2) & 1, us = i >> 3;
      bf16x8 nt = ft;
      if (i + 1 < 16) {
        const int j = i + 1;
        nt = tr_frag_at(dt, 32 * (j >> 3), (j >> 2) & 1, o, j & 3);
      }
      acc[nb] = mfma(pb[us][s], ft, acc[nb]);
      ft = nt;
    }
  };

  // D wave: dS and dK of the previous tile (qp, delp, P parity xp), if any, then dP of
  // tile dt, if any.
  auto d_tile = [&](bool prev, const uint16_t* qp, const float* delp, int xp, bool cur,
                    const uint16_t* dt, int u_prev) __attribute__((always_inline)) {
    fo.opaque();
    const FragOffsets& o = fo;
    if constexpr (!SPILL) __builtin_amdgcn_s_setprio(1);
    if (prev) {
      bf16x8 dsb[2][2];
#pragma unroll
      for (int us = 0; us < 2; ++us)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int rA = 32 * us + 16 * s + 4 * h2;
          const f32x4 d0 = *reinterpret_cast<const f32x4*>(delp + rA);
          const f32x4 d1 = *reinterpret_cast<const f32x4*>(delp + rA + 8);
          const h16x8 ph = s_p[((xp * 4 + kg) * 4 + 2 * us + s) * 64 + lane];
          float dsv[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float pv = static_cast<float>(ph[j]);
            const float del_r = j < 4 ? d0[j] : d1[j - 4];
            // an fma with the fp16 operand widened in the instruction (v_fma_mix)
            dsv[j] = __builtin_fmaf(pv, dpa[us][8 * s + j] - del_r, 0.0f);
          }
          dsb[us][s] = pack8(dsv);
        }
      if constexpr (SPILL) {
        const int hq = g * G + u_prev / tph, qt = qt0 + u_prev % tph;
        uint16_t* rec = ds + ((((static_cast<int64_t>(hq) * nkb + kb) * n_qt + qt) * 4 + kg) * DS_REC) +
                        8 * lane;
#pragma unroll
        for (int us = 0; us < 2; ++us)
#pragma unroll
          for (int sh = 0; sh < 2; ++sh)
            // non-temporal: the records are read once, by the dQ pass after this one
            __builtin_nontemporal_store(__builtin_bit_cast(u32x4, dsb[us][sh]),
                                        reinterpret_cast<u32x4*>(rec + (2 * us + sh) * 512));
      }
      // dK += dS^T Q (the scale is applied once, at the end).
      bf16x8 ft = tr_frag_at(qp, 0, 0, o, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int nb = i & 3, s = (i >> 2) & 1, us = i >> 3;
        bf16x8 nt = ft;
        if (i + 1 < 16) {
          const int j = i + 1;
          nt = tr_frag_at(qp, 32 * (j >> 3), (j >> 2) & 1, o, j & 3);
        }
        acc[nb] = mfma(dsb[us][s], ft, acc[nb]);
        ft = nt;
      }
    }
    if (cur) {
      // dP = dO V^T for both halves, interleaved, fragments one step ahead.
      dpa[0] = f32x16{};
      dpa[1] = f32x16{};
      bf16x8 fd = row_frag_at(dt, 0, o, 0);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int us = i & 1, kk = i >> 1;
        bf16x8 nd = fd;
        if (i + 1 < 16) nd = row_frag_at(dt, 32 * ((i + 1) & 1), o, (i + 1) >> 1);
        dpa[us] = mfma(fd, kvf[kk], dpa[us]);
        fd = nd;
      }
    }
    if constexpr (!SPILL) __builtin_amdgcn_s_setprio(0);
  };

  // Iteration it (0 .. n_it): DMA of tile it + 1 into set (qn, dn, lsen, deln); the P
  // wave does tile it from set (qc, dc, lsec); the D wave finishes tile it - 1 from set
  // (qp, delp) and starts tile it from dc. Each role has its own loop (so neither keeps
  // the other's registers live); both pass the same barriers.
  auto iter = [&](int it, const uint16_t* qc, const uint16_t* dc, const float* lsec,
                  uint16_t* qn, uint16_t* dn, float* lsen, float* deln, const uint16_t* qp,
                  const float* delp, auto is_p) __attribute__((always_inline)) {
    if (it + 1 < n_it) issue_tile(u_begin + it + 1, qn, dn);
    if constexpr (decltype(is_p)::value) {
      if (it < n_it) p_tile(u_begin + it, qc, dc, lsec, it & 1);
    } else {
      d_tile(it > 0, qp, delp, (it + 1) & 1, it < n_it, dc, u_begin + it - 1);
    }
    if (SPILL && !decltype(is_p)::value) {
      // A D wave staged nothing and writes no LDS; its LDS reads fed its products.
      // It leaves its dS stores in flight.
      phase_barrier();
    } else {
      wait_dma();  // the next tile has landed (this wave's part); P is written
      if (it + 1 < n_it) store_rows(lsen, deln);
      if constexpr (SPILL) phase_barrier();
      else __syncthreads();
    }
  };
  auto loop = [&](auto is_p) __attribute__((always_inline)) {
    for (int it = 0; it <= n_it; it += 6) {
      iter(it, s_q0, s_d0, s_lse0, s_q1, s_d1, s_lse1, s_del1, s_q2, s_del2, is_p);
      if (it + 1 > n_it) break;
      iter(it + 1, s_q1, s_d1, s_lse1, s_q2, s_d0, s_lse2, s_del2, s_q0, s_del0, is_p);
      if (it + 2 > n_it) break;
      iter(it + 2, s_q2, s_d0, s_lse2, s_q0, s_d1, s_lse0, s_del0, s_q1, s_del1, is_p);
      if (it + 3 > n_it) break;
      iter(it + 3, s_q0, s_d1, s_lse0, s_q1, s_d0, s_lse1, s_del1, s_q2, s_del2, is_p);
      if (it + 4 > n_it) break;
      iter(it + 4, s_q1, s_d0, s_lse1, s_q2, s_d1, s_lse2, s_del2, s_q0, s_del0, is_p);
      if (it + 5 > n_it) break;
      iter(it + 5, s_q2, s_d1, s_lse2, s_q0, s_d0, s_lse0, s_del0, s_q1, s_del1, is_p);
    }
  };
  if (pwave) loop(std::true_type{});
  else loop(std::false_type{});

  // Write out: register r holds key row m = 8(r/4) + 4h2 + r%4 of this key group,
  // column 32nb + col of d. The P wave owns dV, the D wave dK.
  const float mul = pwave ? 1.0f : a.scale;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = 8 * (r >> 2) + 4 * h2 + (r & 3);
    const int64_t out = s_grow[32 * kg + m];
    if (out < 0) continue;
    if (n_parts == 1) {
      float* row = (pwave ? a.pool.dv_pool : a.pool.dk_pool) + out * D;
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) row[32 * nb + col] += acc[nb][r] * mul;
    } else {
      float* pk = part + ((static_cast<int64_t>(split) * a.pool.Hkv + g) * part_keys + out) * (2 * D) +
                  (pwave ? D : 0);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) pk[32 * nb + col] = acc[nb][r] * mul;
    }
  }
}

// Adds the split partials of every attended key row from k_first on (the rows of the
// split key blocks), in split order, into the gradient pool. One wavefront per (key,
// KV head); lanes over d.
__global__ __launch_bounds__(256) void dkdv_merge_kernel(AttnArgs a, int n_split, const float* part,
                                                         int part_keys, int k_first) {
  const int lane = threadIdx.x & 63;
  const int kidx = k_first + blockIdx.x * 4 + (threadIdx.x >> 6);
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

// Query-stream splits of the dK/dV pass, chosen for load balance: a workgroup's work
// is G times the query tiles its key block can see (all of them for prior pages, fewer
// for the chunk's own pages). The splits are doubled while the largest unit (a prior
// block's share) is more than a quarter of the average work per CU and would stay at
// least 64 tiles, so that longest-first list scheduling over the CUs ends evenly. The
// CU count is fixed at the MI355X's 256, which keeps the choice, and so the result
// bits and the workspace size, independent of the device.
SplitPlan dkdv_plan(const AttnArgs& a) {
  const int64_t n_kb = (static_cast<int64_t>(a.max_att_pages) * a.pool.P + mf::KPW - 1) / mf::KPW;
  SplitPlan forced;
  if (plan_override("OOMB_DKDV_SPLITS", "OOMB_DKDV_WHOLE", static_cast<int>(n_kb), &forced))
    return forced;
  const int G = a.pool.Hq / a.pool.Hkv;
  const int n_qt = (a.n_q + mf::QTB - 1) / mf::QTB;
  const int64_t P = a.pool.P;
  const int64_t n_keys = static_cast<int64_t>(a.max_att_pages) * P;
  const int64_t local0 = static_cast<int64_t>(a.max_att_pages - a.n_local) * P;
  const int64_t nkb = (n_keys + mf::KPW - 1) / mf::KPW;
  double total = 0.0, largest = 0.0;
  int64_t n_largest = 0;  // leading blocks (prior keys) that see every query tile
  for (int64_t kb = 0; kb < nkb; ++kb) {
    // the query tiles of key block kb, as the kernel bounds them
    const int64_t k0 = kb * mf::KPW;
    const int64_t pos0 = static_cast<int64_t>(a.first_local) * P - local0;  // position of index 0
    int64_t qt0 = 0, qt_end = n_qt;
    if (k0 >= local0 || a.window > 0) qt0 = pos0 + k0 > a.t0 ? (pos0 + k0 - a.t0) / mf::QTB : 0;
    if (a.window > 0) {
      const int64_t last = (k0 + mf::KPW < n_keys ? k0 + mf::KPW : n_keys) - 1;
      const int64_t lim = pos0 + last + a.window - 1 - a.t0;
      qt_end = lim < 0 ? 0 : (lim / mf::QTB + 1 < n_qt ? lim / mf::QTB + 1 : n_qt);
    }
    const double t = static_cast<double>(G) * (qt_end > qt0 ? qt_end - qt0 : 0);
    total += t;
    if (t > largest) {
      largest = t;
      n_largest = 0;
    }
    if (t == largest && n_largest == kb) ++n_largest;
  }
  const double per_cu = total * a.pool.Hkv / 256.0;
  int ns = 1;
  while (ns < 8 && largest / ns > per_cu / 4.0 && largest / (2 * ns) >= 64.0) ns *= 2;
  // Cutting every block is more than balance needs when the longest blocks (the prior
  // keys, seen by every query tile) fill a whole number of rounds of the 256 CUs: those
  // run whole, one per CU and round, adding into the pool with no partials, and only
  // the rest (the chunk's own blocks, and prior blocks beyond whole rounds) are cut
  // into ns parts, their pieces filling in behind. Without a window only.
  int whole = 0;
  if (ns > 1 && a.window <= 0 && 256 % a.pool.Hkv == 0)
    whole = static_cast<int>((n_largest * a.pool.Hkv / 256) * 256 / a.pool.Hkv);
  return SplitPlan{ns, whole};
}

size_t dkdv_partial_bytes(const AttnArgs& a, SplitPlan p) {
  const int n_split = p.n_ks;
  if (n_split <= 1) return 0;
  const size_t keys = static_cast<size_t>(a.max_att_pages) * a.pool.P;
  return static_cast<size_t>(n_split) * a.pool.Hkv * keys * 2 * mf::D * sizeof(float);
}

// The dS spill takes 2 bytes per (query, attended key) pair of every 64-query tile and
// 128-key block, and replaces the dQ pass's recomputation of S and dP (6 D of its 8 D
// flops per pair) by a read of those bytes. It is used without a window (where every
// tile of the chunk's rectangle is visited) while the workspace stays within
// OOMB_DS_SPILL_MAX_MIB (default 32768 MiB; 0 turns the spill off), read at every call
// like the split variables.
size_t ds_spill_bytes(const AttnArgs& a) {
  if (a.window > 0) return 0;
  size_t cap = static_cast<size_t>(32768) << 20;
  if (const char* v = getenv("OOMB_DS_SPILL_MAX_MIB")) {
    const long long mib = atoll(v);
    cap = mib > 0 ? static_cast<size_t>(mib) << 20 : 0;
  }
  const size_t nkb = (static_cast<size_t>(a.max_att_pages) * a.pool.P + mf::KPW - 1) / mf::KPW;
  const size_t n_qt = (static_cast<size_t>(a.n_q) + mf::QTB - 1) / mf::QTB;
  const size_t bytes = static_cast<size_t>(a.pool.Hq) * nkb * n_qt * 4 * mf::DS_REC * sizeof(uint16_t);
  return bytes <= cap ? bytes : 0;
}

hipError_t launch_bwd_mfma(const AttnArgs& a, SplitPlan kv, float* part, SplitPlan dq,
                           float* dq_part, uint16_t* ds, hipStream_t s) {
  hipError_t err;
  if (ds == nullptr) {
    // The dQ pass also computes Delta and stores it for the dK/dV pass.
    if ((err = launch_dq_mfma(a, dq, dq_part, nullptr, s)) != hipSuccess) return err;
  } else if ((err = launch_delta_mfma(a, s)) != hipSuccess) {
    return err;
  }
  const int nkb = (a.max_att_pages * a.pool.P + mf::KPW - 1) / mf::KPW;
  const int part_keys = a.max_att_pages * a.pool.P;
  const dim3 grid(a.pool.Hkv * plan_units(kv, nkb));
  if (ds == nullptr) {
    OOMB_LAUNCH("dkdv_mfma", mf::dkdv_mfma_kernel<false>, grid, dim3(64 * mf::DKV_WAVES), 0, s,
                a, kv.n_ks, kv.whole, part, part_keys, nullptr);
  } else {
    OOMB_LAUNCH("dkdv_mfma", mf::dkdv_mfma_kernel<true>, grid, dim3(64 * mf::DKV_WAVES), 0, s,
                a, kv.n_ks, kv.whole, part, part_keys, ds);
  }
  const int k_first = kv.whole * mf::KPW;  // keys of the blocks that ran whole are done
  if (kv.n_ks > 1 && k_first < part_keys) {
    dim3 mgrid((part_keys - k_first + 3) / 4, a.pool.Hkv);
    OOMB_LAUNCH("dkdv_merge", mf::dkdv_merge_kernel, mgrid, dim3(256), 0, s, a, kv.n_ks, part,
                part_keys, k_first);
  }
  if (ds != nullptr && (err = launch_dq_mfma(a, dq, dq_part, ds, s)) != hipSuccess) return err;
  return hipGetLastError();
}

}  // namespace oomb
