// Matrix-core forward of paged chunk attention (online softmax over the attended
// key blocks; writes O and the log-sum-exp the backward recomputes P from).
//
// A workgroup is 8 wavefronts and owns 256 queries of one head, 32 per wavefront;
// wavefronts w and w + 4 share a SIMD. Each wavefront alternates two kinds of phase:
//   M(b): O^T += V_b^T P_b^T and S_{b+1}^T = K_{b+1} Q^T   (matrix cores, LDS reads)
//   V(b): mask, row max, lazy rescale, P_b = exp2(S_b - m)  (vector ALU)
// and the second group (waves 4..7) runs one phase behind the first, so on every SIMD
// one wavefront is in an M phase while the other is in a V phase ("ping-pong"). A
// barrier ends every phase. K and V blocks of 64 keys arrive by global -> LDS DMA four
// phases ahead of their first use, in triple buffers whose roles are static in each of
// the six phases of the loop body: no read ever waits for a DMA into a buffer it does
// not read, and each wave waits only for its batch of two phases ago.
//
// A query tile's key blocks may be cut into n_ks equal ranges, one workgroup each, for
// load balance; each range then writes its unnormalised fp32 O with its running
// maximum and sum, and a merge kernel combines them in range order. With `whole` > 0
// only the tiles after the first `whole` of each KV head (in longest-first order) are
// cut; the first ones run whole and write O directly.
#include <type_traits>

#include "mfma_tiles.hpp"

namespace oomb {
namespace mf {

constexpr int FWD_WAVES = 8;
constexpr int FWD_Q = 32 * FWD_WAVES;  // queries per workgroup

// Page ids held in LDS: all of them when a head attends at most FWD_CAP pages (no window
// slides, and no slide code in the loop), else a window of PCAP that slides.
constexpr int FWD_CAP = 8192;

template <int CAP, bool SLIDE>
__global__ __launch_bounds__(64 * FWD_WAVES) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_mfma_kernel(AttnArgs a, int n_ks, int whole, float* part, float* part_ml) {
  __shared__ __attribute__((aligned(16))) uint16_t s_k0[KB * D];
  __shared__ __attribute__((aligned(16))) uint16_t s_k1[KB * D];
  __shared__ __attribute__((aligned(16))) uint16_t s_k2[KB * D];
  __shared__ __attribute__((aligned(16))) uint16_t s_v0[KB * D];
  __shared__ __attribute__((aligned(16))) uint16_t s_v1[KB * D];
  __shared__ __attribute__((aligned(16))) uint16_t s_v2[KB * D];
  __shared__ int s_page[CAP];
  constexpr int NT = 64 * FWD_WAVES;
  // the wave index is uniform: keep it (and the LDS addresses built from it) scalar
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;  // 0: leading group, 1: one phase behind
  const int h2 = lane >> 5, col = lane & 31;
  const int G = a.pool.Hq / a.pool.Hkv;
  const int n_qt = (a.n_q + FWD_Q - 1) / FWD_Q;
  // A KV head's units: tiles j in longest-first order (latest query tiles, with the most
  // local keys, first; then the group's heads), the first `whole` whole, each later
  // one as n_ks consecutive key ranges.
  const HeadUnit hu = head_unit(blockIdx.x, gridDim.x, a.pool.Hkv);
  const TileRange tr = tile_range(hu.unit, whole, n_ks);
  const int g = hu.head, krange = tr.range, n_rng = tr.n_ranges;
  const int hh = tr.tile % G, qt = n_qt - 1 - tr.tile / G;
  const int h = g * G + hh;
  const Keys km = make_keys(a, g);
  const int q0 = qt * FWD_Q;
  // Key blocks of the tile: from the first one its first query sees (0 without a
  // window) to the last one its last query sees.
  const int blo_tile = first_block(km, a.t0 + q0);
  const int nb_tile = n_blocks(km, a.t0 + min(a.n_q, q0 + FWD_Q) - 1);
  const int span = max(0, nb_tile - blo_tile);
  // This workgroup's blocks are b0 .. b0 + nb - 1; below, block indices are relative
  // to b0 and made absolute (b0 + .) wherever keys are addressed or masked.
  const int b0 = blo_tile + span * krange / n_rng, nb = blo_tile + span * (krange + 1) / n_rng - b0;
  const float c2 = a.scale * kLog2e;

  // This wave's queries: blocks past its last query, or (with a window) before its
  // first query's window, are skipped; blocks reaching past its first query, or below
  // its last query's window, need the mask.
  const int wq0 = q0 + 32 * wave;
  const int wq_last = min(a.n_q, wq0 + 32) - 1;
  const int nblk_w = min(nb, max(0, (wq_last < wq0 ? 0 : n_blocks(km, a.t0 + wq_last)) - b0));
  const int blo_w = max(0, first_block(km, a.t0 + wq0) - b0);
  const int klim_w0 = km.klim(a.t0 + wq0);
  const int klo_wl = km.klo(a.t0 + wq_last);

  // This lane's query (column of S^T) and its Q fragments (B operand over d).
  const int i = wq0 + col;
  const int klim = km.klim(a.t0 + i), klo = km.klo(a.t0 + i);
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
  f32x16 st[2];     // S^T of the block last multiplied: from its M phase to its V phase
  bf16x8 pb[2][2];  // P^T of the block last normalised: from its V phase to the next M phase
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    st[sub] = f32x16{};
    pb[sub][0] = pb[sub][1] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  }

  FragOffsets fo;
  fo.init(lane);
  const uint16_t* kpool = static_cast<const uint16_t*>(a.pool.k_pool);
  const uint16_t* vpool = static_cast<const uint16_t*>(a.pool.v_pool);
  // All 8 waves stage the first blocks; afterwards each group of 4 stages one tensor.
  // With every page id resident the window starts at entry 0, else at block b0's.
  const int win0 = SLIDE ? (b0 * KB) >> km.log2p : 0;
  KeyStage<KB, FWD_WAVES, CAP> ks{km, s_page, win0,
                                  KeyStage<KB, FWD_WAVES, CAP>::lane_offset(wave, lane)};
  KeyStage<KB, 4, CAP> kg{km, s_page, win0, KeyStage<KB, 4, CAP>::lane_offset(wave & 3, lane)};
  fill_pages<NT, CAP>(km, s_page, win0, tid);
  zero_tile<KB, NT>(s_v1, tid);  // read (times a zero P^T) before their first DMA
  zero_tile<KB, NT>(s_v2, tid);
  wait_dma();  // the page-table loads are retired here, not at a later register reuse
  __syncthreads();
  // K_0, K_1 and V_0 before the first phase; every later block arrives four phases
  // ahead of its first use.
  ks.issue_fixed(b0, kpool, s_k0, wave, lane);
  ks.issue_fixed(b0 + 1, kpool, s_k1, wave, lane);
  ks.issue_fixed(b0, vpool, s_v0, wave, lane);
  wait_dma();
  __syncthreads();

  // Both products of an M phase as one software pipeline of eight steps of four MFMAs:
  // four PV steps (one k-step of one 32-key half each) then four S steps (k-steps 2i and
  // 2i + 1 of both halves, alternating halves so that consecutive MFMAs are
  // independent). The fragments of step i + 1 are read from LDS while step i multiplies.
  auto mul_pv_s = [&](const uint16_t* vt, const uint16_t* kt) __attribute__((always_inline)) {
    fo.opaque();
    const FragOffsets& o = fo;
    auto load = [&](int i, bf16x8 (&f)[4]) __attribute__((always_inline)) {
      if (i < 4) {
#pragma unroll
        for (int db = 0; db < 4; ++db) f[db] = tr_frag_at(vt, 32 * (i >> 1), i & 1, o, db);
      } else {
        const int kk = 2 * (i - 4);
        f[0] = row_frag_at(kt, 0, o, kk);
        f[1] = row_frag_at(kt, 32, o, kk);
        f[2] = row_frag_at(kt, 0, o, kk + 1);
        f[3] = row_frag_at(kt, 32, o, kk + 1);
      }
    };
    auto mul = [&](int i, const bf16x8 (&f)[4]) __attribute__((always_inline)) {
      if (i < 4) {
#pragma unroll
        for (int db = 0; db < 4; ++db) ot[db] = mfma(f[db], pb[i >> 1][i & 1], ot[db]);
      } else {
        const int kk = 2 * (i - 4);
        if (i == 4) {
          st[0] = f32x16{};
          st[1] = f32x16{};
        }
        st[0] = mfma(f[0], qf[kk], st[0]);
        st[1] = mfma(f[1], qf[kk], st[1]);
        st[0] = mfma(f[2], qf[kk + 1], st[0]);
        st[1] = mfma(f[3], qf[kk + 1], st[1]);
      }
    };
    bf16x8 fa[4], fb[4];
    load(0, fa);
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      load(i + 1, fb);
      mul(i, fa);
      if (i + 2 < 8) load(i + 2, fa);
      mul(i + 1, fb);
    }
  };
  // Softmax numerator of block b from st into pb.
  auto softmax = [&](int b) __attribute__((always_inline)) {
    const int k0 = (b0 + b) * KB;  // first key of the block
    // Causal / tail mask (and window mask), only in blocks that reach past this wave's
    // first query (or below its last query's window).
    if (k0 + KB - 1 > klim_w0 || k0 < klo_wl) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * sub + 8 * (r >> 2) + 4 * h2 + (r & 3);
          st[sub][r] = ((key > klim) | (key < klo)) ? -__builtin_inff() : st[sub][r];
        }
    }
    // Row maximum: four independent chains, then the other half-wave's rows.
    float mx4[4] = {st[0][0], st[0][1], st[0][2], st[0][3]};
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (sub || r >= 4) mx4[r & 3] = fmaxf(mx4[r & 3], st[sub][r]);
    float mx = fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3]));
    mx = max_halves(mx) * c2;
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
    float ls[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // partial row sums (short dependency chains)
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          p[j] = fast_exp2(__builtin_fmaf(st[sub][8 * s + j], c2, -mref));
          ls[j & 3] += p[j];
        }
        pb[sub][s] = pack8(p);
      }
    l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
  };

  // Phase t, j = t / 2. DMA duties, always in the wave's V phase: at even t the second
  // group stages K_{j+2} into kd, at odd t the first group stages V_{j+1} into vd, a
  // fixed number of instructions each, and each wave waits (at the end of each phase in
  // which it issued) for all but the batch it just issued. A wave's own phase index is
  // u = t - grp: u = 0 computes S_0; odd u runs V(u / 2); even u >= 2 runs M(u / 2 - 1).
  // kr / vr hold K_{b+1} / V_b of whichever M phase runs. Block j's K and V live in
  // buffer j % 3. IS_M and G1 (compile time) make every phase straight-line code.
  int pid[KeyStage<KB, 4, CAP>::NI];  // page ids of this wave's next DMA duty
  auto phase = [&](auto is_m, auto g1, int t, uint16_t* kd, uint16_t* vd, const uint16_t* kr,
                   const uint16_t* vr) __attribute__((always_inline)) {
    constexpr bool kG1 = decltype(g1)::value;
    const int j = t >> 1;
    if constexpr (SLIDE) {
      if ((t & 1) == 0) {
        const int last_e = ((b0 + min(nb, j + 3)) * KB - 1) >> km.log2p;
        if (j + 1 < nb && last_e >= ks.win + CAP) {  // uniform: slide the page window
          ks.win = kg.win = ((b0 + j + 1) * KB) >> km.log2p;
          fill_pages<NT, CAP>(km, s_page, ks.win, tid);
          wait_dma();
          __syncthreads();
        }
      }
    }
    // DMA duty. Its page ids are LDS reads, which queue behind the M phases' tile reads:
    // with every page id resident they are read one duty ahead; with a sliding window,
    // at the start of the phase. The DMA itself is issued after this wave's softmax.
    const bool dma = kG1 ? (t & 1) == 0 : (t & 1) == 1;
    const int dst = b0 + (kG1 ? j + 2 : j + 1);  // absolute block
    if constexpr (SLIDE) {
      if (dma) kg.read_pages(dst, wave & 3, pid);
    }
    const int u = t - grp;
    if constexpr (decltype(is_m)::value) {
      const int b = (u >> 1) - 1;  // M(b): PV of block b, S of block b + 1
      if (u >= 0) {
        // The M phase, the longer of the two, issues at raised priority. (While the DMA
        // duty cost a V phase more cycles than the products, raising the softmax instead
        // was faster.)
        __builtin_amdgcn_s_setprio(1);
        // M(-1) multiplies the zero P^T by the zero-filled V buffer (adds exact zeros);
        // M(nblk_w - 1) computes an S^T no softmax will read. Before this wave's first
        // block (a window) P^T is still zero: M(blo_w - 1) only computes S^T of blo_w.
        if (b < nblk_w && b + 1 >= blo_w) mul_pv_s(vr, kr);
        __builtin_amdgcn_s_setprio(0);
      }
    } else {
      const int b = u >> 1;
      if (u >= 0 && b < nblk_w && b >= blo_w) softmax(b);
    }
    if (dma) {
      __builtin_amdgcn_sched_barrier(0);
      kg.dma_fixed(dst, kG1 ? kpool : vpool, kG1 ? kd : vd, wave & 3, lane, pid);
      if constexpr (!SLIDE) kg.read_pages(dst + 1, wave & 3, pid);  // the next duty's
      wait_vm<KeyStage<KB, 4, CAP>::NI>();  // the batch of two phases ago has landed
    }
    phase_barrier();
  };
  using M = std::integral_constant<bool, true>;
  using V = std::integral_constant<bool, false>;
  const int T = 2 * nb + 2;
  if constexpr (!SLIDE) kg.read_pages(b0 + (grp ? 2 : 1), wave & 3, pid);  // first duty: K_2 / V_1
  if (grp == 0) {
    using G = std::integral_constant<bool, false>;
    for (int t = 0; t < T; t += 6) {
      phase(M{}, G{}, t + 0, s_k2, nullptr, s_k0, s_v2);
      phase(V{}, G{}, t + 1, nullptr, s_v1, s_k0, s_v2);
      phase(M{}, G{}, t + 2, s_k0, nullptr, s_k1, s_v0);
      phase(V{}, G{}, t + 3, nullptr, s_v2, s_k1, s_v0);
      phase(M{}, G{}, t + 4, s_k1, nullptr, s_k2, s_v1);
      phase(V{}, G{}, t + 5, nullptr, s_v0, s_k2, s_v1);
    }
  } else {
    using G = std::integral_constant<bool, true>;
    for (int t = 0; t < T; t += 6) {
      phase(V{}, G{}, t + 0, s_k2, nullptr, s_k0, s_v2);
      phase(M{}, G{}, t + 1, nullptr, s_v1, s_k0, s_v2);
      phase(V{}, G{}, t + 2, s_k0, nullptr, s_k1, s_v0);
      phase(M{}, G{}, t + 3, nullptr, s_v2, s_k1, s_v0);
      phase(V{}, G{}, t + 4, s_k1, nullptr, s_k2, s_v1);
      phase(M{}, G{}, t + 5, nullptr, s_v0, s_k2, s_v1);
    }
  }
  wait_dma();  // no DMA may outlive the workgroup's LDS

  // Epilogue: O = O^T / l, LSE = (m + log2 l) ln 2; or this key range's partial.
  const float lt = add_halves(l_run);
  if (n_rng > 1) {
    if (i < a.n_q) {
      const int64_t row = (static_cast<int64_t>(krange) * a.pool.Hq + h) * a.n_q + i;
      float* prow = part + row * D;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int ga = 0; ga < 4; ++ga) {
          f32x4 w;
#pragma unroll
          for (int b2 = 0; b2 < 4; ++b2) w[b2] = ot[db][4 * ga + b2];
          *reinterpret_cast<f32x4*>(prow + 32 * db + 8 * ga + 4 * h2) = w;
        }
      if (h2 == 0) *reinterpret_cast<f32x2*>(part_ml + 2 * row) = f32x2{m_run, lt};
    }
    return;
  }
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

// O and LSE from the key ranges' partials: with M the largest running maximum (log2
// units), w_r = 2^(m_r - M), O = sum_r w_r O_r / sum_r w_r l_r and
// LSE = (M + log2 sum_r w_r l_r) ln 2, the ranges taken in order. One thread per 4
// columns of a row.
__global__ __launch_bounds__(256) void fwd_merge_kernel(AttnArgs a, int n_ks, int whole,
                                                        const float* part, const float* part_ml) {
  const int64_t rows = static_cast<int64_t>(a.pool.Hq) * a.n_q;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= rows * (D / 4)) return;
  const int64_t row = idx / (D / 4);
  const int c = static_cast<int>(idx % (D / 4)) * 4;
  if (!row_was_split(a, row, FWD_Q, whole)) return;  // its tile ran whole and wrote O
  float mx = -__builtin_inff();
  for (int k = 0; k < n_ks; ++k) mx = fmaxf(mx, part_ml[2 * (k * rows + row)]);
  float l = 0.0f;
  f32x4 o = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  for (int k = 0; k < n_ks; ++k) {
    const f32x2 ml = *reinterpret_cast<const f32x2*>(part_ml + 2 * (k * rows + row));
    const float w = ml[0] == -__builtin_inff() ? 0.0f : exp2f(ml[0] - mx);  // empty range: 0
    l += w * ml[1];
    const f32x4 v = *reinterpret_cast<const f32x4*>(part + (k * rows + row) * D + c);
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] += w * v[j];
  }
  const float inv = 1.0f / l;
  const int h = static_cast<int>(row / a.n_q), i = static_cast<int>(row % a.n_q);
  uint16_t* orow = static_cast<uint16_t*>(a.o) + h * a.o_hs + static_cast<int64_t>(i) * a.o_ts;
  u32x2 w2;
  w2[0] = pack_bf16x2(o[0] * inv, o[1] * inv);
  w2[1] = pack_bf16x2(o[2] * inv, o[3] * inv);
  *reinterpret_cast<u32x2*>(orow + c) = w2;
  if (c == 0) a.lse[row] = (mx + __log2f(l)) * kLn2;
}

}  // namespace mf

// Key ranges per query tile of the forward, chosen for load balance: a tile's work is
// its key blocks. The ranges are halved while the largest is more than a quarter of
// the average work per CU (256 CUs, one workgroup each, fixed so the choice and the
// result bits do not depend on the device) and would stay at least 128 blocks: a CU
// runs one forward workgroup at a time, so each one's start-up (query fragments, page
// list, first key blocks) is exposed, and shorter ranges cost more than they balance.
// When the tiles are cut and their count is not a multiple of the CU count,
// mixed_plan cuts only those beyond a whole number per CU (see launch.hpp).
SplitPlan fwd_plan(const AttnArgs& a) {
  const int n_qt = (a.n_q + mf::FWD_Q - 1) / mf::FWD_Q;
  const int G = a.pool.Hq / a.pool.Hkv;
  SplitPlan forced;
  if (plan_override("OOMB_FWD_SPLITS", "OOMB_FWD_WHOLE", G * n_qt, &forced)) return forced;
  double total = 0.0, largest = 0.0, smallest = 1e300;
  for (int qt = 0; qt < n_qt; ++qt) {
    const double blocks = static_cast<double>(tile_key_blocks(a, qt * mf::FWD_Q, mf::FWD_Q, mf::KB));
    total += blocks;
    largest = blocks > largest ? blocks : largest;
    smallest = blocks < smallest ? blocks : smallest;
  }
  const double per_cu = total * a.pool.Hq / 256.0;
  int nk = 1;
  while (nk < 4 && largest / nk > per_cu / 4.0 && largest / (2 * nk) >= 128.0) nk *= 2;
  return mixed_plan(G * n_qt, a.pool.Hkv, smallest, nk);
}

size_t fwd_partial_bytes(const AttnArgs& a, SplitPlan p) {
  if (p.n_ks <= 1) return 0;
  return static_cast<size_t>(p.n_ks) * a.pool.Hq * a.n_q * (mf::D + 2) * sizeof(float);
}

hipError_t launch_fwd_mfma(const AttnArgs& a, SplitPlan p, float* part, hipStream_t s) {
  const int n_qt = (a.n_q + mf::FWD_Q - 1) / mf::FWD_Q;
  const int G = a.pool.Hq / a.pool.Hkv;
  const dim3 grid(a.pool.Hkv * plan_units(p, G * n_qt)), block(64 * mf::FWD_WAVES);
  // partial O [n_ks][Hq][n_q][D], then (m, l) [n_ks][Hq][n_q][2]
  float* part_ml = part ? part + static_cast<size_t>(p.n_ks) * a.pool.Hq * a.n_q * mf::D : nullptr;
  if (a.max_att_pages <= mf::FWD_CAP) {
    OOMB_LAUNCH("fwd_mfma", (mf::fwd_mfma_kernel<mf::FWD_CAP, false>), grid, block, 0, s, a, p.n_ks,
                p.whole, part, part_ml);
  } else {
    OOMB_LAUNCH("fwd_mfma", (mf::fwd_mfma_kernel<mf::PCAP, true>), grid, block, 0, s, a, p.n_ks,
                p.whole, part, part_ml);
  }
  if (p.n_ks > 1) {
    const int64_t threads = static_cast<int64_t>(a.pool.Hq) * a.n_q * (mf::D / 4);
    OOMB_LAUNCH("fwd_merge", mf::fwd_merge_kernel, dim3(static_cast<unsigned>((threads + 255) / 256)),
                dim3(256), 0, s, a, p.n_ks, p.whole, part, part_ml);
  }
  return hipGetLastError();
}

}  // namespace oomb
