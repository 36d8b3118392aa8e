// Matrix-core backward of paged chunk attention, dQ pass: recompute P from the saved
// log-sum-exp and dP = dO V^T per key block, then dQ^T += K^T dS^T. Each lane holds its
// query's dO row anyway, so the pass also forms Delta = dO . O for its rows and stores
// it for the dK/dV pass (no separate pre-pass).
//
// A workgroup is 8 wavefronts and owns 256 queries of one head (32 per wavefront, Q and
// dO fragments held in registers), one workgroup per CU, two wavefronts per SIMD. The
// key blocks are staged once for all 256 queries: LDS writes cost more than their share
// of LDS bytes, and two 4-wave workgroups per CU (each staging its own blocks) ran 5%
// slower. Key blocks of 128 rows (K and V; 64-row blocks, with twice the barriers,
// ran 1.2% slower) are copied global -> LDS by DMA one block
// ahead, a fixed number of instructions per wave, into double buffers whose roles are
// static in each half of the unrolled loop. The page ids a DMA needs
// are read from LDS one block before it is issued, so the read has left the LDS queue
// by then. Fragment reads are software-pipelined one step ahead of the products.
//
// A query tile's key blocks may be cut into n_ks equal ranges, one workgroup each, for
// load balance (the tiles' work differs, and there are few of them per CU); each range
// then writes an fp32 partial dQ and a merge kernel adds them in range order. With
// `whole` > 0 only the tiles after the first `whole` of each KV head (in longest-first
// order) are cut; the first ones run whole and write dQ directly.
#include "mfma_tiles.hpp"

namespace oomb {
namespace mf {

constexpr int DQ_WAVES = 8;
constexpr int DQ_Q = 32 * DQ_WAVES;  // queries per workgroup
constexpr int DQ_KB = 128;           // keys per staged block

// Blocks of DQ_KB keys that queries up to position qmax_pos must visit, and the first
// block a query at position qpos (or any later one) sees.
__device__ __forceinline__ int dq_n_blocks(const Keys& k, int qmax_pos) {
  const int last = k.klim(qmax_pos);
  return last < 0 ? 0 : last / DQ_KB + 1;
}
__device__ __forceinline__ int dq_first_block(const Keys& k, int qpos) {
  const int lo = k.klo(qpos);
  return lo > 0 ? lo / DQ_KB : 0;
}

__global__ __launch_bounds__(64 * DQ_WAVES) __attribute__((amdgpu_waves_per_eu(2)))
void dq_mfma_kernel(AttnArgs a, int n_ks, int whole, float* part) {
  __shared__ __attribute__((aligned(16))) uint16_t s_k0[DQ_KB * D];
  __shared__ __attribute__((aligned(16))) uint16_t s_v0[DQ_KB * D];
  __shared__ __attribute__((aligned(16))) uint16_t s_k1[DQ_KB * D];
  __shared__ __attribute__((aligned(16))) uint16_t s_v1[DQ_KB * D];
  __shared__ int s_page[PCAP];
  constexpr int NT = 64 * DQ_WAVES;
  using Stage = KeyStage<DQ_KB, DQ_WAVES, PCAP>;
  // the wave index is uniform: keep it (and the LDS addresses built from it) scalar
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h2 = lane >> 5, col = lane & 31;
  const int G = a.pool.Hq / a.pool.Hkv;
  const int n_qt = (a.n_q + DQ_Q - 1) / DQ_Q;
  // A KV head's units: tiles j in longest-first order (latest query tiles, with the most
  // local keys, first; then the group's heads), the first `whole` whole, each later
  // one as n_ks consecutive key ranges.
  const HeadUnit hu = head_unit(blockIdx.x, gridDim.x, a.pool.Hkv);
  const TileRange tr = tile_range(hu.unit, whole, n_ks);
  const int g = hu.head, kr = tr.range, n_rng = tr.n_ranges;
  const int hh = tr.tile % G, qt = n_qt - 1 - tr.tile / G;
  const int h = g * G + hh;
  const Keys km = make_keys(a, g);
  const int q0 = qt * DQ_Q;
  const int nblk = dq_n_blocks(km, a.t0 + min(a.n_q, q0 + DQ_Q) - 1);
  const int blo_tile = dq_first_block(km, a.t0 + q0);  // 0 without a window
  const int span = max(0, nblk - blo_tile);
  const int b0 = blo_tile + span * kr / n_rng, b1 = blo_tile + span * (kr + 1) / n_rng;  // this workgroup's blocks
  const float c2 = a.scale * kLog2e;
  // (Both waves of a SIMD run at the same priority: with blocks of 128 keys, raising one
  // of them, which helped at 64, measured 0-0.5% slower.)

  // This wave's queries: blocks past its last query are skipped; blocks reaching past
  // its first query need the mask.
  const int wq0 = q0 + 32 * wave;
  const int wq_last = min(a.n_q, wq0 + 32) - 1;
  const int nblk_w = wq_last < wq0 ? 0 : dq_n_blocks(km, a.t0 + wq_last);
  const int blo_w = dq_first_block(km, a.t0 + wq0);
  const int klim_w0 = km.klim(a.t0 + wq0);
  const int klo_wl = km.klo(a.t0 + wq_last);

  // This lane's query (column of S^T and dP^T) with its Q and dO fragments; lanes col
  // and col + 32 hold alternate 8-element groups of the row (h2 = 0, 1).
  const int i = wq0 + col;
  const int klim = km.klim(a.t0 + i), klo = km.klo(a.t0 + i);
  const bool ok = i < a.n_q;
  bf16x8 qf[8], df[8];
  u32x4 of[8];
  {
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + h * a.q_hs + static_cast<int64_t>(i) * a.q_ts;
    const uint16_t* drow = static_cast<const uint16_t*>(a.dout) + h * a.do_hs + static_cast<int64_t>(i) * a.do_ts;
    const uint16_t* orow = static_cast<const uint16_t*>(a.o) + h * a.o_hs + static_cast<int64_t>(i) * a.o_ts;
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      qf[kk] = as_bf16x8(ok ? *reinterpret_cast<const u32x4*>(qrow + 16 * kk + 8 * h2) : u32x4{0u, 0u, 0u, 0u});
      df[kk] = as_bf16x8(ok ? *reinterpret_cast<const u32x4*>(drow + 16 * kk + 8 * h2) : u32x4{0u, 0u, 0u, 0u});
      of[kk] = ok ? *reinterpret_cast<const u32x4*>(orow + 16 * kk + 8 * h2) : u32x4{0u, 0u, 0u, 0u};
    }
  }
  const int64_t rid = static_cast<int64_t>(h) * a.n_q + i;
  const float lse2 = ok ? a.lse_in[rid] * kLog2e : __builtin_inff();
  // Delta_i = dO_i . O_i in fp32: each lane sums its half of the row in element order,
  // then the two halves are added (the same sum in both lanes, so every unit that holds
  // the row gets the same bits). The first key range of each tile stores it for the
  // dK/dV pass, which runs after this one on the same stream.
  float delta = 0.0f;
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) {
    const bf16x8 ob = as_bf16x8(of[kk]);
#pragma unroll
    for (int e = 0; e < 8; ++e)
      delta = __builtin_fmaf(static_cast<float>(df[kk][e]), static_cast<float>(ob[e]), delta);
  }
  delta += __shfl_xor(delta, 32, 64);
  if (ok && kr == 0 && h2 == 0) a.delta[rid] = delta;

  f32x16 dqt[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) dqt[db] = f32x16{};

  FragOffsets fo;
  fo.init(lane);
  const uint16_t* kpool = static_cast<const uint16_t*>(a.pool.k_pool);
  const uint16_t* vpool = static_cast<const uint16_t*>(a.pool.v_pool);
  const int win0 = (b0 * DQ_KB) >> km.log2p;
  Stage ks{km, s_page, win0, Stage::lane_offset(wave, lane)};
  fill_pages<NT>(km, s_page, win0, tid);
  wait_dma();  // the page-table loads are retired here, not at a later register reuse
  __syncthreads();
  int pid[Stage::NI];  // page ids of the next block's DMA (K and V rows share them)
  if (b0 < b1) {
    ks.read_pages(b0, wave, pid);
    ks.dma_fixed(b0, kpool, s_k0, wave, lane, pid);
    ks.dma_fixed(b0, vpool, s_v0, wave, lane, pid);
  }
  ks.read_pages(b0 + 1, wave, pid);
  wait_dma();
  __syncthreads();

  // One key block b from (kt, vt); DMA of block b + 1 into (kn, vn) first.
  auto block = [&](int b, const uint16_t* kt, const uint16_t* vt, uint16_t* kn,
                   uint16_t* vn) __attribute__((always_inline)) {
    if (b + 1 < b1) {
      const int last_e = ((b + 1) * DQ_KB + DQ_KB - 1) >> km.log2p;
      if (last_e >= ks.win + PCAP) {  // uniform over the workgroup: slide the page window
        ks.win = ((b + 1) * DQ_KB) >> km.log2p;
        fill_pages<NT>(km, s_page, ks.win, tid);
        wait_dma();
        __syncthreads();
        ks.read_pages(b + 1, wave, pid);
      }
      ks.dma_fixed(b + 1, kpool, kn, wave, lane, pid);
      ks.dma_fixed(b + 1, vpool, vn, wave, lane, pid);
      if (b + 2 < b1) {
        const int last2 = ((b + 2) * DQ_KB + DQ_KB - 1) >> km.log2p;
        if (last2 < ks.win + PCAP) ks.read_pages(b + 2, wave, pid);  // else after the slide
      }
    }
    if (b < nblk_w && b >= blo_w) {
      fo.opaque();
      const FragOffsets& o = fo;
      const bool mask = b * DQ_KB + DQ_KB - 1 > klim_w0 || b * DQ_KB < klo_wl;
#pragma unroll
      for (int sub = 0; sub < DQ_KB / 32; ++sub) {
        // S^T = K Q^T and dP^T = V dO^T for 32 keys: two independent chains, fragment
        // reads one k-step ahead.
        f32x16 st = f32x16{}, dpt = f32x16{};
        bf16x8 fk = row_frag_at(kt, 32 * sub, o, 0), fv = row_frag_at(vt, 32 * sub, o, 0);
#pragma unroll
        for (int kk = 0; kk < 8; ++kk) {
          bf16x8 nk = fk, nv = fv;
          if (kk + 1 < 8) {
            nk = row_frag_at(kt, 32 * sub, o, kk + 1);
            nv = row_frag_at(vt, 32 * sub, o, kk + 1);
          }
          st = mfma(fk, qf[kk], st);
          dpt = mfma(fv, df[kk], dpt);
          fk = nk;
          fv = nv;
        }
        // dS^T = P^T (dP^T - Delta), P = exp2(S c - lse log2 e); masked keys give 0
        // (one uniform branch, branch-free inside).
        bf16x8 ta[4];
#pragma unroll
        for (int db = 0; db < 4; ++db) ta[db] = tr_frag_at(kt, 32 * sub, 0, o, db);
#pragma unroll
        for (int r = 0; r < 16; ++r) st[r] = fast_exp2(__builtin_fmaf(st[r], c2, -lse2));
        if (mask) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = b * DQ_KB + 32 * sub + 8 * (r >> 2) + 4 * h2 + (r & 3);
            st[r] = ((key > klim) | (key < klo)) ? 0.0f : st[r];
          }
        }
        bf16x8 dsb[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          float ds[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) ds[j] = st[8 * s + j] * (dpt[8 * s + j] - delta);
          dsb[s] = pack8(ds);
        }
        // dQ^T += K^T dS^T, the second k-step's fragments read during the first's products.
        bf16x8 tb[4];
#pragma unroll
        for (int db = 0; db < 4; ++db) tb[db] = tr_frag_at(kt, 32 * sub, 1, o, db);
#pragma unroll
        for (int db = 0; db < 4; ++db) dqt[db] = mfma(ta[db], dsb[0], dqt[db]);
#pragma unroll
        for (int db = 0; db < 4; ++db) dqt[db] = mfma(tb[db], dsb[1], dqt[db]);
      }
    }
    wait_vm<0>();     // block b + 1 has landed (this wave's part) ...
    phase_barrier();  // ... everyone's, and nobody reads block b any more
  };
  // Unrolled by two so that each half names its read and write buffers statically.
  for (int b = b0; b < b1; b += 2) {
    block(b, s_k0, s_v0, s_k1, s_v1);
    if (b + 1 < b1) block(b + 1, s_k1, s_v1, s_k0, s_v0);
  }

  if (i < a.n_q) {
    // the whole dQ row, or this key range's partial of it
    float* drow = n_rng == 1 ? a.dq + h * a.dq_hs + static_cast<int64_t>(i) * a.dq_ts
                            : part + ((static_cast<int64_t>(kr) * a.pool.Hq + h) * a.n_q + i) * D;
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

// dQ = the sum of the key ranges' partials, in range order. One thread per 4 columns
// of a row.
__global__ __launch_bounds__(256) void dq_merge_kernel(AttnArgs a, int n_ks, int whole,
                                                       const float* part) {
  const int64_t rows = static_cast<int64_t>(a.pool.Hq) * a.n_q;
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= rows * (D / 4)) return;
  const int64_t row = idx / (D / 4);
  if (!row_was_split(a, row, DQ_Q, whole)) return;  // its tile ran whole and wrote dQ
  const int c = static_cast<int>(idx % (D / 4)) * 4;
  f32x4 s = *reinterpret_cast<const f32x4*>(part + row * D + c);
  for (int k = 1; k < n_ks; ++k) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(part + (k * rows + row) * D + c);
#pragma unroll
    for (int j = 0; j < 4; ++j) s[j] += v[j];
  }
  const int h = static_cast<int>(row / a.n_q), i = static_cast<int>(row % a.n_q);
  *reinterpret_cast<f32x4*>(a.dq + h * a.dq_hs + static_cast<int64_t>(i) * a.dq_ts + c) = s;
}

// Delta_i = dO_i . O_i for the backward that spills dS, formed in the order the
// recomputing dQ pass uses (each half of the row, 8-element groups 16 kk + 8 half .. +7
// in element order by fused multiply-adds, then the two halves added), so that both
// backward paths give the dK/dV pass the same Delta bits and so the same dK and dV.
// Two lanes per row.
__global__ __launch_bounds__(256) void delta_mfma_kernel(AttnArgs a) {
  const int64_t t = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t row = t >> 1;
  const int half = static_cast<int>(t & 1);
  const bool ok = row < static_cast<int64_t>(a.pool.Hq) * a.n_q;
  const int h = ok ? static_cast<int>(row / a.n_q) : 0, i = ok ? static_cast<int>(row % a.n_q) : 0;
  const uint16_t* dr = static_cast<const uint16_t*>(a.dout) + h * a.do_hs + static_cast<int64_t>(i) * a.do_ts;
  const uint16_t* orow = static_cast<const uint16_t*>(a.o) + h * a.o_hs + static_cast<int64_t>(i) * a.o_ts;
  float acc = 0.0f;
  if (ok) {
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const u32x4 dv = *reinterpret_cast<const u32x4*>(dr + 16 * kk + 8 * half);
      const u32x4 ov = *reinterpret_cast<const u32x4*>(orow + 16 * kk + 8 * half);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc = __builtin_fmaf(__uint_as_float(dv[w] << 16), __uint_as_float(ov[w] << 16), acc);
        acc = __builtin_fmaf(__uint_as_float(dv[w] & 0xFFFF0000u), __uint_as_float(ov[w] & 0xFFFF0000u), acc);
      }
    }
  }
  acc += __shfl_xor(acc, 1, 64);
  if (ok && half == 0) a.delta[row] = acc;
}

// ============================================================================ dQ from dS
// When the dK/dV pass has spilled its dS tiles (see dkdv_mfma_kernel), dQ needs no
// recomputation: dQ^T = scale K^T dS^T, one product per key block with K from the pool
// and dS^T from the spill. The work units, key ranges and partials are those of
// dq_mfma_kernel (256 queries of one head per workgroup, one workgroup per CU), over
// stages of 64 keys: K rows (a swizzled row-major tile) and the spilled record blocks
// arrive by DMA two stages ahead, into triple buffers. This pass streams the spill
// once, so HBM bandwidth bounds it.
//
// Wave w owns the 64-query tile jq = w % 4 and key half kh = w / 4 of every stage (the
// key group 2 (b % 2) + kh of the spill): dQ^T of its 64 queries over all 128 d columns
// (two query halves x four column blocks, 128 accumulators a lane), from 8 transposed K
// fragments and 4 dS^T fragments per stage for 16 products. It stages its own record
// block (4 KiB), in which a lane holds one key and runs of four consecutive queries
// (8 bytes): ds_read_b64_tr_b16 gathers exactly the B operand (a lane per query, keys
// along it) from those runs, source lane 4k + m reading key k's run 4m .. 4m + 3, in the
// key order of the transposed K fragment. Records land in LDS with their lane index
// XORed by 4 ((l / 32) | 2 (p % 2)), which makes every half-wave of those reads
// conflict-free. The two key halves' sums are added through LDS at the end.
constexpr int DQS_KB = 64;  // keys per stage

// LDS slot of spilled record lane l in pack p (an involution: bit 5 is kept).
__device__ __forceinline__ int ds_slot(int p, int l) { return l ^ (4 * ((l >> 5) | ((p & 1) << 1))); }

__global__ __launch_bounds__(64 * DQ_WAVES) __attribute__((amdgpu_waves_per_eu(2)))
void dqs_mfma_kernel(AttnArgs a, int n_ks, int whole, float* part, const uint16_t* ds) {
  __shared__ __attribute__((aligned(16))) uint16_t s_k0[DQS_KB * D];
  __shared__ __attribute__((aligned(16))) uint16_t s_k1[DQS_KB * D];
  __shared__ __attribute__((aligned(16))) uint16_t s_k2[DQS_KB * D];
  __shared__ __attribute__((aligned(16))) uint16_t s_s0[DQ_WAVES * DS_REC];
  __shared__ __attribute__((aligned(16))) uint16_t s_s1[DQ_WAVES * DS_REC];
  __shared__ __attribute__((aligned(16))) uint16_t s_s2[DQ_WAVES * DS_REC];
  __shared__ int s_page[PCAP];
  constexpr int NT = 64 * DQ_WAVES;
  using Stage = KeyStage<DQS_KB, DQ_WAVES, PCAP>;  // K rows
  static_assert(Stage::NI == 2, "stage instruction count");
  constexpr int kStageOps = Stage::NI + 4;  // + the wave's four dS record rows
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h2 = lane >> 5, col = lane & 31;
  const int G = a.pool.Hq / a.pool.Hkv;
  const int n_qt = (a.n_q + DQ_Q - 1) / DQ_Q;
  const int n_qt64 = (a.n_q + QTB - 1) / QTB;
  const int nkb = (a.max_att_pages * a.pool.P + KPW - 1) / KPW;  // the spill's key blocks
  const HeadUnit hu = head_unit(blockIdx.x, gridDim.x, a.pool.Hkv);
  const TileRange tr = tile_range(hu.unit, whole, n_ks);
  const int g = hu.head, kr = tr.range, n_rng = tr.n_ranges;
  const int hh = tr.tile % G, qt = n_qt - 1 - tr.tile / G;
  const int h = g * G + hh;
  const Keys km = make_keys(a, g);
  const int q0 = qt * DQ_Q;
  const int nblk = n_blocks(km, a.t0 + min(a.n_q, q0 + DQ_Q) - 1);  // stages of 64 keys
  const int b0 = nblk * kr / n_rng, b1 = nblk * (kr + 1) / n_rng;

  // This wave's 64-query tile and key half; the stages its queries see (those up to the
  // tile's last query: the dK/dV pass visited this tile for each of their key blocks).
  const int jq = wave & 3, kh = wave >> 2;
  const int qt64 = 4 * qt + jq;
  const int wq0 = QTB * qt64;
  const int nblk_w = wq0 < a.n_q ? n_blocks(km, a.t0 + min(a.n_q, wq0 + QTB) - 1) : 0;
  const uint16_t* ds_tile = ds + (static_cast<int64_t>(h) * nkb * n_qt64 + (qt64 < n_qt64 ? qt64 : 0)) * (4 * DS_REC);
  // DMA source offsets of this lane's slot in even and odd packs
  const int src_even = 8 * ds_slot(0, lane), src_odd = 8 * ds_slot(1, lane);
  // dS^T operand reads (see above): this lane's offsets for the two key quartets of a
  // k-step of the first query half
  const int qh = (lane >> 4) & 1, kq = (lane & 15) >> 2, m = lane & 3;
  int boff[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) boff[r] = qh * 512 + 8 * ds_slot(qh, 32 * (m & 1) + 4 * h2 + kq + 8 * r) + 4 * (m >> 1);

  f32x16 acc[2][4];  // [query half][d block]: dQ^T over this wave's key halves
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  FragOffsets fo;
  fo.init(lane);
  const uint16_t* kpool = static_cast<const uint16_t*>(a.pool.k_pool);
  const int win0 = (b0 * DQS_KB) >> km.log2p;
  Stage ks{km, s_page, win0, Stage::lane_offset(wave, lane)};
  fill_pages<NT>(km, s_page, win0, tid);
  wait_dma();
  __syncthreads();

  // Stage b: K rows into kt, and this wave's dS record block into its 4 KiB of st.
  // Every stage issues the same operations, also past the last one (b >= b1: zero
  // sources, never used) and where this wave's tile does not see the stage, so that
  // the waits count them exactly.
  auto issue = [&](int b, uint16_t* kt, uint16_t* st) __attribute__((always_inline)) {
    if (b < b1) {
      ks.issue_fixed(b, kpool, kt, wave, lane);
    } else {
#pragma unroll
      for (int i = 0; i < Stage::NI; ++i)
        lds_dma16(g_zero_rows + ks.lane_off, kt + 4 * (DQ_WAVES * i + wave) * D);
    }
    const bool ok = b < nblk_w && b < b1;
    const uint16_t* rec = ds_tile + (static_cast<int64_t>(b >> 1) * n_qt64 * 4 + 2 * (b & 1) + kh) * DS_REC;
    uint16_t* dst = st + wave * DS_REC;
    if (ok) {  // uniform: one base per 512-value part, the lane's offset in the instruction
      const uint32_t lo_e = 2u * static_cast<uint32_t>(src_even), lo_o = 2u * static_cast<uint32_t>(src_odd);
#pragma unroll
      for (int p = 0; p < 4; ++p) lds_dma16_s(rec + p * 512, (p & 1) ? lo_o : lo_e, dst + p * 512);
    } else {
#pragma unroll
      for (int p = 0; p < 4; ++p) lds_dma16(g_zero_rows + 8 * lane, dst + p * 512);
    }
  };
  auto compute = [&](const uint16_t* kt, const uint16_t* st) __attribute__((always_inline)) {
    fo.opaque();
    const FragOffsets& o = fo;
    const uint16_t* sb = st + wave * DS_REC;
    bf16x8 af[2][4], bf[2][2];
#pragma unroll
    for (int sp = 0; sp < 2; ++sp) {
#pragma unroll
      for (int db = 0; db < 4; ++db) af[sp][db] = tr_frag_at(kt, 32 * kh, sp, o, db);
#pragma unroll
      for (int us = 0; us < 2; ++us) {
        const uint16_t* base = sb + us * 1024 + sp * 128;
        const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + boff[0]));
        const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(base + boff[1]));
        bf[us][sp] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    }
#pragma unroll
    for (int sp = 0; sp < 2; ++sp)
#pragma unroll
      for (int us = 0; us < 2; ++us)
#pragma unroll
        for (int db = 0; db < 4; ++db) acc[us][db] = mfma(af[sp][db], bf[us][sp], acc[us][db]);
  };
  // Stage b: once stage b has landed for everyone (and nobody reads stage b - 1 any
  // more), stage b + 2 is issued into (kn, sn) and stage b computed from (kt, st).
  auto stage = [&](int b, const uint16_t* kt, const uint16_t* st, uint16_t* kn, uint16_t* sn)
      __attribute__((always_inline)) {
    wait_vm<kStageOps>();  // this wave's part of stage b (stage b + 1 may stay in flight)
    phase_barrier();       // ... everyone's
    if (b + 2 < b1) {
      const int last_e = ((b + 2) * DQS_KB + DQS_KB - 1) >> km.log2p;
      if (last_e >= ks.win + PCAP) {  // uniform: slide the page window to stage b + 2
        ks.win = ((b + 2) * DQS_KB) >> km.log2p;
        fill_pages<NT>(km, s_page, ks.win, tid);
        wait_dma();
        __syncthreads();
      }
    }
    issue(b + 2, kn, sn);
    if (b < nblk_w && b < b1) compute(kt, st);
  };
  issue(b0, s_k0, s_s0);
  issue(b0 + 1, s_k1, s_s1);
  // Unrolled by three so that each third names its buffers statically; the stages past
  // b1 that complete the last three are empty (no products).
  for (int b = b0; b < b1; b += 3) {
    stage(b, s_k0, s_s0, s_k2, s_s2);
    stage(b + 1, s_k1, s_s1, s_k0, s_s0);
    stage(b + 2, s_k2, s_s2, s_k1, s_s1);
  }

  // The key halves' sums: the second half's waves hand theirs over through LDS (the K
  // buffers are free now), one column block at a time.
  float* xch = reinterpret_cast<float*>(jq < 2 ? s_k0 : s_k1) + (jq & 1) * (2 * 16 * 64);
  wait_dma();
  __syncthreads();
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    if (kh == 1) {
#pragma unroll
      for (int us = 0; us < 2; ++us)
#pragma unroll
        for (int r = 0; r < 16; ++r) xch[(us * 16 + r) * 64 + lane] = acc[us][db][r];
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int us = 0; us < 2; ++us)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[us][db][r] += xch[(us * 16 + r) * 64 + lane];
    }
    __syncthreads();
  }
  if (kh != 0) return;

#pragma unroll
  for (int us = 0; us < 2; ++us) {
    const int i = wq0 + 32 * us + col;
    if (i >= a.n_q) continue;
    float* drow = n_rng == 1 ? a.dq + h * a.dq_hs + static_cast<int64_t>(i) * a.dq_ts
                            : part + ((static_cast<int64_t>(kr) * a.pool.Hq + h) * a.n_q + i) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int ga = 0; ga < 4; ++ga) {
        f32x4 w;
#pragma unroll
        for (int b2 = 0; b2 < 4; ++b2) w[b2] = acc[us][db][4 * ga + b2] * a.scale;
        *reinterpret_cast<f32x4*>(drow + 32 * db + 8 * ga + 4 * h2) = w;
      }
  }
}

}  // namespace mf

// Key ranges per query tile of the dQ pass, chosen for load balance: a tile's work is
// its key blocks (prior keys plus the chunk keys its last query sees). The ranges are
// halved while the largest is more than a quarter of the average work per workgroup
// slot (one per CU, 256 CUs, fixed so the choice and the result bits do not depend on
// the device) and would stay at least 128 blocks, below which the partials' traffic and
// each workgroup's start-up outweigh the balance gained (as in the forward). When the
// tiles are cut and their count is not a multiple of the CU count, mixed_plan cuts
// only those beyond a whole number per CU (see launch.hpp).
SplitPlan dq_plan(const AttnArgs& a) {
  const int n_qt = (a.n_q + mf::DQ_Q - 1) / mf::DQ_Q;
  const int G = a.pool.Hq / a.pool.Hkv;
  SplitPlan forced;
  if (plan_override("OOMB_DQ_SPLITS", "OOMB_DQ_WHOLE", G * n_qt, &forced)) return forced;
  double total = 0.0, largest = 0.0, smallest = 1e300;
  for (int qt = 0; qt < n_qt; ++qt) {
    const double blocks = static_cast<double>(tile_key_blocks(a, qt * mf::DQ_Q, mf::DQ_Q, mf::KB));
    total += blocks;
    largest = blocks > largest ? blocks : largest;
    smallest = blocks < smallest ? blocks : smallest;
  }
  const double per_slot = total * a.pool.Hq / 256.0;
  int nk = 1;
  while (nk < 4 && largest / nk > per_slot / 4.0 && largest / (2 * nk) >= 128.0) nk *= 2;
  return mixed_plan(G * n_qt, a.pool.Hkv, smallest, nk);
}

hipError_t launch_delta_mfma(const AttnArgs& a, hipStream_t s) {
  const int64_t lanes = 2 * static_cast<int64_t>(a.pool.Hq) * a.n_q;
  OOMB_LAUNCH("delta_mfma", mf::delta_mfma_kernel, dim3(static_cast<unsigned>((lanes + 255) / 256)),
              dim3(256), 0, s, a);
  return hipGetLastError();
}

size_t dq_partial_bytes(const AttnArgs& a, SplitPlan p) {
  if (p.n_ks <= 1) return 0;
  return static_cast<size_t>(p.n_ks) * a.pool.Hq * a.n_q * mf::D * sizeof(float);
}

hipError_t launch_dq_mfma(const AttnArgs& a, SplitPlan p, float* part, const uint16_t* ds,
                          hipStream_t s) {
  const int n_qt = (a.n_q + mf::DQ_Q - 1) / mf::DQ_Q;
  const int G = a.pool.Hq / a.pool.Hkv;
  const dim3 grid(a.pool.Hkv * plan_units(p, G * n_qt));
  if (ds != nullptr) {
    OOMB_LAUNCH("dqs_mfma", mf::dqs_mfma_kernel, grid, dim3(64 * mf::DQ_WAVES), 0, s, a, p.n_ks,
                p.whole, part, ds);
  } else {
    OOMB_LAUNCH("dq_mfma", mf::dq_mfma_kernel, grid, dim3(64 * mf::DQ_WAVES), 0, s, a, p.n_ks,
                p.whole, part);
  }
  if (p.n_ks > 1) {
    const int64_t threads = static_cast<int64_t>(a.pool.Hq) * a.n_q * (mf::D / 4);
    OOMB_LAUNCH("dq_merge", mf::dq_merge_kernel, dim3(static_cast<unsigned>((threads + 255) / 256)),
                dim3(256), 0, s, a, p.n_ks, p.whole, part);
  }
  return hipGetLastError();
}

}  // namespace oomb
