// Matrix-core forward of paged chunk attention (online softmax over the attended
// key blocks; writes O and the log-sum-exp the backward recomputes P from).
#include "mfma_tiles.hpp"

namespace oomb {
namespace mf {

// ============================================================================ forward
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_mfma_kernel(AttnArgs a) {
  OOMB_KV_BUFFERS
  constexpr int QT = 128;
  // the wave index is uniform: keep it (and the LDS addresses built from it) scalar
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

  KeyStream ks{km, s_page, 0, static_cast<const uint16_t*>(a.pool.k_pool),
               static_cast<const uint16_t*>(a.pool.v_pool)};
  start_stream(ks, s_page, km, nblk, tid, wave, lane, s_k0, s_v0, s_k1, s_v1);
  // One key block: prefetch block b + 1 into (kn, vn), compute block b from (kt, vt).
  auto step = [&](int b, const uint16_t* kt, const uint16_t* vt, uint16_t* kn,
                  uint16_t* vn) __attribute__((always_inline)) {
    prefetch_next(ks, s_page, km, b, nblk, tid, wave, lane, kn, vn);

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
    // Row maximum: four independent chains, then the other half-wave's rows.
    float mx4[4] = {st[0][0], st[0][1], st[0][2], st[0][3]};
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (sub || r >= 4) mx4[r & 3] = fmaxf(mx4[r & 3], st[sub][r]);
    float mx = fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3]));
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

    wait_dma();  // block b + 1 has landed (this wave's part) ...
    __syncthreads();  // ... everyone's, and nobody reads block b any more
  };
  // Unrolled by two so that each half names its read and write buffers statically.
  for (int b = 0; b < nblk; b += 2) {
    step(b, s_k0, s_v0, s_k1, s_v1);
    if (b + 1 < nblk) step(b + 1, s_k1, s_v1, s_k0, s_v0);
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

}  // namespace mf

hipError_t launch_fwd_mfma(const AttnArgs& a, hipStream_t s) {
  const int n_qt = (a.n_q + 127) / 128;
  OOMB_LAUNCH("fwd_mfma", mf::fwd_mfma_kernel, dim3(a.pool.Hq * n_qt), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace oomb
