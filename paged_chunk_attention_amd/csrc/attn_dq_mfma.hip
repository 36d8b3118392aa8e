// Matrix-core backward of paged chunk attention, dQ pass: recompute P from the saved
// log-sum-exp and dP = dO V^T per key block, then dQ^T += K^T dS^T.
//
// Key blocks are staged through registers (a global load at the top of a block, an
// LDS store at its end) rather than by global->LDS DMA: this kernel keeps Q and dO
// fragments, the dQ accumulator and two score tiles live at once, and the register
// path leaves the compiler more room than the DMA address arithmetic does.
#include "mfma_tiles.hpp"

namespace oomb {
namespace mf {

// 256 threads stage one 64-key block: thread = (rows tid/16 + 16i, 16-byte chunk tid%16).
struct RegKeyStream {
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

struct DqSmem {
  uint16_t k[2][KB * D];
  uint16_t v[2][KB * D];
  int page[PCAP];
};

// Load block b + 1 into registers (sliding the page-id window first when needed).
__device__ __forceinline__ void reg_prefetch_next(RegKeyStream& ks, DqSmem& sm, const Keys& km,
                                                  int b, int nblk, int tid) {
  if (b + 1 >= nblk) return;
  const int last_e = ((b + 1) * KB + KB - 1) >> km.log2p;
  if (last_e >= ks.win + PCAP) {  // uniform over the workgroup
    ks.win = ((b + 1) * KB) >> km.log2p;
    fill_pages<256>(km, sm.page, ks.win, tid);
    __syncthreads();
  }
  ks.load(b + 1, tid);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2)))
void dq_mfma_kernel(AttnArgs a) {
  __shared__ DqSmem sm;
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

  // This lane's query (column of S^T and dP^T) with its Q and dO fragments.
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

  fill_pages<256>(km, sm.page, 0, tid);
  __syncthreads();
  RegKeyStream ks{km, sm.page, 0, a.pool.k_pool, a.pool.v_pool};
  if (nblk > 0) {
    ks.load(0, tid);
    ks.store(sm.k[0], sm.v[0], tid);
  }
  __syncthreads();
  for (int b = 0; b < nblk; ++b) {
    const int buf = b & 1;
    reg_prefetch_next(ks, sm, km, b, nblk, tid);
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

}  // namespace mf

hipError_t launch_dq_mfma(const AttnArgs& a, hipStream_t s) {
  const int n_qt = (a.n_q + 127) / 128;
  OOMB_LAUNCH("dq_mfma", mf::dq_mfma_kernel, dim3(a.pool.Hq * n_qt), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace oomb
