// Scalar (non-matrix-core) paged chunk attention for gfx950: one wavefront per
// query row (forward, dQ) or per key row (dK/dV), lanes spread over the head
// dimension, fp32 arithmetic throughout. This instance serves the fp32 pool and
// every shape the matrix-core kernels do not take; it is exact enough for the
// fp32 tolerance (no rounding of P or dS to a narrower type).
//
// What is computed (gist.science explainer of OOMB, 2.A recomputation, 2.B paged
// K/V and paged gradients with in-place accumulation, 2.D page selection): query
// i at position t0+i attends to key t iff t <= t0+i and page(t) is selected or
// local (and, with a window W, t > t0+i-W); forward writes O and the natural-log LSE,
// backward recomputes
// P = exp(s - LSE) and writes dQ and adds dK/dV into the gradient pool.
#include "device_common.hpp"
#include "launch.hpp"
#include "profiling.hpp"

namespace oomb {

__device__ __forceinline__ AttendMap make_map(const AttnArgs& a, int g) {
  AttendMap m;
  m.table = a.table + g * a.tstride;
  m.sel = a.sel ? a.sel + g * a.sel_stride : nullptr;
  m.n_sel = a.sel ? clamp_count(a.count, g, a.sel_stride, a.n_cand) : a.n_cand;
  m.prior0 = a.prior0;
  m.first_local = a.first_local;
  m.n_pages_att = m.n_sel + a.n_local;
  m.num_pages = a.pool.N;
  m.log2p = a.pool.log2p;
  return m;
}

// Logical page of entry e, or -1 for a selected id outside the candidate range.
__device__ __forceinline__ int checked_logical(const AttendMap& m, int e) {
  const int lp = m.logical(e);
  if (e < m.n_sel && m.sel && (lp < 0 || lp >= m.first_local)) return -1;
  return lp;
}

template <typename T>
__device__ __forceinline__ float ld(const void* base, int64_t off) {
  return to_f32(reinterpret_cast<const T*>(base)[off]);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void fwd_scalar_kernel(AttnArgs a) {
  constexpr int R = D / 64;
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int h = blockIdx.y;
  if (i >= a.n_q) return;
  const int G = a.pool.Hq / a.pool.Hkv, g = h / G;
  const AttendMap m = make_map(a, g);
  const float c = a.scale * kLog2e;
  float q[R], acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    q[r] = ld<T>(a.q, h * a.q_hs + i * a.q_ts + lane + 64 * r);
    acc[r] = 0.0f;
  }
  const int qpos = a.t0 + i;
  const int kmin = a.window > 0 ? qpos - a.window + 1 : 0;  // first visible position
  float mx = -__builtin_inff(), l = 0.0f;
  for (int e = 0; e < m.n_pages_att; ++e) {
    const int lp = checked_logical(m, e);
    const int64_t ph = m.physical(e, lp);
    if (ph < 0) continue;
    const int base = lp << m.log2p;
    if (base > qpos) break;  // local pages ascend: every later page is in the future
    const int n = min(a.pool.P, qpos - base + 1);
    for (int s = max(0, kmin - base); s < n; ++s) {
      const int64_t row = ((ph << m.log2p) + s) * D;
      float dot = 0.0f;
#pragma unroll
      for (int r = 0; r < R; ++r) dot += q[r] * ld<T>(a.pool.k_pool, row + lane + 64 * r);
      const float s2 = wave_sum(dot) * c;
      const float mnew = fmaxf(mx, s2);
      const float alpha = exp2f(mx - mnew);
      const float p = exp2f(s2 - mnew);
      l = l * alpha + p;
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = acc[r] * alpha + p * ld<T>(a.pool.v_pool, row + lane + 64 * r);
      mx = mnew;
    }
  }
  const float inv = 1.0f / l;
#pragma unroll
  for (int r = 0; r < R; ++r)
    reinterpret_cast<T*>(a.o)[h * a.o_hs + i * a.o_ts + lane + 64 * r] = from_f32<T>(acc[r] * inv);
  if (lane == 0) a.lse[static_cast<int64_t>(h) * a.n_q + i] = (mx + __log2f(l)) * kLn2;
}

// Delta_i = sum_d dO_i[d] * O_i[d] in fp32, with 16-byte loads: L = D * sizeof(T) / 16
// lanes per row, 64 / L rows per wave (bf16, D = 128: 16 lanes, 4 rows). The boundary
// guarantees 16-byte aligned rows (aligned pointers, strides in multiples of 16 bytes).
template <typename T, int D>
__global__ __launch_bounds__(256) void delta_kernel(AttnArgs a) {
  constexpr int EPL = 16 / static_cast<int>(sizeof(T));  // elements per lane
  constexpr int L = D / EPL;
  constexpr int RPW = 64 / L;
  static_assert(L >= 1 && L <= 64 && 64 % L == 0, "row split");
  const int lane = threadIdx.x & 63;
  const int i = (blockIdx.x * 4 + (threadIdx.x >> 6)) * RPW + lane / L;
  const int h = blockIdx.y;
  const int c = (lane % L) * EPL;
  float s = 0.0f;
  if (i < a.n_q) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(static_cast<const T*>(a.dout) + h * a.do_hs +
                                                   static_cast<int64_t>(i) * a.do_ts + c);
    const u32x4 y = *reinterpret_cast<const u32x4*>(static_cast<const T*>(a.o) + h * a.o_hs +
                                                   static_cast<int64_t>(i) * a.o_ts + c);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (sizeof(T) == 2) {  // bf16: two values per word
        s += __uint_as_float(x[k] << 16) * __uint_as_float(y[k] << 16);
        s += __uint_as_float(x[k] & 0xFFFF0000u) * __uint_as_float(y[k] & 0xFFFF0000u);
      } else {
        s += __uint_as_float(x[k]) * __uint_as_float(y[k]);
      }
    }
  }
#pragma unroll
  for (int m = L / 2; m >= 1; m >>= 1) s += __shfl_xor(s, m);  // within the row's L lanes
  if (lane % L == 0 && i < a.n_q) a.delta[static_cast<int64_t>(h) * a.n_q + i] = s;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void dq_scalar_kernel(AttnArgs a) {
  constexpr int R = D / 64;
  const int lane = threadIdx.x & 63;
  const int i = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int h = blockIdx.y;
  if (i >= a.n_q) return;
  const int G = a.pool.Hq / a.pool.Hkv, g = h / G;
  const AttendMap m = make_map(a, g);
  const float c = a.scale * kLog2e;
  float q[R], dob[R], acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    q[r] = ld<T>(a.q, h * a.q_hs + i * a.q_ts + lane + 64 * r);
    dob[r] = ld<T>(a.dout, h * a.do_hs + i * a.do_ts + lane + 64 * r);
    acc[r] = 0.0f;
  }
  const int64_t row_id = static_cast<int64_t>(h) * a.n_q + i;
  const float lse2 = a.lse_in[row_id] * kLog2e;
  const float delta = a.delta[row_id];
  const int qpos = a.t0 + i;
  const int kmin = a.window > 0 ? qpos - a.window + 1 : 0;  // first visible position
  for (int e = 0; e < m.n_pages_att; ++e) {
    const int lp = checked_logical(m, e);
    const int64_t ph = m.physical(e, lp);
    if (ph < 0) continue;
    const int base = lp << m.log2p;
    if (base > qpos) break;
    const int n = min(a.pool.P, qpos - base + 1);
    for (int s = max(0, kmin - base); s < n; ++s) {
      const int64_t row = ((ph << m.log2p) + s) * D;
      float dot = 0.0f, dpv = 0.0f;
      float k[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        k[r] = ld<T>(a.pool.k_pool, row + lane + 64 * r);
        dot += q[r] * k[r];
        dpv += dob[r] * ld<T>(a.pool.v_pool, row + lane + 64 * r);
      }
      const float p = exp2f(wave_sum(dot) * c - lse2);
      const float ds = p * (wave_sum(dpv) - delta);
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] += ds * k[r];
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) a.dq[h * a.dq_hs + i * a.dq_ts + lane + 64 * r] = acc[r] * a.scale;
}

// One wavefront per attended key row (KV head g, attended index). The row is
// owned by this wavefront alone, so the gradient-pool update is a plain
// read-modify-write.
template <typename T, int D>
__global__ __launch_bounds__(256) void dkdv_scalar_kernel(AttnArgs a) {
  constexpr int R = D / 64;
  const int lane = threadIdx.x & 63;
  const int kidx = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int g = blockIdx.y;
  const int G = a.pool.Hq / a.pool.Hkv;
  const AttendMap m = make_map(a, g);
  const int e = kidx >> m.log2p, slot = kidx & (a.pool.P - 1);
  if (e >= m.n_pages_att) return;
  const int lp = checked_logical(m, e);
  const int64_t ph = m.physical(e, lp);
  if (ph < 0) return;
  const int kpos = (lp << m.log2p) + slot;
  if (kpos >= a.t0 + a.n_q) return;  // not yet in the sequence
  const int64_t gph = a.gtable[g * a.gtstride + lp];
  if (gph < 0 || gph >= a.pool.Ng) return;
  const float c = a.scale * kLog2e;
  const int64_t row = ((ph << m.log2p) + slot) * D;
  float k[R], v[R], dk[R], dv[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    k[r] = ld<T>(a.pool.k_pool, row + lane + 64 * r);
    v[r] = ld<T>(a.pool.v_pool, row + lane + 64 * r);
    dk[r] = 0.0f;
    dv[r] = 0.0f;
  }
  const int i0 = kpos > a.t0 ? kpos - a.t0 : 0;
  // with a window, queries at kpos + window and later no longer see this key
  const int i1 = a.window > 0 ? min(a.n_q, kpos + a.window - a.t0) : a.n_q;
  for (int hh = 0; hh < G; ++hh) {
    const int h = g * G + hh;
    for (int i = i0; i < i1; ++i) {
      float q[R], dob[R], dot = 0.0f, dpv = 0.0f;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        q[r] = ld<T>(a.q, h * a.q_hs + i * a.q_ts + lane + 64 * r);
        dob[r] = ld<T>(a.dout, h * a.do_hs + i * a.do_ts + lane + 64 * r);
        dot += q[r] * k[r];
        dpv += dob[r] * v[r];
      }
      const int64_t row_id = static_cast<int64_t>(h) * a.n_q + i;
      const float p = exp2f(wave_sum(dot) * c - a.lse_in[row_id] * kLog2e);
      const float ds = p * (wave_sum(dpv) - a.delta[row_id]);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        dk[r] += ds * q[r];
        dv[r] += p * dob[r];
      }
    }
  }
  const int64_t grow = ((gph << m.log2p) + slot) * D;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    a.pool.dk_pool[grow + lane + 64 * r] += dk[r] * a.scale;
    a.pool.dv_pool[grow + lane + 64 * r] += dv[r];
  }
}

#define OOMB_DISPATCH(KERNEL, GRID)                                                       \
  do {                                                                                    \
    if (a.pool.dtype == 0 && a.pool.D == 128)                                             \
      OOMB_LAUNCH(#KERNEL, (KERNEL<bf16_t, 128>), GRID, dim3(256), 0, s, a);                \
    else if (a.pool.dtype == 0)                                                           \
      OOMB_LAUNCH(#KERNEL, (KERNEL<bf16_t, 64>), GRID, dim3(256), 0, s, a);                 \
    else if (a.pool.D == 128)                                                             \
      OOMB_LAUNCH(#KERNEL, (KERNEL<float, 128>), GRID, dim3(256), 0, s, a);                 \
    else                                                                                  \
      OOMB_LAUNCH(#KERNEL, (KERNEL<float, 64>), GRID, dim3(256), 0, s, a);                  \
  } while (0)

hipError_t launch_fwd_scalar(const AttnArgs& a, hipStream_t s) {
  dim3 grid((a.n_q + 3) / 4, a.pool.Hq);
  OOMB_DISPATCH(fwd_scalar_kernel, grid);
  return hipGetLastError();
}

hipError_t launch_delta(const AttnArgs& a, hipStream_t s) {
  const int elems_per_lane = a.pool.dtype == 0 ? 8 : 4;
  const int rows_per_block = 4 * (64 / (a.pool.D / elems_per_lane));
  dim3 grid((a.n_q + rows_per_block - 1) / rows_per_block, a.pool.Hq);
  OOMB_DISPATCH(delta_kernel, grid);
  return hipGetLastError();
}

hipError_t launch_bwd_scalar(const AttnArgs& a, hipStream_t s) {
  hipError_t err = launch_delta(a, s);
  if (err != hipSuccess) return err;
  dim3 gq((a.n_q + 3) / 4, a.pool.Hq);
  OOMB_DISPATCH(dq_scalar_kernel, gq);
  const int64_t keys = static_cast<int64_t>(a.max_att_pages) * a.pool.P;
  dim3 gk(static_cast<unsigned>((keys + 3) / 4), a.pool.Hkv);
  OOMB_DISPATCH(dkdv_scalar_kernel, gk);
  return hipGetLastError();
}

}  // namespace oomb
