// Scalar (non-matrix-core) paged chunk attention for gfx950: one workgroup per
// query row (forward, dQ) or per key row (dK/dV), its waves splitting the other
// side's rows in blocks of 64, fp32 arithmetic throughout. This instance serves the
// fp32 pool and every shape the matrix-core kernels do not take; it is exact enough
// for the fp32 tolerance (no rounding of P or dS to a narrower type).
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

// Keys (or queries) are taken 64 at a time, one per lane; each lane forms its own row's
// dot products, and the weighted row sums are then accumulated with the lanes over the
// head dimension (dimension lane + 64r), the weights and row ids of the 64 rows broadcast
// from their lanes. A block of 64 rows thus costs two wavefront reductions at most (the
// forward's row maximum and sum), not two per row.

// sum_d x[d] * row[d]: x is this wave's fp32 copy in LDS, row the D elements of T at
// base + off (16-byte aligned: pools and views are, and rows are D elements long).
template <typename T, int D>
__device__ __forceinline__ float row_dot(const float* x, const void* base, int64_t off) {
  constexpr int EPL = 16 / static_cast<int>(sizeof(T));
  const u32x4* p = reinterpret_cast<const u32x4*>(static_cast<const T*>(base) + off);
  float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int c = 0; c < D / EPL; ++c) {
    const u32x4 w = p[c];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if constexpr (sizeof(T) == 2) {  // bf16: element 2k in the low half of word k
        s[k] = fmaf(x[c * 8 + 2 * k], __uint_as_float(w[k] << 16), s[k]);
        s[k] = fmaf(x[c * 8 + 2 * k + 1], __uint_as_float(w[k] & 0xFFFF0000u), s[k]);
      } else {
        s[k] = fmaf(x[c * 4 + k], __uint_as_float(w[k]), s[k]);
      }
    }
  }
  return (s[0] + s[1]) + (s[2] + s[3]);
}

// Copy row `off` of a [token][D] view (D elements of T) into this wave's LDS row as fp32.
template <typename T, int D>
__device__ __forceinline__ void row_to_lds(float* dst, const void* base, int64_t off, int lane) {
#pragma unroll
  for (int r = 0; r < D / 64; ++r) dst[lane + 64 * r] = ld<T>(base, off + lane + 64 * r);
  // the other lanes' rows are read next: one wave's LDS operations complete in order, and
  // the wavefront-scope fences keep the compiler from moving the reads above the writes
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float lane_f32(float x, int j) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), j));
}
__device__ __forceinline__ int64_t lane_i64(int64_t x, int j) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(x), j);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(x >> 32), j);
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Pool row (physical token index) of attended key slot u = e * P + s, or -1 when the slot
// is past u_end, its page is out of range or the key is not visible from position qpos
// (future, or before kmin).
__device__ __forceinline__ int64_t key_row(const AttendMap& m, int u, int u_end, int qpos, int kmin) {
  if (u >= u_end) return -1;
  const int e = u >> m.log2p, s = u & ((1 << m.log2p) - 1);
  const int lp = checked_logical(m, e);
  const int64_t ph = m.physical(e, lp);
  const int pos = (lp << m.log2p) + s;
  return (ph >= 0 && pos <= qpos && pos >= kmin) ? (ph << m.log2p) + s : -1;
}

// Key slots that can be visible from position qpos: entries up to the local page holding it.
__device__ __forceinline__ int key_slots(const AttendMap& m, int qpos) {
  const int n_end = min(m.n_pages_att, m.n_sel + (qpos >> m.log2p) - m.first_local + 1);
  return max(n_end, 0) << m.log2p;
}

// One workgroup per query row; its 4 waves take every 4th block of 64 key slots and
// merge their partial softmax states through LDS at the end.
template <typename T, int D>
__global__ __launch_bounds__(256) void fwd_scalar_kernel(AttnArgs a) {
  constexpr int R = D / 64;
  __shared__ float s_q[4][D], s_acc[4][D], s_m[4], s_l[4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i = blockIdx.x;
  const int h = blockIdx.y;
  const int G = a.pool.Hq / a.pool.Hkv, g = h / G;
  const AttendMap m = make_map(a, g);
  const float c = a.scale * kLog2e;
  row_to_lds<T, D>(s_q[w], a.q, static_cast<int64_t>(h) * a.q_hs + static_cast<int64_t>(i) * a.q_ts, lane);
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;
  const int qpos = a.t0 + i;
  const int kmin = a.window > 0 ? qpos - a.window + 1 : 0;  // first visible position
  const int u_end = key_slots(m, qpos);
  float mx = -__builtin_inff(), l = 0.0f;
  for (int u0 = 64 * w; u0 < u_end; u0 += 256) {
    const int64_t row = key_row(m, u0 + lane, u_end, qpos, kmin);
    const uint64_t valid = __ballot(row >= 0);
    if (valid == 0) continue;
    const float s2 = row >= 0 ? row_dot<T, D>(s_q[w], a.pool.k_pool, row * D) * c : -__builtin_inff();
    const float mnew = fmaxf(mx, wave_max(s2));
    const float alpha = exp2f(mx - mnew);
    const float p = row >= 0 ? exp2f(s2 - mnew) : 0.0f;
    l = l * alpha + wave_sum(p);
    mx = mnew;
    // masked lanes read a visible row of this block with weight 0
    const int64_t rowc = row >= 0 ? row : lane_i64(row, __builtin_ctzll(valid));
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] *= alpha;
#pragma unroll
    for (int j = 0; j < 64; ++j) {
      const float pj = lane_f32(p, j);
      const int64_t vr = lane_i64(rowc, j) * D + lane;
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = fmaf(pj, ld<T>(a.pool.v_pool, vr + 64 * r), acc[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) s_acc[w][lane + 64 * r] = acc[r];
  if (lane == 0) {
    s_m[w] = mx;
    s_l[w] = l;
  }
  __syncthreads();
  if (w != 0) return;
  float mall = -__builtin_inff();
#pragma unroll
  for (int x = 0; x < 4; ++x) mall = fmaxf(mall, s_m[x]);
  float lall = 0.0f, o[R];
#pragma unroll
  for (int r = 0; r < R; ++r) o[r] = 0.0f;
#pragma unroll
  for (int x = 0; x < 4; ++x) {
    const float f = s_m[x] == -__builtin_inff() ? 0.0f : exp2f(s_m[x] - mall);  // a wave with no keys adds 0
    lall = fmaf(s_l[x], f, lall);
#pragma unroll
    for (int r = 0; r < R; ++r) o[r] = fmaf(s_acc[x][lane + 64 * r], f, o[r]);
  }
  const float inv = 1.0f / lall;
#pragma unroll
  for (int r = 0; r < R; ++r)
    reinterpret_cast<T*>(a.o)[h * a.o_hs + i * a.o_ts + lane + 64 * r] = from_f32<T>(o[r] * inv);
  if (lane == 0) a.lse[static_cast<int64_t>(h) * a.n_q + i] = (mall + __log2f(lall)) * kLn2;
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

// One workgroup per query row; its 4 waves take every 4th block of 64 key slots and add
// their partial sums through LDS at the end.
template <typename T, int D>
__global__ __launch_bounds__(256) void dq_scalar_kernel(AttnArgs a) {
  constexpr int R = D / 64;
  __shared__ float s_q[4][D], s_do[4][D];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int i = blockIdx.x;
  const int h = blockIdx.y;
  const int G = a.pool.Hq / a.pool.Hkv, g = h / G;
  const AttendMap m = make_map(a, g);
  const float c = a.scale * kLog2e;
  row_to_lds<T, D>(s_q[w], a.q, static_cast<int64_t>(h) * a.q_hs + static_cast<int64_t>(i) * a.q_ts, lane);
  row_to_lds<T, D>(s_do[w], a.dout, static_cast<int64_t>(h) * a.do_hs + static_cast<int64_t>(i) * a.do_ts, lane);
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) acc[r] = 0.0f;
  const int64_t row_id = static_cast<int64_t>(h) * a.n_q + i;
  const float lse2 = a.lse_in[row_id] * kLog2e;
  const float delta = a.delta[row_id];
  const int qpos = a.t0 + i;
  const int kmin = a.window > 0 ? qpos - a.window + 1 : 0;  // first visible position
  const int u_end = key_slots(m, qpos);
  for (int u0 = 64 * w; u0 < u_end; u0 += 256) {
    const int64_t row = key_row(m, u0 + lane, u_end, qpos, kmin);
    const uint64_t valid = __ballot(row >= 0);
    if (valid == 0) continue;
    float ds = 0.0f;
    if (row >= 0) {
      const float p = exp2f(row_dot<T, D>(s_q[w], a.pool.k_pool, row * D) * c - lse2);
      ds = p * (row_dot<T, D>(s_do[w], a.pool.v_pool, row * D) - delta);
    }
    const int64_t rowc = row >= 0 ? row : lane_i64(row, __builtin_ctzll(valid));
#pragma unroll
    for (int j = 0; j < 64; ++j) {
      const float dsj = lane_f32(ds, j);
      const int64_t kr = lane_i64(rowc, j) * D + lane;
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r] = fmaf(dsj, ld<T>(a.pool.k_pool, kr + 64 * r), acc[r]);
    }
  }
  // each wave's sums go to its own q row (only this wave read it, and the sums depend on
  // every read)
#pragma unroll
  for (int r = 0; r < R; ++r) s_q[w][lane + 64 * r] = acc[r];
  __syncthreads();
  if (w != 0) return;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int d = lane + 64 * r;
    a.dq[h * a.dq_hs + i * a.dq_ts + d] = ((s_q[0][d] + s_q[1][d]) + (s_q[2][d] + s_q[3][d])) * a.scale;
  }
}

// One workgroup per attended key row (KV head g, attended index); its 4 waves take every
// 4th (query head, block of 64 queries) pair, lanes over the queries, and add their sums
// through LDS. The row is owned by this workgroup alone, so the gradient-pool update is a
// plain read-modify-write.
template <typename T, int D>
__global__ __launch_bounds__(256) void dkdv_scalar_kernel(AttnArgs a) {
  constexpr int R = D / 64;
  __shared__ float s_k[4][D], s_v[4][D];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int kidx = blockIdx.x;
  const int g = blockIdx.y;
  const int G = a.pool.Hq / a.pool.Hkv;
  const AttendMap m = make_map(a, g);
  const int e = kidx >> m.log2p, slot = kidx & (a.pool.P - 1);
  if (e >= m.n_pages_att) return;  // the exits below are uniform over the workgroup
  const int lp = checked_logical(m, e);
  const int64_t ph = m.physical(e, lp);
  if (ph < 0) return;
  const int kpos = (lp << m.log2p) + slot;
  if (kpos >= a.t0 + a.n_q) return;  // not yet in the sequence
  const int64_t gph = a.gtable[g * a.gtstride + lp];
  if (gph < 0 || gph >= a.pool.Ng) return;
  const float c = a.scale * kLog2e;
  const int64_t row = ((ph << m.log2p) + slot) * D;
  row_to_lds<T, D>(s_k[w], a.pool.k_pool, row, lane);
  row_to_lds<T, D>(s_v[w], a.pool.v_pool, row, lane);
  float dk[R], dv[R];
#pragma unroll
  for (int r = 0; r < R; ++r) dk[r] = dv[r] = 0.0f;
  const int i0 = kpos > a.t0 ? kpos - a.t0 : 0;
  // with a window, queries at kpos + window and later no longer see this key
  const int i1 = a.window > 0 ? min(a.n_q, kpos + a.window - a.t0) : a.n_q;
  const int nblk = (i1 - i0 + 63) / 64;
  for (int t = w; t < G * nblk; t += 4) {
    const int h = g * G + t / nblk;
    const int ib = i0 + 64 * (t % nblk);
    const int i = ib + lane;
    float p = 0.0f, ds = 0.0f;
    if (i < i1) {
      const int64_t row_id = static_cast<int64_t>(h) * a.n_q + i;
      p = exp2f(row_dot<T, D>(s_k[w], a.q, h * a.q_hs + static_cast<int64_t>(i) * a.q_ts) * c -
                a.lse_in[row_id] * kLog2e);
      ds = p * (row_dot<T, D>(s_v[w], a.dout, h * a.do_hs + static_cast<int64_t>(i) * a.do_ts) -
                a.delta[row_id]);
    }
    // lanes past i1 stand for query i1 - 1 with weight 0
#pragma unroll
    for (int j = 0; j < 64; ++j) {
      const float pj = lane_f32(p, j), dsj = lane_f32(ds, j);
      const int64_t ij = min(ib + j, i1 - 1);
      const int64_t qo = h * a.q_hs + ij * a.q_ts + lane, oo = h * a.do_hs + ij * a.do_ts + lane;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        dk[r] = fmaf(dsj, ld<T>(a.q, qo + 64 * r), dk[r]);
        dv[r] = fmaf(pj, ld<T>(a.dout, oo + 64 * r), dv[r]);
      }
    }
  }
  // each wave's sums go to its own k / v rows (only this wave read them, and the sums
  // depend on every read)
#pragma unroll
  for (int r = 0; r < R; ++r) {
    s_k[w][lane + 64 * r] = dk[r];
    s_v[w][lane + 64 * r] = dv[r];
  }
  __syncthreads();
  if (w != 0) return;
  const int64_t grow = ((gph << m.log2p) + slot) * D;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int d = lane + 64 * r;
    a.pool.dk_pool[grow + d] += ((s_k[0][d] + s_k[1][d]) + (s_k[2][d] + s_k[3][d])) * a.scale;
    a.pool.dv_pool[grow + d] += (s_v[0][d] + s_v[1][d]) + (s_v[2][d] + s_v[3][d]);
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
  dim3 grid(a.n_q, a.pool.Hq);
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
  dim3 gq(a.n_q, a.pool.Hq);
  OOMB_DISPATCH(dq_scalar_kernel, gq);
  const int64_t keys = static_cast<int64_t>(a.max_att_pages) * a.pool.P;
  dim3 gk(static_cast<unsigned>(keys), a.pool.Hkv);
  OOMB_DISPATCH(dkdv_scalar_kernel, gk);
  return hipGetLastError();
}

}  // namespace oomb
