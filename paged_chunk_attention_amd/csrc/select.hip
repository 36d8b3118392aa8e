// Top-k page retrieval for gfx950 (gist.science explainer of OOMB, 2.D
// "Page-Level Sparse Attention": per chunk, keep only the K most relevant prior
// key pages, scored through an averaged stand-in vector). The rule is Quest-style:
//   qbar   = mean of the chunk's queries over the KV head's query-head group;
//   score  = sum_d max(qbar_d * kmax_d, qbar_d * kmin_d) with per-page key min/max;
//   keep the top-k scores, ties to the lower logical page id, ascending output.
// All float arithmetic is IEEE fp32 without contraction, in one fixed order, so the
// selection is reproducible bit for bit:
//   qbar: sequential sums (from +0) over blocks of 64 consecutive rows (head-major,
//         then query order), a stride-halving tree over the zero-padded block sums,
//         one multiply by fp32(1/(G*n_q));
//   score: products rounded to fp32, the larger kept (qbar*kmax only if strictly
//         larger), a stride-halving tree over d (a wavefront butterfly).
#pragma clang fp contract(off)

#include <mutex>

#include "device_common.hpp"
#include "launch.hpp"
#include "profiling.hpp"
#include "scratch.hpp"

namespace oomb {

constexpr int kQBlock = 64;

// Queries in tile j of the chunk (the last tile may be shorter).
__device__ __forceinline__ int tile_len(const SelectArgs& a, int j) {
  return j + 1 < a.n_tiles ? a.tile : a.n_q - j * a.tile;
}

// Block partial sums. Thread t of the grid owns block b = t / (D/8) of 64 consecutive
// rows of unit blockIdx.y (query tile j, KV head g) and head dimensions 8 (t % (D/8))
// .. +7: one 16-byte load per row (issued in groups of 16), each dimension summed
// strictly in row order.
template <bool kBf16>
__global__ __launch_bounds__(256) void qbar_partial_kernel(SelectArgs a) {
  const int D = a.pool.D;
  const int lanes_per_block = D / 8;
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  const int b = t / lanes_per_block, d0 = 8 * (t % lanes_per_block);
  const int u = blockIdx.y, tj = u / a.pool.Hkv, g = u % a.pool.Hkv;
  const int G = a.pool.Hq / a.pool.Hkv;
  const int nq = tile_len(a, tj), qoff = tj * a.tile;
  const int M = G * nq;
  if (b >= (M + kQBlock - 1) / kQBlock) return;
  const int m0 = b * kQBlock;
  const int m1 = (m0 + kQBlock < M) ? m0 + kQBlock : M;
  constexpr int kGroup = 16;
  float s[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) s[c] = 0.0f;
  // (head, query) of row m, stepped row by row (no division per row). The body is
  // branch-free (rows past the block's end load its first row and count as zero): a
  // branch per row would make each load wait for the previous one.
  const int h0 = g * G + m0 / nq, i0 = qoff + m0 % nq;
  int h = h0, i = i0;
  for (int mg = m0; mg < m1; mg += kGroup) {
    float x[kGroup][8];
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      const bool live = mg + u < m1;
      const int64_t off = (live ? h * a.q_hs + static_cast<int64_t>(i) * a.q_ts
                                : h0 * a.q_hs + static_cast<int64_t>(i0) * a.q_ts) + d0;
      const int in = i + 1;
      const bool wrap = in == qoff + nq;
      i = wrap ? qoff : in;
      h += wrap ? 1 : 0;
      if (kBf16) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16_t*>(a.q) + off);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          x[u][2 * c] = live ? __uint_as_float(w[c] << 16) : 0.0f;
          x[u][2 * c + 1] = live ? __uint_as_float(w[c] & 0xFFFF0000u) : 0.0f;
        }
      } else {
        const f32x4 lo = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(a.q) + off);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(a.q) + off + 4);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          x[u][c] = live ? lo[c] : 0.0f;
          x[u][4 + c] = live ? hi[c] : 0.0f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      if (mg + u < m1) {
#pragma unroll
        for (int c = 0; c < 8; ++c) s[c] = s[c] + x[u][c];
      }
    }
  }
  float* dst = a.partial + (static_cast<int64_t>(u) * a.nb + b) * D + d0;
#pragma unroll
  for (int c = 0; c < 8; ++c) dst[c] = s[c];
}

// Pairwise tree over the block sums of one (head dimension, unit), zero-padded to the
// power of two of the unit's own block count.
__global__ __launch_bounds__(256) void qbar_final_kernel(SelectArgs a) {
  extern __shared__ float s_tree[];
  const int d = blockIdx.x, u = blockIdx.y, tj = u / a.pool.Hkv;
  const int D = a.pool.D;
  const int G = a.pool.Hq / a.pool.Hkv;
  const int nb = (G * tile_len(a, tj) + kQBlock - 1) / kQBlock;
  int n2 = 1;
  while (n2 < nb) n2 <<= 1;
  for (int i = threadIdx.x; i < n2; i += 256)
    s_tree[i] = i < nb ? a.partial[(static_cast<int64_t>(u) * a.nb + i) * D + d] : 0.0f;
  __syncthreads();
  for (int s = n2 >> 1; s >= 1; s >>= 1) {
    for (int i = threadIdx.x; i < s; i += 256) s_tree[i] = s_tree[i] + s_tree[i + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.qbar[u * D + d] = s_tree[0] * (tj + 1 < a.n_tiles ? a.inv : a.inv_last);
}

// D / 8 lanes per candidate page (64 / (D / 8) pages per wavefront, 4 wavefronts per
// workgroup): lane l of a page holds dimensions 8l .. 8l + 7, loaded as one 16-byte
// row piece of kmin and of kmax (bf16). The stride-halving tree over d keeps its order:
// the levels s = D/2 .. 8 pair lane l with lane l ^ (s / 8) (same slot), the levels
// s = 4, 2, 1 pair slots within the lane, each sum a[d] + a[d + s] as in the definition.
template <bool kBf16, int D>
__global__ __launch_bounds__(256) void page_score_kernel(SelectArgs a) {
  constexpr int LP = D / 8;        // lanes per page
  constexpr int PW = 64 / LP;      // pages per wavefront
  const int lane = threadIdx.x & 63, sub = lane % LP;
  const int j = (blockIdx.x * 4 + (threadIdx.x >> 6)) * PW + lane / LP;
  const int u = blockIdx.y, g = u % a.pool.Hkv;  // unit (query tile, KV head)
  const bool cand = j < a.n_cand;
  const int64_t ph = cand ? a.table[g * a.tstride + j] : -1;
  const bool ok = ph >= 0 && ph < a.pool.N;
  const int d0 = 8 * sub;
  float e[8];
  {
    float qb[8], kmin[8], kmax[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) qb[c] = a.qbar[u * D + d0 + c];  // qbar_out may be 4-byte aligned only
    const int64_t row = ok ? ph * 2 * D : 0;  // invalid pages read page 0 and are discarded
    if (kBf16) {
      const bf16_t* sm = reinterpret_cast<const bf16_t*>(a.pool.k_summary) + row + d0;
      const u32x4 wmin = *reinterpret_cast<const u32x4*>(sm);
      const u32x4 wmax = *reinterpret_cast<const u32x4*>(sm + D);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        kmin[2 * c] = __uint_as_float(wmin[c] << 16);
        kmin[2 * c + 1] = __uint_as_float(wmin[c] & 0xFFFF0000u);
        kmax[2 * c] = __uint_as_float(wmax[c] << 16);
        kmax[2 * c + 1] = __uint_as_float(wmax[c] & 0xFFFF0000u);
      }
    } else {
      const float* sm = reinterpret_cast<const float*>(a.pool.k_summary) + row + d0;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x4 n4 = *reinterpret_cast<const f32x4*>(sm + 4 * h);
        const f32x4 x4 = *reinterpret_cast<const f32x4*>(sm + D + 4 * h);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          kmin[4 * h + c] = n4[c];
          kmax[4 * h + c] = x4[c];
        }
      }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const float hi = qb[c] * kmax[c], lo = qb[c] * kmin[c];
      e[c] = hi > lo ? hi : lo;
    }
  }
  // levels s = D/2 .. 8: lane l (dimension block l) receives the block s / 8 lanes on
  // (only the lanes still in the lower half keep a meaningful sum, as in the tree)
#pragma unroll
  for (int s = D / 2; s >= 8; s >>= 1) {
#pragma unroll
    for (int c = 0; c < 8; ++c) e[c] = e[c] + __shfl_xor(e[c], s / 8, 64);
  }
  // levels s = 4, 2, 1 inside the lane
  e[0] = e[0] + e[4];
  e[1] = e[1] + e[5];
  e[2] = e[2] + e[6];
  e[3] = e[3] + e[7];
  e[0] = e[0] + e[2];
  e[1] = e[1] + e[3];
  e[0] = e[0] + e[1];
  if (cand && sub == 0) a.score[u * a.score_stride + j] = ok ? e[0] : -__builtin_inff();
}

// Mean-key scores: score_j = sum_d fp32(qbar_d * kmean_jd), the products rounded to
// fp32 and summed by the same stride-halving tree over d as the min/max scores.
template <int D>
__global__ __launch_bounds__(256) void page_score_mean_kernel(SelectArgs a) {
  // the min/max kernel's layout: D / 8 lanes per page, lane l holds dimensions
  // 8l .. 8l + 7 (two 16-byte loads of the page's fp32 mean), the same tree order
  constexpr int LP = D / 8;
  constexpr int PW = 64 / LP;
  const int lane = threadIdx.x & 63, sub = lane % LP;
  const int j = (blockIdx.x * 4 + (threadIdx.x >> 6)) * PW + lane / LP;
  const int u = blockIdx.y, g = u % a.pool.Hkv;  // unit (query tile, KV head)
  const bool cand = j < a.n_cand;
  const int64_t ph = cand ? a.table[g * a.tstride + j] : -1;
  const bool ok = ph >= 0 && ph < a.pool.N;
  const int d0 = 8 * sub;
  const float* km = a.kmean + (ok ? ph * D : 0) + d0;  // invalid pages read page 0, discarded
  const f32x4 k0 = *reinterpret_cast<const f32x4*>(km);
  const f32x4 k1 = *reinterpret_cast<const f32x4*>(km + 4);
  float e[8];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    e[c] = a.qbar[u * D + d0 + c] * k0[c];
    e[4 + c] = a.qbar[u * D + d0 + 4 + c] * k1[c];
  }
#pragma unroll
  for (int s = D / 2; s >= 8; s >>= 1) {
#pragma unroll
    for (int c = 0; c < 8; ++c) e[c] = e[c] + __shfl_xor(e[c], s / 8, 64);
  }
  e[0] = e[0] + e[4];
  e[1] = e[1] + e[5];
  e[2] = e[2] + e[6];
  e[3] = e[3] + e[7];
  e[0] = e[0] + e[2];
  e[1] = e[1] + e[3];
  e[0] = e[0] + e[1];
  if (cand && sub == 0) a.score[u * a.score_stride + j] = ok ? e[0] : -__builtin_inff();
}

// Order-preserving unsigned key of an fp32 score (-0 folded onto +0, NaN lowest).
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;  // NaN
  if ((u & 0x7FFFFFFFu) == 0u) u = 0u;             // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / 64;
// Candidates whose keys are kept in LDS (128 KiB plus one padding word per 32, so that
// threads scanning contiguous ranges of 32 hit distinct banks); longer lists are read
// from memory on every pass.
constexpr int kTopkLds = 32768;
__device__ __forceinline__ int key_slot(int j) { return j + (j >> 5); }

// Exclusive prefix sum of one int per thread over the workgroup (ids in thread order);
// writes the total. Wave scans by shuffles, then one pass over the wave totals.
__device__ __forceinline__ int block_exclusive_sum(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int before = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const int c = s_wave[w];
    before += (w < wave) ? c : 0;
    sum += c;
  }
  __syncthreads();
  *total = sum;
  return before + incl - v;
}

// One workgroup per KV head: radix select of the k-th largest (score, -id) key over
// 4 digits of 8 bits, then an ordered compaction that emits ids ascending. The keys
// are made once (into LDS when they fit); each digit is picked by one wavefront from
// suffix sums of the histogram; in the compaction each thread owns a contiguous range
// of ids, so the ties taken (the lowest ids) and the output order come from two
// workgroup-wide prefix sums.
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(SelectArgs a) {
  extern __shared__ uint32_t s_keys[];  // min(n, kTopkLds) keys
  __shared__ int s_hist[256];
  __shared__ int s_whist[kTopkWaves][256];  // per-wave histograms: no contention across waves
  __shared__ int s_wave[kTopkWaves];
  __shared__ uint32_t s_prefix;
  __shared__ int s_krem;
  const int u = blockIdx.x;  // unit (query tile u / Hkv, KV head u % Hkv)
  const int n = a.n_cand;
  const int k = a.top_k < n ? a.top_k : n;
  const float* sc = a.score + u * a.score_stride;
  int32_t* out = a.sel + u * a.sel_stride;
  // after the k ids: the chunk's pages wholly before this tile's first query
  const int tj = u / a.pool.Hkv;
  const int first_local = static_cast<int>(a.t0 >> a.pool.log2p);
  const int n_app = static_cast<int>((a.t0 + static_cast<int64_t>(tj) * a.tile) >> a.pool.log2p) - first_local;
  for (int r = threadIdx.x; r < n_app; r += kTopkThreads) out[k + r] = first_local + r;
  if (k == n) {  // every candidate
    for (int j = threadIdx.x; j < n; j += kTopkThreads) out[j] = j;
    if (threadIdx.x == 0) a.count[u] = n + n_app;
    return;
  }
  if (k <= 0) {
    if (threadIdx.x == 0) a.count[u] = n_app;
    return;
  }
  const bool in_lds = n <= kTopkLds;
  if (in_lds)
    for (int j = threadIdx.x; j < n; j += kTopkThreads) s_keys[key_slot(j)] = score_key(sc[j]);
  auto key = [&](int j) -> uint32_t { return in_lds ? s_keys[key_slot(j)] : score_key(sc[j]); };
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // The keys' range: a leading digit on which the smallest and the largest key agree
  // (with every digit above it) is that of every key, so its histogram pass would only
  // confirm it. Page scores are close together, so this usually skips the first pass.
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
  for (int j = threadIdx.x; j < n; j += kTopkThreads) {
    const uint32_t u = key(j);
    lo = u < lo ? u : lo;
    hi = u > hi ? u : hi;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint32_t ol = __shfl_xor(lo, off, 64), oh = __shfl_xor(hi, off, 64);
    lo = ol < lo ? ol : lo;
    hi = oh > hi ? oh : hi;
  }
  if (lane == 0) {
    s_whist[wave][0] = static_cast<int>(lo);
    s_whist[wave][1] = static_cast<int>(hi);
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const uint32_t wl = static_cast<uint32_t>(s_whist[w][0]), wh = static_cast<uint32_t>(s_whist[w][1]);
    lo = wl < lo ? wl : lo;
    hi = wh > hi ? wh : hi;
  }
  __syncthreads();
  uint32_t prefix = 0, mask = 0;
  int krem = k;
  bool leading = true;  // every pass so far was skipped
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (leading && ((lo ^ hi) >> shift) == 0u) {  // uniform: every key has this digit
      prefix |= lo & (255u << shift);
      mask |= 255u << shift;
      continue;
    }
    leading = false;
    for (int i = lane; i < 256; i += 64) s_whist[wave][i] = 0;
    __syncthreads();
    for (int j = threadIdx.x; j < n; j += kTopkThreads) {
      const uint32_t u = key(j);
      if ((u & mask) == prefix) atomicAdd(&s_whist[wave][(u >> shift) & 255], 1);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < 256; i += kTopkThreads) {
      int c = 0;
#pragma unroll
      for (int w = 0; w < kTopkWaves; ++w) c += s_whist[w][i];
      s_hist[i] = c;
    }
    __syncthreads();
    if (wave == 0) {
      // lane l holds digits 4l .. 4l + 3; count(digit >= d) is a suffix sum, and the
      // digit sought is the largest d with count(digit >= d) >= krem
      int c[4], lsum = 0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        c[t] = s_hist[4 * lane + t];
        lsum += c[t];
      }
      int incl = lsum;  // sum over lanes >= lane
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_down(incl, off, 64);
        if (lane + off < 64) incl += o;
      }
      int above = incl - lsum;  // keys with a digit above this lane's four
      int found = -1, rem = 0;
#pragma unroll
      for (int t = 3; t >= 0; --t) {
        if (found < 0 && above + c[t] >= krem) {
          found = 4 * lane + t;
          rem = krem - above;
        }
        above += c[t];
      }
      const unsigned long long ball = __ballot(found >= 0);
      const int top = 63 - __builtin_clzll(ball);  // digit 0 always qualifies: ball != 0
      if (lane == top) {
        s_prefix = prefix | (static_cast<uint32_t>(found) << shift);
        s_krem = rem;
      }
    }
    __syncthreads();
    prefix = s_prefix;
    krem = s_krem;
    mask |= 255u << shift;
  }
  // prefix = key of the k-th largest score; krem = how many keys equal to it to take
  // (the lowest ids among them). Thread t owns ids [t * per, (t + 1) * per).
  const int per = (n + kTopkThreads - 1) / kTopkThreads;
  const int j0 = threadIdx.x * per, j1 = min(n, j0 + per);
  int n_eq_mine = 0, n_gt_mine = 0;
  for (int j = j0; j < j1; ++j) {
    const uint32_t u = key(j);
    n_eq_mine += u == prefix;
    n_gt_mine += u > prefix;
  }
  int tot;
  const int eq_before = block_exclusive_sum(n_eq_mine, s_wave, &tot);
  const int eq_take = max(0, min(n_eq_mine, krem - eq_before));  // my lowest-id ties taken
  const int pos0 = block_exclusive_sum(n_gt_mine + eq_take, s_wave, &tot);
  int pos = pos0, eq_seen = 0;
  for (int j = j0; j < j1; ++j) {
    const uint32_t u = key(j);
    const bool eq = u == prefix;
    if (u > prefix || (eq && eq_seen < eq_take)) {
      if (pos < k) out[pos] = j;  // pos < k always; the bound guards the row
      ++pos;
    }
    eq_seen += eq;
  }
  if (threadIdx.x == 0) a.count[u] = k + n_app;
}

static void launch_scores(const SelectArgs& a, hipStream_t s) {
  const bool bf = a.pool.dtype == 0;
  const int D = a.pool.D;
  // one wavefront per workgroup: the few hundred threads per KV head spread over all CUs
  const int units = a.pool.Hkv * a.n_tiles;
  dim3 g1((a.nb * (D / 8) + 63) / 64, units);
  if (bf) OOMB_LAUNCH("qbar_partial", qbar_partial_kernel<true>, g1, dim3(64), 0, s, a);
  else OOMB_LAUNCH("qbar_partial", qbar_partial_kernel<false>, g1, dim3(64), 0, s, a);
  int n2 = 1;
  while (n2 < a.nb) n2 <<= 1;
  OOMB_LAUNCH("qbar_final", qbar_final_kernel, dim3(D, units), dim3(256), n2 * sizeof(float), s, a);
  // 64 / (D / 8) pages per wavefront, 4 wavefronts per workgroup
  const int per_wg = 4 * (64 / (D / 8));
  dim3 g4((a.n_cand + per_wg - 1) / per_wg, units);
  if (a.kmean != nullptr) {
    if (D == 128) OOMB_LAUNCH("page_score_mean", page_score_mean_kernel<128>, g4, dim3(256), 0, s, a);
    else OOMB_LAUNCH("page_score_mean", page_score_mean_kernel<64>, g4, dim3(256), 0, s, a);
    return;
  }
  if (bf && D == 128) OOMB_LAUNCH("page_score", (page_score_kernel<true, 128>), g4, dim3(256), 0, s, a);
  else if (bf) OOMB_LAUNCH("page_score", (page_score_kernel<true, 64>), g4, dim3(256), 0, s, a);
  else if (D == 128) OOMB_LAUNCH("page_score", (page_score_kernel<false, 128>), g4, dim3(256), 0, s, a);
  else OOMB_LAUNCH("page_score", (page_score_kernel<false, 64>), g4, dim3(256), 0, s, a);
}

// Workspace of oomb_select_pages_noalloc, in static device memory: each device that
// loads the library holds its own copy until the process ends. Host code must not pass
// this name to a kernel (on the host it only stands for the symbol); it uses the device
// address that select_scratch_address returns.
static __device__ __align__(256) char scratch[kSelectScratchBytes];

hipError_t select_scratch_address(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

// Scores are always computed when there are candidates (the top-k needs them unless
// k = 0 or k >= n_cand; the query summary and scores are also diagnostics).
hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  if (a.n_cand > 0) launch_scores(a, s);
  const int n_lds = a.n_cand <= kTopkLds ? a.n_cand + (a.n_cand >> 5) + 1 : 0;
  OOMB_LAUNCH("topk", topk_kernel, dim3(a.pool.Hkv * a.n_tiles), dim3(kTopkThreads),
              static_cast<size_t>(n_lds) * sizeof(uint32_t), s, a);
  return hipGetLastError();
}

}  // namespace oomb
