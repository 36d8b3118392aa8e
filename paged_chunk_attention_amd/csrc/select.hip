// Top-k page retrieval for gfx950 (gist.science explainer of OOMB, 2.D
// "Page-Level Sparse Attention": per chunk, keep only the K most relevant prior
// key pages, judged from a representative vector). The rule is Quest-style:
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

#include "device_common.hpp"
#include "launch.hpp"
#include "profiling.hpp"

namespace oomb {

constexpr int kQBlock = 64;

// Block partial sums: grid (nb, Hkv), one thread per head dimension.
template <bool kBf16>
__global__ __launch_bounds__(128) void qbar_partial_kernel(SelectArgs a) {
  const int d = threadIdx.x;
  const int b = blockIdx.x, g = blockIdx.y;
  const int D = a.pool.D;
  if (d >= D) return;
  const int G = a.pool.Hq / a.pool.Hkv;
  const int M = G * a.n_q;
  const int m0 = b * kQBlock;
  const int m1 = (m0 + kQBlock < M) ? m0 + kQBlock : M;
  float s = 0.0f;
  for (int m = m0; m < m1; ++m) {
    const int h = g * G + m / a.n_q, i = m % a.n_q;
    const int64_t off = h * a.q_hs + i * a.q_ts + d;
    float x;
    if (kBf16) x = to_f32(reinterpret_cast<const bf16_t*>(a.q)[off]);
    else x = reinterpret_cast<const float*>(a.q)[off];
    s = s + x;
  }
  a.partial[(static_cast<int64_t>(g) * a.nb + b) * D + d] = s;
}

// Pairwise tree over the block sums of one (head dimension, KV head).
__global__ __launch_bounds__(256) void qbar_final_kernel(SelectArgs a) {
  extern __shared__ float s_tree[];
  const int d = blockIdx.x, g = blockIdx.y;
  const int D = a.pool.D;
  int n2 = 1;
  while (n2 < a.nb) n2 <<= 1;
  for (int i = threadIdx.x; i < n2; i += 256)
    s_tree[i] = i < a.nb ? a.partial[(static_cast<int64_t>(g) * a.nb + i) * D + d] : 0.0f;
  __syncthreads();
  for (int s = n2 >> 1; s >= 1; s >>= 1) {
    for (int i = threadIdx.x; i < s; i += 256) s_tree[i] = s_tree[i] + s_tree[i + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) a.qbar[g * D + d] = s_tree[0] * a.inv;
}

// One wavefront per candidate page; 4 pages per workgroup.
template <bool kBf16, int D>
__global__ __launch_bounds__(256) void page_score_kernel(SelectArgs a) {
  const int lane = threadIdx.x & 63;
  const int j = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int g = blockIdx.y;
  if (j >= a.n_cand) return;
  const int64_t ph = a.table[g * a.tstride + j];
  float score;
  if (ph < 0 || ph >= a.pool.N) {
    score = -__builtin_inff();
  } else {
    constexpr int R = D / 64;
    float e[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int d = lane + 64 * r;
      const float qb = a.qbar[g * D + d];
      float kmin, kmax;
      if (kBf16) {
        const bf16_t* sm = reinterpret_cast<const bf16_t*>(a.pool.k_summary) + ph * 2 * D;
        kmin = to_f32(sm[d]);
        kmax = to_f32(sm[D + d]);
      } else {
        const float* sm = reinterpret_cast<const float*>(a.pool.k_summary) + ph * 2 * D;
        kmin = sm[d];
        kmax = sm[D + d];
      }
      const float hi = qb * kmax, lo = qb * kmin;
      e[r] = hi > lo ? hi : lo;
    }
    float acc = e[0];
    if (R == 2) acc = e[0] + e[1];  // tree level s = 64: a[d] + a[d + 64]
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
      const float other = __shfl_xor(acc, s, 64);  // lane d < s receives a[d + s]
      acc = acc + other;
    }
    score = acc;
  }
  if (lane == 0) a.score[g * a.score_stride + j] = score;
}

// Order-preserving unsigned key of an fp32 score (-0 folded onto +0, NaN lowest).
__device__ __forceinline__ uint32_t score_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;  // NaN
  if ((u & 0x7FFFFFFFu) == 0u) u = 0u;             // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

constexpr int kTopkThreads = 1024;

// Exclusive prefix count of a per-thread flag over the workgroup; returns the
// prefix and writes the total. Uses wave ballots plus one LDS pass over 16 waves.
__device__ __forceinline__ int block_exclusive_count(bool flag, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const unsigned long long ball = __ballot(flag);
  const int in_wave = __popcll(ball & ((1ull << lane) - 1ull));
  if (lane == 0) s_wave[wave] = __popcll(ball);
  __syncthreads();
  int before = 0, sum = 0;
  for (int w = 0; w < kTopkThreads / 64; ++w) {
    const int c = s_wave[w];
    before += (w < wave) ? c : 0;
    sum += c;
  }
  __syncthreads();
  *total = sum;
  return before + in_wave;
}

// One workgroup per KV head: radix select of the k-th largest (score, -id) key over
// 4 digits of 8 bits, then an ordered compaction that emits ids ascending.
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(SelectArgs a) {
  __shared__ int s_hist[256];
  __shared__ int s_wave[kTopkThreads / 64];
  __shared__ uint32_t s_prefix;
  __shared__ int s_krem;
  const int g = blockIdx.x;
  const int n = a.n_cand;
  const int k = a.top_k < n ? a.top_k : n;
  const float* sc = a.score + g * a.score_stride;
  int32_t* out = a.sel + g * a.sel_stride;
  if (k == n) {  // every candidate
    for (int j = threadIdx.x; j < n; j += kTopkThreads) out[j] = j;
    if (threadIdx.x == 0) a.count[g] = n;
    return;
  }
  if (k <= 0) {
    if (threadIdx.x == 0) a.count[g] = 0;
    return;
  }
  uint32_t prefix = 0, mask = 0;
  int krem = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += kTopkThreads) s_hist[i] = 0;
    __syncthreads();
    for (int j = threadIdx.x; j < n; j += kTopkThreads) {
      const uint32_t u = score_key(sc[j]);
      if ((u & mask) == prefix) atomicAdd(&s_hist[(u >> shift) & 255], 1);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      int above = 0, digit = 255;
      for (; digit > 0; --digit) {
        if (above + s_hist[digit] >= krem) break;
        above += s_hist[digit];
      }
      s_prefix = prefix | (static_cast<uint32_t>(digit) << shift);
      s_krem = krem - above;
    }
    __syncthreads();
    prefix = s_prefix;
    krem = s_krem;
    mask |= 255u << shift;
    __syncthreads();
  }
  // prefix = key of the k-th largest score; krem = how many keys equal to it to take.
  int base_eq = 0, base_sel = 0;
  for (int start = 0; start < n; start += kTopkThreads) {
    const int j = start + threadIdx.x;
    const uint32_t u = j < n ? score_key(sc[j]) : 0u;
    const bool gt = j < n && u > prefix;
    const bool eq = j < n && u == prefix;
    int n_eq, n_take;
    const int eq_rank = base_eq + block_exclusive_count(eq, s_wave, &n_eq);
    const bool take = gt || (eq && eq_rank < krem);
    const int pos = base_sel + block_exclusive_count(take, s_wave, &n_take);
    if (take) out[pos] = j;
    base_eq += n_eq;
    base_sel += n_take;
  }
  if (threadIdx.x == 0) a.count[g] = k;
}

static void launch_scores(const SelectArgs& a, hipStream_t s) {
  const bool bf = a.pool.dtype == 0;
  const int D = a.pool.D;
  dim3 g1(a.nb, a.pool.Hkv);
  if (bf) OOMB_LAUNCH("qbar_partial", qbar_partial_kernel<true>, g1, dim3(128), 0, s, a);
  else OOMB_LAUNCH("qbar_partial", qbar_partial_kernel<false>, g1, dim3(128), 0, s, a);
  int n2 = 1;
  while (n2 < a.nb) n2 <<= 1;
  OOMB_LAUNCH("qbar_final", qbar_final_kernel, dim3(D, a.pool.Hkv), dim3(256), n2 * sizeof(float), s, a);
  dim3 g3((a.n_cand + 3) / 4, a.pool.Hkv);
  if (bf && D == 128) OOMB_LAUNCH("page_score", (page_score_kernel<true, 128>), g3, dim3(256), 0, s, a);
  else if (bf) OOMB_LAUNCH("page_score", (page_score_kernel<true, 64>), g3, dim3(256), 0, s, a);
  else if (D == 128) OOMB_LAUNCH("page_score", (page_score_kernel<false, 128>), g3, dim3(256), 0, s, a);
  else OOMB_LAUNCH("page_score", (page_score_kernel<false, 64>), g3, dim3(256), 0, s, a);
}

// Scores are always computed when there are candidates (the top-k needs them unless
// k = 0 or k >= n_cand; the query summary and scores are also diagnostics).
hipError_t launch_select(const SelectArgs& a, hipStream_t s) {
  if (a.n_cand > 0) launch_scores(a, s);
  OOMB_LAUNCH("topk", topk_kernel, dim3(a.pool.Hkv), dim3(kTopkThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace oomb
