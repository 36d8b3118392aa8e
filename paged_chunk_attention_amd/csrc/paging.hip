// Paged K/V storage kernels for gfx950: appending a chunk's keys/values into
// their pages, and the per-page key min/max summaries used for page retrieval.
//
// Paging follows the gist.science explainer of OOMB, 2.B "Paged KV Cache and
// Gradient Management": the cache is a pool of fixed-size pages and grows by
// filling page slots, never by reallocating or copying what is already stored.
// The min/max summary is the per-page representative for top-k retrieval
// (explainer 2.D), in the form used by Quest (cited by the paper); the mean-key
// summary is the other plain reading of that representative (an average).
#include "device_common.hpp"
#include "launch.hpp"
#include "profiling.hpp"

namespace oomb {

// One work item = one 16-byte chunk of one token row of one KV head; K and V are
// copied together. Rows whose page is unmapped are skipped. Grid: x strides over the
// chunks of one head's tokens, y = KV head. The chunks per row (D * esize / 16) are a
// power of two, so indices come from shifts. The copy is streaming: non-temporal loads
// and stores keep it from evicting the caches.
__global__ __launch_bounds__(256) void kv_append_kernel(AppendArgs a, int log2_cpr) {
  const int esize = a.pool.dtype == 0 ? 2 : 4;
  const int g = blockIdx.y;
  const int64_t total = static_cast<int64_t>(a.n_tok) << log2_cpr;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  const char* ks = static_cast<const char*>(a.k_new) + g * a.hs * esize;
  const char* vs = static_cast<const char*>(a.v_new) + g * a.hs * esize;
  const int32_t* trow = a.table + g * a.tstride;
  const int64_t row_bytes = static_cast<int64_t>(a.pool.D) * esize;
  // Four chunks per thread per pass: all eight loads are issued before the stores.
  constexpr int kU = 4;
  for (int64_t w0 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; w0 < total;
       w0 += kU * stride) {
    u32x4 kv[kU], vv[kU];
    int64_t dst[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t w = w0 + u * stride;
      dst[u] = -1;
      if (w < total) {
        const int c = static_cast<int>(w & ((1 << log2_cpr) - 1));
        const int i = static_cast<int>(w >> log2_cpr);
        const int64_t t = a.start + i;
        const int64_t ph = trow[t >> a.pool.log2p];
        if (ph >= 0 && ph < a.pool.N) {
          const int64_t src = i * a.ts * esize + c * 16;
          dst[u] = ((ph << a.pool.log2p) + (t & (a.pool.P - 1))) * row_bytes + c * 16;
          kv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(ks + src));
          vv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vs + src));
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (dst[u] < 0) continue;
      __builtin_nontemporal_store(kv[u], reinterpret_cast<u32x4*>(static_cast<char*>(a.pool.k_pool_w) + dst[u]));
      __builtin_nontemporal_store(vv[u], reinterpret_cast<u32x4*>(static_cast<char*>(a.pool.v_pool_w) + dst[u]));
    }
  }
}

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t s) {
  const int esize = a.pool.dtype == 0 ? 2 : 4;
  const int cpr = a.pool.D * esize / 16;
  int log2_cpr = 0;
  while ((1 << log2_cpr) < cpr) ++log2_cpr;
  const int64_t per_head = static_cast<int64_t>(a.n_tok) << log2_cpr;
  int64_t blocks = (per_head + 255) / 256;
  const int64_t cap = (256 * 16 + a.pool.Hkv - 1) / a.pool.Hkv;  // ~16 waves of 256 per CU
  if (blocks > cap) blocks = cap;
  if (blocks < 1) return hipSuccess;
  OOMB_LAUNCH("kv_append", kv_append_kernel, dim3(static_cast<unsigned>(blocks), a.pool.Hkv), dim3(256), 0,
              s, a, log2_cpr);
  return hipGetLastError();
}

// Order-preserving integer key of a float: increasing in value, -0 below +0. It is
// an involution on the bit pattern, so the same function maps a key back to bits.
__device__ __forceinline__ int32_t order_key_bf16(uint32_t bits16) {
  const int32_t b = static_cast<int32_t>(static_cast<int16_t>(bits16));
  return b ^ ((b >> 31) & 0x7FFF);
}
__device__ __forceinline__ int32_t order_key_f32(uint32_t bits) {
  const int32_t b = static_cast<int32_t>(bits);
  return b ^ ((b >> 31) & 0x7FFFFFFF);
}

// One workgroup per (logical page, KV head). Each thread owns one 16-byte column
// chunk and a strided subset of the page's valid rows; the row groups are merged
// in LDS. Min/max are taken on order keys, so the result does not depend on the
// reduction order.
template <bool kBf16>
__global__ __launch_bounds__(256) void page_summarize_kernel(SummarizeArgs a) {
  constexpr int kEsize = kBf16 ? 2 : 4;
  constexpr int kPer = 16 / kEsize;  // elements per 16-byte chunk
  __shared__ int32_t s_min[256 * kPer];
  __shared__ int32_t s_max[256 * kPer];
  const int g = blockIdx.y;
  const int64_t lp = a.first_page + blockIdx.x;
  const int P = a.pool.P, D = a.pool.D;
  const int64_t n_valid64 = a.seq_len - (lp << a.pool.log2p);
  if (n_valid64 <= 0) return;
  const int n_valid = n_valid64 < P ? static_cast<int>(n_valid64) : P;
  const int64_t ph = a.table[g * a.tstride + lp];
  if (ph < 0 || ph >= a.pool.N) return;
  const int cpr = D / kPer;             // chunks per row
  const int groups = 256 / cpr;         // row groups
  const int c = threadIdx.x % cpr, rg = threadIdx.x / cpr;
  int32_t mn[kPer], mx[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) { mn[e] = 0x7FFFFFFF; mx[e] = static_cast<int32_t>(0x80000000); }
  const char* base = static_cast<const char*>(a.pool.k_pool) + (ph << a.pool.log2p) * D * kEsize;
  auto fold = [&](const u32x4& v) {
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const uint32_t word = v[e * kEsize / 4];
      const int32_t key = kBf16 ? order_key_bf16((e & 1) ? (word >> 16) : (word & 0xFFFF))
                                : order_key_f32(word);
      mn[e] = key < mn[e] ? key : mn[e];
      mx[e] = key > mx[e] ? key : mx[e];
    }
  };
  auto row = [&](int r) {
    return __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(base + (static_cast<int64_t>(r) * D + c * kPer) * kEsize));
  };
  int r = rg;
  // eight rows per thread in flight at a time (a full page of 128 rows at 16 groups)
  for (; r + 7 * groups < n_valid; r += 8 * groups) {
    u32x4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = row(r + j * groups);
#pragma unroll
    for (int j = 0; j < 8; ++j) fold(v[j]);
  }
  for (; r < n_valid; r += groups) fold(row(r));
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    s_min[rg * D + c * kPer + e] = mn[e];
    s_max[rg * D + c * kPer + e] = mx[e];
  }
  __syncthreads();
  for (int d = threadIdx.x; d < D; d += 256) {
    int32_t lo = 0x7FFFFFFF, hi = static_cast<int32_t>(0x80000000);
    const int used = groups < n_valid ? groups : n_valid;
    for (int j = 0; j < used; ++j) {
      const int32_t x = s_min[j * D + d], y = s_max[j * D + d];
      lo = x < lo ? x : lo;
      hi = y > hi ? y : hi;
    }
    char* out = static_cast<char*>(a.pool.k_summary) + ph * 2 * D * kEsize;
    if (kBf16) {
      reinterpret_cast<uint16_t*>(out)[d] = static_cast<uint16_t>(order_key_bf16(static_cast<uint32_t>(lo) & 0xFFFF));
      reinterpret_cast<uint16_t*>(out)[D + d] = static_cast<uint16_t>(order_key_bf16(static_cast<uint32_t>(hi) & 0xFFFF));
    } else {
      reinterpret_cast<uint32_t*>(out)[d] = static_cast<uint32_t>(order_key_f32(static_cast<uint32_t>(lo)));
      reinterpret_cast<uint32_t*>(out)[D + d] = static_cast<uint32_t>(order_key_f32(static_cast<uint32_t>(hi)));
    }
  }
}

// Mean-key summary of a page (the other reading of the page representative, a plain
// average): kmean[ph][d] = fp32(sum) * fp32(1 / n_valid), the sum taken in fp32 from
// +0 over the page's valid tokens in slot order, 1 / n_valid rounded once from fp64.
// Thread t of the grid owns page blockIdx.x * 16 + t / (D / 8) of KV head blockIdx.y
// and head dimensions 8 (t % (D / 8)) .. +7: one 16-byte load per token, sixteen
// issued together (branch-free, so that no load waits for the previous one), each
// dimension summed strictly in token order.
template <bool kBf16>
__global__ __launch_bounds__(256) void page_mean_kernel(SummarizeArgs a) {
  const int D = a.pool.D;
  const int lpp = D / 8;  // threads per page
  const int64_t lp = a.first_page + static_cast<int64_t>(blockIdx.x) * (256 / lpp) + threadIdx.x / lpp;
  const int d0 = 8 * (threadIdx.x % lpp);
  const int g = blockIdx.y;
  if (lp >= a.first_page + a.n_pages) return;
  const int P = a.pool.P;
  const int64_t n_valid64 = a.seq_len - (lp << a.pool.log2p);
  if (n_valid64 <= 0) return;
  const int n_valid = n_valid64 < P ? static_cast<int>(n_valid64) : P;
  const int64_t ph = a.table[g * a.tstride + lp];
  if (ph < 0 || ph >= a.pool.N) return;
  const int64_t page0 = (ph << a.pool.log2p) * D + d0;  // element offset of token 0
  constexpr int kGroup = 16;
  float s[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) s[c] = 0.0f;
  for (int t0 = 0; t0 < n_valid; t0 += kGroup) {
    float x[kGroup][8];
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      const bool live = t0 + u < n_valid;
      const int64_t off = page0 + static_cast<int64_t>(live ? t0 + u : 0) * D;
      if (kBf16) {
        const u32x4 w = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.pool.k_pool) + off));
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          x[u][2 * c] = live ? __uint_as_float(w[c] << 16) : 0.0f;
          x[u][2 * c + 1] = live ? __uint_as_float(w[c] & 0xFFFF0000u) : 0.0f;
        }
      } else {
        const float* src = static_cast<const float*>(a.pool.k_pool) + off;
        const f32x4 lo = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src));
        const f32x4 hi = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src + 4));
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          x[u][c] = live ? lo[c] : 0.0f;
          x[u][4 + c] = live ? hi[c] : 0.0f;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kGroup; ++u) {
      if (t0 + u < n_valid) {
#pragma unroll
        for (int c = 0; c < 8; ++c) s[c] = s[c] + x[u][c];
      }
    }
  }
  const float inv = static_cast<float>(1.0 / static_cast<double>(n_valid));
  float* dst = a.kmean + ph * D + d0;
#pragma unroll
  for (int c = 0; c < 8; ++c) dst[c] = s[c] * inv;
}

hipError_t launch_page_mean(const SummarizeArgs& a, hipStream_t s) {
  if (a.n_pages <= 0) return hipSuccess;
  const int pages_per_block = 256 / (a.pool.D / 8);
  dim3 grid(static_cast<unsigned>((a.n_pages + pages_per_block - 1) / pages_per_block), a.pool.Hkv);
  if (a.pool.dtype == 0)
    OOMB_LAUNCH("page_mean", page_mean_kernel<true>, grid, dim3(256), 0, s, a);
  else
    OOMB_LAUNCH("page_mean", page_mean_kernel<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_page_summarize(const SummarizeArgs& a, hipStream_t s) {
  if (a.n_pages <= 0) return hipSuccess;
  dim3 grid(static_cast<unsigned>(a.n_pages), a.pool.Hkv);
  if (a.pool.dtype == 0)
    OOMB_LAUNCH("page_summarize", page_summarize_kernel<true>, grid, dim3(256), 0, s, a);
  else
    OOMB_LAUNCH("page_summarize", page_summarize_kernel<false>, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace oomb
