// Page movement between the device pools and pinned host memory for gfx950: the
// asynchronous CPU offload of the KV cache and its gradients (gist.science explainer of
// OOMB, 2.C "Asynchronous KV Cache CPU Offloading": the cache and its gradients move
// between GPU and CPU memory while other work runs; for dense and local layers the
// next layer's pages are fetched while the current one computes, for sparse layers
// only the selected pages move).
//
// The copies are kernels, not copy-engine transfers: a page list is one launch
// whatever its length, the page ids (a selection, a table) are read on the device with
// no host round trip, and pinned host memory is read or written directly through its
// device mapping. Each workgroup moves one page at a time with every lane holding
// eight 16-byte loads in flight before it stores, which keeps enough requests
// outstanding to fill the host link. Ids outside their pool are skipped.
#include "device_common.hpp"
#include "launch.hpp"
#include "profiling.hpp"

namespace oomb {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;  // 16-byte loads in flight per lane

__device__ __forceinline__ bool valid_id(int64_t id, int64_t n) { return id >= 0 && id < n; }

// One page: dst = src, 16 bytes per lane per step, all loads of a step before its stores.
__device__ __forceinline__ void copy_page(const u32x4* __restrict__ s, u32x4* __restrict__ d,
                                          int64_t nv) {
  for (int64_t v0 = threadIdx.x; v0 < nv; v0 += kThreads * kUnroll) {
    u32x4 r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t v = v0 + static_cast<int64_t>(u) * kThreads;
      if (v < nv) r[u] = s[v];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t v = v0 + static_cast<int64_t>(u) * kThreads;
      if (v < nv) d[v] = r[u];
    }
  }
}

__global__ __launch_bounds__(kThreads) void copy_pages_kernel(PageCopyArgs a) {
  const int n = a.n_dev ? min(a.n, max(0, *a.n_dev)) : a.n;
  const int64_t nv = a.page_bytes / 16;
  for (int i = blockIdx.x; i < n; i += gridDim.x) {
    const int64_t s = a.src_ids[i], d = a.dst_ids[i];
    if (!valid_id(s, a.n_src) || !valid_id(d, a.n_dst)) continue;  // uniform over the block
    copy_page(reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(a.src) + s * a.page_bytes),
              reinterpret_cast<u32x4*>(static_cast<uint8_t*>(a.dst) + d * a.page_bytes), nv);
  }
}

// fp32 pages: dst += src (one rounding per element), then optionally src = 0.
__global__ __launch_bounds__(kThreads) void add_pages_kernel(PageCopyArgs a, int zero_src) {
  const int n = a.n_dev ? min(a.n, max(0, *a.n_dev)) : a.n;
  const int64_t nv = a.page_bytes / 16;
  for (int i = blockIdx.x; i < n; i += gridDim.x) {
    const int64_t s = a.src_ids[i], d = a.dst_ids[i];
    if (!valid_id(s, a.n_src) || !valid_id(d, a.n_dst)) continue;
    f32x4* sp = reinterpret_cast<f32x4*>(static_cast<uint8_t*>(const_cast<void*>(a.src)) + s * a.page_bytes);
    f32x4* dp = reinterpret_cast<f32x4*>(static_cast<uint8_t*>(a.dst) + d * a.page_bytes);
    for (int64_t v0 = threadIdx.x; v0 < nv; v0 += kThreads * kUnroll) {
      f32x4 x[kUnroll], y[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t v = v0 + static_cast<int64_t>(u) * kThreads;
        if (v < nv) {
          x[u] = sp[v];
          y[u] = dp[v];
        }
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t v = v0 + static_cast<int64_t>(u) * kThreads;
        if (v < nv) {
#pragma unroll
          for (int j = 0; j < 4; ++j) y[u][j] += x[u][j];
          dp[v] = y[u];
          if (zero_src) sp[v] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
      }
    }
  }
}

// Selected pages of KV head g = blockIdx.y, entry j = blockIdx.x: logical page
// lp = sel[g][j] is copied from the host pages host_table[g][lp] (K and V) into the
// device staging page stage[g][j], and table[g][lp] is pointed at it.
__global__ __launch_bounds__(kThreads) void fetch_selected_kernel(FetchArgs a) {
  const int g = blockIdx.y, j = blockIdx.x;
  const int64_t cnt = a.count[g];
  if (j >= cnt || j >= a.sel_stride) return;
  const int64_t lp = a.sel[g * a.sel_stride + j];
  if (!valid_id(lp, a.n_logical)) return;
  const int64_t hp = a.host_table[g * a.host_tstride + lp];
  const int64_t sp = a.stage[g * a.stage_stride + j];
  if (!valid_id(hp, a.host_pages) || !valid_id(sp, a.dev_pages)) return;
  const int64_t nv = a.page_bytes / 16;
  copy_page(reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(a.host_k) + hp * a.page_bytes),
            reinterpret_cast<u32x4*>(static_cast<uint8_t*>(a.k_pool) + sp * a.page_bytes), nv);
  copy_page(reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(a.host_v) + hp * a.page_bytes),
            reinterpret_cast<u32x4*>(static_cast<uint8_t*>(a.v_pool) + sp * a.page_bytes), nv);
  if (threadIdx.x == 0) a.table[g * a.tstride + lp] = static_cast<int32_t>(sp);
}

// Workgroups for a page list: one per page up to a cap (a grid-stride loop takes the
// rest); the cap keeps a long list from occupying every CU slot while attention runs.
unsigned list_grid(int n) { return static_cast<unsigned>(n < 1024 ? (n > 0 ? n : 1) : 1024); }

}  // namespace

hipError_t launch_copy_pages(const PageCopyArgs& a, hipStream_t s) {
  OOMB_LAUNCH("copy_pages", copy_pages_kernel, dim3(list_grid(a.n)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_add_pages(const PageCopyArgs& a, int zero_src, hipStream_t s) {
  OOMB_LAUNCH("add_pages", add_pages_kernel, dim3(list_grid(a.n)), dim3(kThreads), 0, s, a, zero_src);
  return hipGetLastError();
}

hipError_t launch_fetch_selected(const FetchArgs& a, hipStream_t s) {
  const int64_t k = a.sel_stride;
  OOMB_LAUNCH("fetch_selected", fetch_selected_kernel,
              dim3(static_cast<unsigned>(k > 0 ? k : 1), static_cast<unsigned>(a.n_heads)),
              dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace oomb
