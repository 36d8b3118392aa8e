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
// device mapping. Each workgroup moves one page at a time with every lane holding four
// 16-byte loads in flight before it stores, and 8 workgroups are enough to keep the
// host link busy for plain copies (~55 GB/s host to device, ~50 device to host; 16
// measured the same, and added into host memory 45 GB/s against 36). Transfers run
// beside attention kernels on other streams, so they are made light for them: few
// workgroups (one per page slowed a concurrent attention step by a third; 16 cost it
// 7%, 8 cost 3%), few registers, and non-temporal accesses that stream through the
// caches instead of evicting the attention's tiles. Ids outside their pool are
// skipped.
#include "device_common.hpp"
#include "launch.hpp"
#include "profiling.hpp"

namespace oomb {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;  // 16-byte loads in flight per lane

__device__ __forceinline__ bool valid_id(int64_t id, int64_t n) { return id >= 0 && id < n; }

// One page: dst = src, 16 bytes per lane per step, all loads of a step before its stores.
__device__ __forceinline__ void copy_page(const u32x4* __restrict__ s, u32x4* __restrict__ d,
                                          int64_t nv) {
#pragma unroll 1
  for (int64_t v0 = threadIdx.x; v0 < nv; v0 += kThreads * kUnroll) {
    u32x4 r[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t v = v0 + static_cast<int64_t>(u) * kThreads;
      if (v < nv) r[u] = __builtin_nontemporal_load(s + v);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t v = v0 + static_cast<int64_t>(u) * kThreads;
      if (v < nv) __builtin_nontemporal_store(r[u], d + v);
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
    // half the copies' depth: two operands per element (few registers, see above)
    constexpr int kU = kUnroll / 2;
#pragma unroll 1
    for (int64_t v0 = threadIdx.x; v0 < nv; v0 += kThreads * kU) {
      f32x4 x[kU], y[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t v = v0 + static_cast<int64_t>(u) * kThreads;
        if (v < nv) {
          x[u] = __builtin_nontemporal_load(sp + v);
          y[u] = __builtin_nontemporal_load(dp + v);
        }
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int64_t v = v0 + static_cast<int64_t>(u) * kThreads;
        if (v < nv) {
#pragma unroll
          for (int j = 0; j < 4; ++j) y[u][j] += x[u][j];
          __builtin_nontemporal_store(y[u], dp + v);
          if (zero_src) __builtin_nontemporal_store(f32x4{0.0f, 0.0f, 0.0f, 0.0f}, sp + v);
        }
      }
    }
  }
}

// Item (g, j), KV head g and selection entry j: logical page lp = sel[g][j] is copied
// from the host pages host_table[g][lp] (K and V) into the device staging page
// stage[g][j], and table[g][lp] is pointed at it.
__global__ __launch_bounds__(kThreads) void fetch_selected_kernel(FetchArgs a) {
  const int64_t items = static_cast<int64_t>(a.n_heads) * a.sel_stride;
  const int64_t nv = a.page_bytes / 16;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int g = static_cast<int>(it / a.sel_stride);
    const int64_t j = it % a.sel_stride;
    if (j >= a.count[g]) continue;  // uniform over the block
    const int64_t lp = a.sel[g * a.sel_stride + j];
    if (!valid_id(lp, a.n_logical)) continue;
    const int64_t hp = a.host_table[g * a.host_tstride + lp];
    const int64_t sp = a.stage[g * a.stage_stride + j];
    if (!valid_id(hp, a.host_pages) || !valid_id(sp, a.dev_pages)) continue;
    copy_page(reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(a.host_k) + hp * a.page_bytes),
              reinterpret_cast<u32x4*>(static_cast<uint8_t*>(a.k_pool) + sp * a.page_bytes), nv);
    copy_page(reinterpret_cast<const u32x4*>(static_cast<const uint8_t*>(a.host_v) + hp * a.page_bytes),
              reinterpret_cast<u32x4*>(static_cast<uint8_t*>(a.v_pool) + sp * a.page_bytes), nv);
    if (threadIdx.x == 0) a.table[g * a.tstride + lp] = static_cast<int32_t>(sp);
  }
}

// Workgroups for a list of n items: one per item up to kMaxBlocks (grid-stride loops
// take the rest).
constexpr int kMaxBlocks = 8;
unsigned list_grid(int64_t n) {
  return static_cast<unsigned>(n < kMaxBlocks ? (n > 0 ? n : 1) : kMaxBlocks);
}

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
  OOMB_LAUNCH("fetch_selected", fetch_selected_kernel,
              dim3(list_grid(static_cast<int64_t>(a.n_heads) * a.sel_stride)), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace oomb
