// C ABI of the paged chunk-attention library: argument validation, workspace
// layout and kernel dispatch. Every check runs on the host before any HIP call,
// so an invalid call returns its status without touching the device.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

#include "launch.hpp"
#include "oomb.h"
#include "scratch.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return OOMB_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(OOMB_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int ilog2(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

constexpr int64_t kMaxPos = (int64_t(1) << 31) - 4096;  // positions are 32-bit in kernels

int check_pool(const oomb_pool* p, oomb::PoolView* v, bool need_summary, bool need_grad) {
  if (p == nullptr) return fail(OOMB_ERR_INVALID, "pool descriptor is NULL");
  if (p->reserved != 0) return fail(OOMB_ERR_INVALID, "pool.reserved must be 0");
  if (p->dtype != OOMB_DTYPE_BF16 && p->dtype != OOMB_DTYPE_FP32)
    return fail(OOMB_ERR_UNSUPPORTED, "dtype %d not supported", p->dtype);
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(OOMB_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", p->head_dim);
  const int P = p->page_size;
  if (P < 16 || P > 256 || (P & (P - 1)) != 0)
    return fail(OOMB_ERR_UNSUPPORTED, "page_size %d not supported (power of two in [16, 256])", P);
  if (p->num_q_heads <= 0 || p->num_kv_heads <= 0 || p->num_q_heads % p->num_kv_heads != 0)
    return fail(OOMB_ERR_INVALID, "num_q_heads %d must be a positive multiple of num_kv_heads %d",
                p->num_q_heads, p->num_kv_heads);
  if (p->num_q_heads > 4096 || p->num_kv_heads > 4096)
    return fail(OOMB_ERR_INVALID, "too many heads");
  if (p->num_pages <= 0 || p->num_pages > (int64_t(1) << 40))
    return fail(OOMB_ERR_INVALID, "num_pages %lld out of range", (long long)p->num_pages);
  if (p->k_pool == nullptr || p->v_pool == nullptr)
    return fail(OOMB_ERR_INVALID, "k_pool / v_pool is NULL");
  if (!aligned16(p->k_pool) || !aligned16(p->v_pool))
    return fail(OOMB_ERR_INVALID, "k_pool / v_pool must be 16-byte aligned");
  if (need_summary && (p->k_summary == nullptr || !aligned16(p->k_summary)))
    return fail(OOMB_ERR_INVALID, "k_summary must be a 16-byte aligned device pointer");
  if (need_grad) {
    if (p->dk_pool == nullptr || p->dv_pool == nullptr)
      return fail(OOMB_ERR_INVALID, "dk_pool / dv_pool is NULL");
    if (!aligned16(p->dk_pool) || !aligned16(p->dv_pool))
      return fail(OOMB_ERR_INVALID, "dk_pool / dv_pool must be 16-byte aligned");
    if (p->num_grad_pages <= 0)
      return fail(OOMB_ERR_INVALID, "num_grad_pages must be positive");
  }
  v->dtype = p->dtype;
  v->P = P;
  v->log2p = ilog2(P);
  v->D = p->head_dim;
  v->Hq = p->num_q_heads;
  v->Hkv = p->num_kv_heads;
  v->N = p->num_pages;
  v->Ng = p->num_grad_pages;
  v->k_pool = p->k_pool;
  v->v_pool = p->v_pool;
  v->k_pool_w = p->k_pool;
  v->v_pool_w = p->v_pool;
  v->k_summary = p->k_summary;
  v->dk_pool = p->dk_pool;
  v->dv_pool = p->dv_pool;
  return OOMB_OK;
}

int elem_size(const oomb::PoolView& v) { return v.dtype == OOMB_DTYPE_BF16 ? 2 : 4; }

// A [head][token][D] view: pointer 16-byte aligned, strides non-negative and a
// whole number of 16-byte units.
int check_view(const void* ptr, int64_t hs, int64_t ts, int esize, const char* name) {
  if (ptr == nullptr) return fail(OOMB_ERR_INVALID, "%s is NULL", name);
  if (!aligned16(ptr)) return fail(OOMB_ERR_INVALID, "%s must be 16-byte aligned", name);
  const int unit = 16 / esize;
  if (hs < 0 || ts < 0 || hs % unit != 0 || ts % unit != 0)
    return fail(OOMB_ERR_INVALID, "%s strides (%lld, %lld) must be non-negative multiples of %d",
                name, (long long)hs, (long long)ts, unit);
  return OOMB_OK;
}

int check_table(const int32_t* t, int64_t stride, int64_t pages_needed, const char* name) {
  if (t == nullptr) return fail(OOMB_ERR_INVALID, "%s is NULL", name);
  if ((reinterpret_cast<uintptr_t>(t) & 3u) != 0) return fail(OOMB_ERR_INVALID, "%s misaligned", name);
  if (stride < pages_needed)
    return fail(OOMB_ERR_INVALID, "%s stride %lld < %lld logical pages needed", name,
                (long long)stride, (long long)pages_needed);
  return OOMB_OK;
}

struct ChunkGeom {
  int n_cand, first_local, n_local;
};

int check_chunk(const oomb::PoolView& v, int32_t n_q, int64_t t0, ChunkGeom* cg) {
  if (n_q <= 0) return fail(OOMB_ERR_INVALID, "n_q must be positive (got %d)", n_q);
  if (t0 < 0 || t0 + n_q > kMaxPos) return fail(OOMB_ERR_INVALID, "t0 %lld out of range", (long long)t0);
  if (n_q > (1 << 24)) return fail(OOMB_ERR_INVALID, "n_q %d too large", n_q);
  cg->n_cand = static_cast<int>(t0 / v.P);
  cg->first_local = cg->n_cand;
  cg->n_local = static_cast<int>((t0 + n_q - 1) / v.P) - cg->first_local + 1;
  return OOMB_OK;
}

// The attended-page geometry of a chunk, shared by the attention calls and their
// workspace queries so that both derive the same split counts. With a window (local
// attention, dense calls only) the prior pages attended are the suffix from the page
// holding position t0 - window + 1.
int attn_geometry(const oomb::PoolView& v, int32_t n_q, int64_t t0, bool has_sel,
                  int64_t sel_stride, int32_t window, oomb::AttnArgs* a) {
  ChunkGeom cg;
  int st = check_chunk(v, n_q, t0, &cg);
  if (st) return st;
  if (window < 0) return fail(OOMB_ERR_INVALID, "window must be >= 0 (got %d)", window);
  if (window > 0 && has_sel)
    return fail(OOMB_ERR_INVALID, "a window (local attention) excludes a page selection");
  int64_t prior0 = 0;
  if (window > 0 && t0 - window + 1 > 0) prior0 = (t0 - window + 1) / v.P;
  a->n_q = n_q;
  a->t0 = static_cast<int>(t0);
  a->window = window;
  a->prior0 = static_cast<int>(prior0);
  a->n_cand = static_cast<int>(cg.n_cand - prior0);
  a->first_local = cg.first_local;
  a->n_local = cg.n_local;
  const int64_t prior = has_sel ? (sel_stride < a->n_cand ? sel_stride : a->n_cand) : a->n_cand;
  a->max_att_pages = static_cast<int>(prior + cg.n_local);
  return OOMB_OK;
}

// Shared argument checks of the forward and backward calls.
int check_attn(const oomb_pool* pool, const int32_t* table, int64_t tstride, const void* q,
               int64_t q_hs, int64_t q_ts, int32_t n_q, int64_t t0, const int32_t* sel,
               int64_t sel_stride, const int32_t* count, int32_t window, bool need_grad,
               oomb::AttnArgs* a) {
  *a = oomb::AttnArgs{};
  int st = check_pool(pool, &a->pool, false, need_grad);
  if (st) return st;
  if ((st = attn_geometry(a->pool, n_q, t0, sel != nullptr, sel_stride, window, a))) return st;
  if ((st = check_table(table, tstride, a->first_local + a->n_local, "table"))) return st;
  if ((st = check_view(q, q_hs, q_ts, elem_size(a->pool), "q"))) return st;
  if (sel != nullptr) {
    if (count == nullptr) return fail(OOMB_ERR_INVALID, "count is NULL while sel is given");
    if (sel_stride < 0) return fail(OOMB_ERR_INVALID, "sel_stride must be >= 0");
  }
  a->table = table;
  a->tstride = tstride;
  a->q = q;
  a->q_hs = q_hs;
  a->q_ts = q_ts;
  a->sel = sel;
  a->sel_stride = sel_stride;
  a->count = count;
  return OOMB_OK;
}

bool use_mfma(const oomb::PoolView& v) { return v.dtype == OOMB_DTYPE_BF16 && v.D == 128; }

// The address a kernel uses for a buffer: device memory as given, pinned host memory
// through its device mapping. Anything else (pageable host memory, an unknown pointer)
// is rejected here, before a launch could fault on it. `align` is the alignment the
// kernel's accesses need.
int device_address(const void* p, uintptr_t align, const char* name, const void** out) {
  if (p == nullptr) return fail(OOMB_ERR_INVALID, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) & (align - 1))
    return fail(OOMB_ERR_INVALID, "%s must be %u-byte aligned", name, static_cast<unsigned>(align));
  hipPointerAttribute_t at{};
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return fail(OOMB_ERR_INVALID, "%s is neither device memory nor pinned host memory", name);
  }
  if (at.type == hipMemoryTypeDevice) {
    *out = p;
    return OOMB_OK;
  }
  if (at.type == hipMemoryTypeHost) {
    void* d = nullptr;
    if (hipHostGetDevicePointer(&d, const_cast<void*>(p), 0) != hipSuccess || d == nullptr) {
      (void)hipGetLastError();
      return fail(OOMB_ERR_INVALID, "%s is host memory without a device mapping", name);
    }
    *out = d;
    return OOMB_OK;
  }
  // unregistered (pageable) host memory, managed or array memory
  return fail(OOMB_ERR_INVALID, "%s is neither device memory nor pinned host memory (type %d)", name,
              static_cast<int>(at.type));
}
template <typename T>
int device_address(T* p, uintptr_t align, const char* name, T** out) {
  const void* d = nullptr;
  const int st = device_address(static_cast<const void*>(p), align, name, &d);
  *out = static_cast<T*>(const_cast<void*>(d));
  return st;
}

// Shared checks of the page-list calls.
int check_page_list(const void* src, void* dst, int64_t page_bytes, int64_t n_src, int64_t n_dst,
                    const int32_t* src_ids, const int32_t* dst_ids, int32_t n,
                    const int32_t* n_dev, oomb::PageCopyArgs* a) {
  if (page_bytes <= 0 || page_bytes % 16 != 0)
    return fail(OOMB_ERR_INVALID, "page size %lld bytes must be a positive multiple of 16",
                static_cast<long long>(page_bytes));
  if (n < 0) return fail(OOMB_ERR_INVALID, "n must be >= 0 (got %d)", n);
  if (n_src <= 0 || n_dst <= 0) return fail(OOMB_ERR_INVALID, "page counts must be positive");
  int st;
  if ((st = device_address(src, 16, "src", &a->src))) return st;
  void* d = nullptr;
  if ((st = device_address(dst, 16, "dst", &d))) return st;
  a->dst = d;
  if ((st = device_address(src_ids, 4, "src_ids", &a->src_ids))) return st;
  if ((st = device_address(dst_ids, 4, "dst_ids", &a->dst_ids))) return st;
  a->n_dev = nullptr;
  if (n_dev != nullptr && (st = device_address(n_dev, 4, "n_dev", &a->n_dev))) return st;
  a->page_bytes = page_bytes;
  a->n = n;
  a->n_src = n_src;
  a->n_dst = n_dst;
  return OOMB_OK;
}

}  // namespace

extern "C" {

const char* oomb_status_string(int status) {
  switch (status) {
    case OOMB_OK: return "ok";
    case OOMB_ERR_INVALID: return "invalid argument";
    case OOMB_ERR_UNSUPPORTED: return "unsupported configuration";
    case OOMB_ERR_HIP: return "HIP launch failure";
    case OOMB_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

const char* oomb_last_error(void) { return g_last_error.c_str(); }

int oomb_abi_version(void) { return 11; }

int oomb_kv_append(const oomb_pool* pool, const int32_t* table, int64_t table_stride,
                   const void* k_new, const void* v_new, int64_t head_stride,
                   int64_t tok_stride, int32_t n_tok, int64_t start_pos, void* stream) {
  oomb::AppendArgs a{};
  int st = check_pool(pool, &a.pool, false, false);
  if (st) return st;
  if (n_tok < 0) return fail(OOMB_ERR_INVALID, "n_tok must be >= 0");
  if (start_pos < 0 || start_pos + n_tok > kMaxPos) return fail(OOMB_ERR_INVALID, "start_pos out of range");
  if (n_tok == 0) return ok();
  if ((st = check_table(table, table_stride, (start_pos + n_tok - 1) / a.pool.P + 1, "table"))) return st;
  if ((st = check_view(k_new, head_stride, tok_stride, elem_size(a.pool), "k_new"))) return st;
  if ((st = check_view(v_new, head_stride, tok_stride, elem_size(a.pool), "v_new"))) return st;
  a.table = table;
  a.tstride = table_stride;
  a.k_new = k_new;
  a.v_new = v_new;
  a.hs = head_stride;
  a.ts = tok_stride;
  a.n_tok = n_tok;
  a.start = start_pos;
  return hip_status(oomb::launch_kv_append(a, static_cast<hipStream_t>(stream)), "kv_append");
}

int oomb_page_summarize(const oomb_pool* pool, const int32_t* table, int64_t table_stride,
                        int64_t first_page, int64_t n_pages, int64_t seq_len, void* stream) {
  oomb::SummarizeArgs a{};
  int st = check_pool(pool, &a.pool, true, false);
  if (st) return st;
  if (first_page < 0 || n_pages < 0 || seq_len < 0 || seq_len > kMaxPos)
    return fail(OOMB_ERR_INVALID, "first_page / n_pages / seq_len out of range");
  if (n_pages > 0x7FFFFFFF) return fail(OOMB_ERR_INVALID, "n_pages too large");
  if (n_pages == 0) return ok();
  if ((st = check_table(table, table_stride, first_page + n_pages, "table"))) return st;
  a.table = table;
  a.tstride = table_stride;
  a.first_page = first_page;
  a.n_pages = n_pages;
  a.seq_len = seq_len;
  return hip_status(oomb::launch_page_summarize(a, static_cast<hipStream_t>(stream)), "page_summarize");
}

static void select_layout(int Hkv, int D, int nb, int n_cand, size_t* off_qbar, size_t* off_score,
                          size_t* total) {
  const size_t partial = align256(static_cast<size_t>(Hkv) * nb * D * sizeof(float));
  const size_t qbar = align256(static_cast<size_t>(Hkv) * D * sizeof(float));
  const size_t score = align256(static_cast<size_t>(Hkv) * (n_cand > 0 ? n_cand : 1) * sizeof(float));
  *off_qbar = partial;
  *off_score = partial + qbar;
  *total = partial + qbar + score;
}

// Query tiles of a chunk of n_q queries cut into tiles of `tile` (tile <= 0 or >= n_q:
// one tile, the per-chunk selection).
static int n_tiles_of(int32_t n_q, int32_t tile) {
  return (tile <= 0 || tile >= n_q) ? 1 : (n_q + tile - 1) / tile;
}

static size_t select_bytes(const oomb::PoolView& v, int32_t n_q, int64_t t0, int32_t tile) {
  const int nt = n_tiles_of(n_q, tile);
  const int32_t tl = nt == 1 ? n_q : tile;
  const int G = v.Hq / v.Hkv;
  const int64_t nb = (static_cast<int64_t>(G) * tl + 63) / 64;
  size_t oq, os, total;
  select_layout(v.Hkv * nt, v.D, static_cast<int>(nb), static_cast<int>(t0 / v.P), &oq, &os, &total);
  return total;
}

size_t oomb_select_workspace_bytes(const oomb_pool* pool, int32_t n_q, int64_t t0) {
  oomb::PoolView v{};
  if (check_pool(pool, &v, false, false) != OOMB_OK || n_q <= 0 || t0 < 0) return 0;
  return select_bytes(v, n_q, t0, 0);
}

size_t oomb_select_tiled_workspace_bytes(const oomb_pool* pool, int32_t n_q, int64_t t0,
                                         int32_t tile) {
  oomb::PoolView v{};
  if (check_pool(pool, &v, false, false) != OOMB_OK || n_q <= 0 || t0 < 0 || tile <= 0) return 0;
  return select_bytes(v, n_q, t0, tile);
}

// Page selection from min/max summaries (kmean == nullptr) or mean-key summaries:
// every argument check, and the fill of `a` except its workspace pointers; *total is
// the workspace the call needs.
static int select_prepare(const oomb_pool* pool, const int32_t* table, int64_t table_stride,
                          const void* q, int64_t q_head_stride, int64_t q_tok_stride, int32_t n_q,
                          int64_t t0, int32_t top_k, const float* kmean, int32_t* sel,
                          int64_t sel_stride, int32_t* count, int64_t score_stride,
                          bool has_score_out, oomb::SelectArgs* a, size_t* off_qbar,
                          size_t* off_score, size_t* total, int32_t tile = 0) {
  int st = check_pool(pool, &a->pool, kmean == nullptr, false);
  if (st) return st;
  a->kmean = kmean;
  ChunkGeom cg;
  if ((st = check_chunk(a->pool, n_q, t0, &cg))) return st;
  if (top_k < 0) return fail(OOMB_ERR_INVALID, "top_k must be >= 0");
  if ((st = check_table(table, table_stride, cg.n_cand, "table"))) return st;
  if ((st = check_view(q, q_head_stride, q_tok_stride, elem_size(a->pool), "q"))) return st;
  if (count == nullptr) return fail(OOMB_ERR_INVALID, "count is NULL");
  const int nt = n_tiles_of(n_q, tile);
  const int32_t tl = nt == 1 ? n_q : tile;
  const int k = top_k < cg.n_cand ? top_k : cg.n_cand;
  // tile j's row also lists the chunk's pages wholly before its first query
  const int64_t n_app = (t0 + static_cast<int64_t>(nt - 1) * tl) / a->pool.P - t0 / a->pool.P;
  if ((k > 0 || n_app > 0) && (sel == nullptr || sel_stride < k + n_app))
    return fail(OOMB_ERR_INVALID, "sel rows must hold %lld ids (sel_stride %lld)",
                static_cast<long long>(k + n_app), static_cast<long long>(sel_stride));
  if (has_score_out && score_stride < cg.n_cand)
    return fail(OOMB_ERR_INVALID, "score_stride %lld < %d candidates", (long long)score_stride, cg.n_cand);
  const int G = a->pool.Hq / a->pool.Hkv;
  const int64_t nb = (static_cast<int64_t>(G) * tl + 63) / 64;
  if (nb > 16384) return fail(OOMB_ERR_INVALID, "G * n_q = %lld exceeds 1048576", (long long)G * tl);
  select_layout(a->pool.Hkv * nt, a->pool.D, static_cast<int>(nb), cg.n_cand, off_qbar, off_score,
                total);
  a->table = table;
  a->tstride = table_stride;
  a->q = q;
  a->q_hs = q_head_stride;
  a->q_ts = q_tok_stride;
  a->n_q = n_q;
  a->t0 = t0;
  a->top_k = top_k;
  a->sel = sel;
  a->sel_stride = sel_stride;
  a->count = count;
  a->score_stride = has_score_out ? score_stride : (cg.n_cand > 0 ? cg.n_cand : 1);
  a->n_cand = cg.n_cand;
  a->nb = static_cast<int>(nb);
  a->n_tiles = nt;
  a->tile = tl;
  a->inv = static_cast<float>(1.0 / (static_cast<double>(G) * tl));
  a->inv_last = static_cast<float>(1.0 / (static_cast<double>(G) * (n_q - (nt - 1) * tl)));
  return OOMB_OK;
}

// Launch a prepared selection with its workspace at `ws` (the caller's or the static one).
static int select_launch(oomb::SelectArgs& a, char* ws, size_t off_qbar, size_t off_score,
                         float* qbar_out, float* score_out, void* stream) {
  a.partial = reinterpret_cast<float*>(ws);
  a.qbar = qbar_out ? qbar_out : reinterpret_cast<float*>(ws + off_qbar);
  a.score = score_out ? score_out : reinterpret_cast<float*>(ws + off_score);
  return hip_status(oomb::launch_select(a, static_cast<hipStream_t>(stream)), "select_pages");
}

static int select_common(const oomb_pool* pool, const int32_t* table, int64_t table_stride,
                         const void* q, int64_t q_head_stride, int64_t q_tok_stride, int32_t n_q,
                         int64_t t0, int32_t top_k, const float* kmean, int32_t* sel,
                         int64_t sel_stride, int32_t* count, float* qbar_out, float* score_out,
                         int64_t score_stride, void* workspace, size_t workspace_bytes,
                         void* stream) {
  oomb::SelectArgs a{};
  size_t off_qbar, off_score, total;
  int st = select_prepare(pool, table, table_stride, q, q_head_stride, q_tok_stride, n_q, t0,
                          top_k, kmean, sel, sel_stride, count, score_stride, score_out != nullptr,
                          &a, &off_qbar, &off_score, &total);
  if (st) return st;
  if (workspace == nullptr || workspace_bytes < total || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return fail(OOMB_ERR_WORKSPACE, "select needs %zu bytes of 256-byte aligned workspace", total);
  return select_launch(a, static_cast<char*>(workspace), off_qbar, off_score, qbar_out,
                       score_out, stream);
}

int oomb_select_pages(const oomb_pool* pool, const int32_t* table, int64_t table_stride,
                      const void* q, int64_t q_head_stride, int64_t q_tok_stride, int32_t n_q,
                      int64_t t0, int32_t top_k, int32_t* sel, int64_t sel_stride,
                      int32_t* count, float* qbar_out, float* score_out, int64_t score_stride,
                      void* workspace, size_t workspace_bytes, void* stream) {
  return select_common(pool, table, table_stride, q, q_head_stride, q_tok_stride, n_q, t0, top_k,
                       nullptr, sel, sel_stride, count, qbar_out, score_out, score_stride,
                       workspace, workspace_bytes, stream);
}

int oomb_select_pages_noalloc(const oomb_pool* pool, const int32_t* table, int64_t table_stride,
                              const void* q, int64_t q_head_stride, int64_t q_tok_stride,
                              int32_t n_q, int64_t t0, int32_t top_k, int32_t* sel,
                              int64_t sel_stride, int32_t* count, float* qbar_out,
                              float* score_out, int64_t score_stride, void* stream) {
  oomb::SelectArgs a{};
  size_t off_qbar, off_score, total;
  int st = select_prepare(pool, table, table_stride, q, q_head_stride, q_tok_stride, n_q, t0,
                          top_k, nullptr, sel, sel_stride, count, score_stride,
                          score_out != nullptr, &a, &off_qbar, &off_score, &total);
  if (st) return st;
  if (total > oomb::kSelectScratchBytes)
    return fail(OOMB_ERR_INVALID,
                "select_pages_noalloc: this call needs %zu bytes of scratch, the static scratch "
                "holds %zu (use oomb_select_pages with a workspace)",
                total, oomb::kSelectScratchBytes);
  void* scratch_ptr = nullptr;
  hipError_t e = oomb::select_scratch_address(&scratch_ptr);
  if (e != hipSuccess)
    return fail(OOMB_ERR_HIP, "select_pages_noalloc: scratch address: %s", hipGetErrorString(e));
  return select_launch(a, static_cast<char*>(scratch_ptr), off_qbar, off_score, qbar_out,
                       score_out, stream);
}

int oomb_select_pages_tiled(const oomb_pool* pool, const int32_t* table, int64_t table_stride,
                            const void* q, int64_t q_head_stride, int64_t q_tok_stride,
                            int32_t n_q, int64_t t0, int32_t tile, int32_t top_k, int32_t* sel,
                            int64_t sel_stride, int32_t* count, float* qbar_out,
                            float* score_out, int64_t score_stride, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (tile <= 0) return fail(OOMB_ERR_INVALID, "tile must be positive (got %d)", tile);
  oomb::SelectArgs a{};
  size_t off_qbar, off_score, total;
  int st = select_prepare(pool, table, table_stride, q, q_head_stride, q_tok_stride, n_q, t0,
                          top_k, nullptr, sel, sel_stride, count, score_stride,
                          score_out != nullptr, &a, &off_qbar, &off_score, &total, tile);
  if (st) return st;
  if (workspace == nullptr || workspace_bytes < total || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return fail(OOMB_ERR_WORKSPACE, "select needs %zu bytes of 256-byte aligned workspace", total);
  return select_launch(a, static_cast<char*>(workspace), off_qbar, off_score, qbar_out,
                       score_out, stream);
}

int oomb_select_pages_mean(const oomb_pool* pool, const int32_t* table, int64_t table_stride,
                           const void* q, int64_t q_head_stride, int64_t q_tok_stride,
                           int32_t n_q, int64_t t0, int32_t top_k, const float* kmean,
                           int32_t* sel, int64_t sel_stride, int32_t* count, float* qbar_out,
                           float* score_out, int64_t score_stride, void* workspace,
                           size_t workspace_bytes, void* stream) {
  if (kmean == nullptr || !aligned16(kmean))
    return fail(OOMB_ERR_INVALID, "kmean must be a 16-byte aligned device pointer");
  return select_common(pool, table, table_stride, q, q_head_stride, q_tok_stride, n_q, t0, top_k,
                       kmean, sel, sel_stride, count, qbar_out, score_out, score_stride, workspace,
                       workspace_bytes, stream);
}

int oomb_page_summarize_mean(const oomb_pool* pool, const int32_t* table, int64_t table_stride,
                             int64_t first_page, int64_t n_pages, int64_t seq_len, float* kmean,
                             void* stream) {
  oomb::SummarizeArgs a{};
  int st = check_pool(pool, &a.pool, false, false);
  if (st) return st;
  if (kmean == nullptr || !aligned16(kmean))
    return fail(OOMB_ERR_INVALID, "kmean must be a 16-byte aligned device pointer");
  if (first_page < 0 || n_pages < 0 || seq_len < 0 || seq_len > kMaxPos)
    return fail(OOMB_ERR_INVALID, "first_page / n_pages / seq_len out of range");
  if (n_pages > 0x7FFFFFFF) return fail(OOMB_ERR_INVALID, "n_pages too large");
  if (n_pages == 0) return ok();
  if ((st = check_table(table, table_stride, first_page + n_pages, "table"))) return st;
  a.table = table;
  a.tstride = table_stride;
  a.first_page = first_page;
  a.n_pages = n_pages;
  a.seq_len = seq_len;
  a.kmean = kmean;
  return hip_status(oomb::launch_page_mean(a, static_cast<hipStream_t>(stream)), "page_summarize_mean");
}

// Forward workspace: (matrix-core path, when query tiles are split into key ranges)
// the ranges' fp32 partials.
static size_t fwd_workspace(const oomb::AttnArgs& a) {
  if (!use_mfma(a.pool)) return 0;
  return align256(oomb::fwd_partial_bytes(a, oomb::fwd_plan(a)));
}

size_t oomb_fwd_workspace_bytes(const oomb_pool* pool, int32_t n_q, int64_t t0,
                                int64_t sel_stride, int32_t window) {
  oomb::AttnArgs a{};
  if (check_pool(pool, &a.pool, false, false) != OOMB_OK) return 0;
  if (attn_geometry(a.pool, n_q, t0, sel_stride >= 0, sel_stride, window, &a) != OOMB_OK) return 0;
  return fwd_workspace(a);
}

int oomb_paged_chunk_attn_fwd(const oomb_pool* pool, const int32_t* table, int64_t table_stride,
                              const void* q, int64_t q_head_stride, int64_t q_tok_stride,
                              int32_t n_q, int64_t t0, const int32_t* sel, int64_t sel_stride,
                              const int32_t* count, int32_t window, float scale, void* o,
                              int64_t o_head_stride, int64_t o_tok_stride, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream) {
  oomb::AttnArgs a;
  int st = check_attn(pool, table, table_stride, q, q_head_stride, q_tok_stride, n_q, t0, sel,
                      sel_stride, count, window, false, &a);
  if (st) return st;
  if ((st = check_view(o, o_head_stride, o_tok_stride, elem_size(a.pool), "o"))) return st;
  if (lse == nullptr || (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(OOMB_ERR_INVALID, "lse must be a 4-byte aligned device pointer");
  if (!(scale > 0.0f) || scale > 1e30f) return fail(OOMB_ERR_INVALID, "scale must be positive and finite");
  a.scale = scale;
  a.o = o;
  a.o_hs = o_head_stride;
  a.o_ts = o_tok_stride;
  a.lse = lse;
  const size_t need = fwd_workspace(a);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need ||
                   (reinterpret_cast<uintptr_t>(workspace) & 255u)))
    return fail(OOMB_ERR_WORKSPACE, "fwd needs %zu bytes of 256-byte aligned workspace", need);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (!use_mfma(a.pool)) return hip_status(oomb::launch_fwd_scalar(a, s), "paged_chunk_attn_fwd");
  return hip_status(oomb::launch_fwd_mfma(a, oomb::fwd_plan(a), static_cast<float*>(workspace), s),
                    "paged_chunk_attn_fwd");
}

// Backward workspace: Delta [Hq][n_q] fp32, then (matrix-core path) the fp32 partials
// of the dK/dV pass when it is split over the query stream, then those of the dQ pass
// when it is split over key ranges, then the bf16 dS spill when it is used.
static size_t bwd_workspace(const oomb::AttnArgs& a, size_t* off_part, size_t* off_dq,
                            size_t* off_ds) {
  const size_t delta = align256(static_cast<size_t>(a.pool.Hq) * a.n_q * sizeof(float));
  *off_part = delta;
  *off_dq = delta;
  *off_ds = 0;
  if (!use_mfma(a.pool)) return delta;
  *off_dq = delta + align256(oomb::dkdv_partial_bytes(a, oomb::dkdv_plan(a)));
  const size_t end = *off_dq + align256(oomb::dq_partial_bytes(a, oomb::dq_plan(a)));
  const size_t ds = oomb::ds_spill_bytes(a);
  if (ds == 0) return end;
  *off_ds = end;
  return end + align256(ds);
}

size_t oomb_bwd_workspace_bytes(const oomb_pool* pool, int32_t n_q, int64_t t0,
                                int64_t sel_stride, int32_t window) {
  oomb::AttnArgs a{};
  if (check_pool(pool, &a.pool, false, false) != OOMB_OK) return 0;
  if (attn_geometry(a.pool, n_q, t0, sel_stride >= 0, sel_stride, window, &a) != OOMB_OK) return 0;
  size_t off, off_dq, off_ds;
  return bwd_workspace(a, &off, &off_dq, &off_ds);
}

int oomb_split_plan(const oomb_pool* pool, int32_t n_q, int64_t t0, int64_t sel_stride,
                    int32_t window, int32_t* out) {
  oomb::AttnArgs a{};
  int st = check_pool(pool, &a.pool, false, false);
  if (st) return st;
  if ((st = attn_geometry(a.pool, n_q, t0, sel_stride >= 0, sel_stride, window, &a))) return st;
  if (out == nullptr) return fail(OOMB_ERR_INVALID, "out must hold 6 int32");
  oomb::SplitPlan p[3] = {{1, 0}, {1, 0}, {1, 0}};
  if (use_mfma(a.pool)) {
    p[0] = oomb::fwd_plan(a);
    p[1] = oomb::dq_plan(a);
    p[2] = oomb::dkdv_plan(a);
  }
  for (int i = 0; i < 3; ++i) {
    out[2 * i] = p[i].n_ks;
    out[2 * i + 1] = p[i].n_ks > 1 ? p[i].whole : 0;
  }
  return OOMB_OK;
}

int oomb_paged_chunk_attn_bwd(const oomb_pool* pool, const int32_t* table, int64_t table_stride,
                              const int32_t* gtable, int64_t gtable_stride, const void* q,
                              int64_t q_head_stride, int64_t q_tok_stride, int32_t n_q, int64_t t0,
                              const int32_t* sel, int64_t sel_stride, const int32_t* count,
                              int32_t window, float scale, const void* o, int64_t o_head_stride,
                              int64_t o_tok_stride, const void* dout, int64_t do_head_stride,
                              int64_t do_tok_stride, const float* lse, float* dq,
                              int64_t dq_head_stride, int64_t dq_tok_stride, void* workspace,
                              size_t workspace_bytes, void* stream) {
  oomb::AttnArgs a;
  int st = check_attn(pool, table, table_stride, q, q_head_stride, q_tok_stride, n_q, t0, sel,
                      sel_stride, count, window, true, &a);
  if (st) return st;
  if ((st = check_table(gtable, gtable_stride, a.first_local + a.n_local, "gtable"))) return st;
  if ((st = check_view(o, o_head_stride, o_tok_stride, elem_size(a.pool), "o"))) return st;
  if ((st = check_view(dout, do_head_stride, do_tok_stride, elem_size(a.pool), "dout"))) return st;
  if ((st = check_view(dq, dq_head_stride, dq_tok_stride, 4, "dq"))) return st;
  if (lse == nullptr || (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(OOMB_ERR_INVALID, "lse must be a 4-byte aligned device pointer");
  if (!(scale > 0.0f) || scale > 1e30f) return fail(OOMB_ERR_INVALID, "scale must be positive and finite");
  size_t off_part = 0, off_dq = 0, off_ds = 0;
  const size_t need = bwd_workspace(a, &off_part, &off_dq, &off_ds);
  if (workspace == nullptr || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return fail(OOMB_ERR_WORKSPACE, "bwd needs %zu bytes of 256-byte aligned workspace", need);
  a.gtable = gtable;
  a.gtstride = gtable_stride;
  a.scale = scale;
  a.o = const_cast<void*>(o);
  a.o_hs = o_head_stride;
  a.o_ts = o_tok_stride;
  a.dout = dout;
  a.do_hs = do_head_stride;
  a.do_ts = do_tok_stride;
  a.lse_in = lse;
  a.dq = dq;
  a.dq_hs = dq_head_stride;
  a.dq_ts = dq_tok_stride;
  a.delta = static_cast<float*>(workspace);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (!use_mfma(a.pool)) return hip_status(oomb::launch_bwd_scalar(a, s), "paged_chunk_attn_bwd");
  float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + off_part);
  float* dq_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + off_dq);
  uint16_t* ds = off_ds ? reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + off_ds) : nullptr;
  return hip_status(oomb::launch_bwd_mfma(a, oomb::dkdv_plan(a), part, oomb::dq_plan(a), dq_part, ds, s),
                    "paged_chunk_attn_bwd");
}

int oomb_rope(const void* x, int64_t x_head_stride, int64_t x_tok_stride, void* y,
              int64_t y_head_stride, int64_t y_tok_stride, int32_t n_heads, int32_t n_tok,
              int32_t head_dim, int32_t dtype, int64_t pos0, float theta, int32_t inverse,
              void* stream) {
  if (dtype != OOMB_DTYPE_BF16 && dtype != OOMB_DTYPE_FP32)
    return fail(OOMB_ERR_UNSUPPORTED, "dtype %d", dtype);
  if (head_dim <= 0 || head_dim % 2 != 0 || head_dim > 1024)
    return fail(OOMB_ERR_INVALID, "head_dim %d must be even and at most 1024", head_dim);
  if (n_heads < 0 || n_tok < 0) return fail(OOMB_ERR_INVALID, "negative sizes");
  if (pos0 < 0 || pos0 + n_tok > kMaxPos) return fail(OOMB_ERR_INVALID, "positions out of range");
  if (!(theta > 1.0f) || theta > 1e30f) return fail(OOMB_ERR_INVALID, "theta must be > 1 and finite");
  if (x == nullptr || y == nullptr) return fail(OOMB_ERR_INVALID, "x or y is NULL");
  const int es = dtype == OOMB_DTYPE_BF16 ? 2 : 4;
  if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(y)) % es)
    return fail(OOMB_ERR_INVALID, "x / y misaligned");
  if (x_head_stride < 0 || x_tok_stride < 0 || y_head_stride < 0 || y_tok_stride < 0)
    return fail(OOMB_ERR_INVALID, "negative strides");
  if (n_heads == 0 || n_tok == 0) return ok();
  oomb::RopeArgs a{x, x_head_stride, x_tok_stride, y, y_head_stride, y_tok_stride,
                   n_heads, n_tok, head_dim, dtype, pos0, theta, inverse != 0};
  return hip_status(oomb::launch_rope(a, static_cast<hipStream_t>(stream)), "rope");
}

int oomb_copy_pages(const void* src, void* dst, int64_t page_bytes, int64_t n_src_pages,
                    int64_t n_dst_pages, const int32_t* src_ids, const int32_t* dst_ids, int32_t n,
                    const int32_t* n_dev, void* stream) {
  oomb::PageCopyArgs a{};
  const int st = check_page_list(src, dst, page_bytes, n_src_pages, n_dst_pages, src_ids, dst_ids,
                                 n, n_dev, &a);
  if (st) return st;
  if (n == 0) return OOMB_OK;
  return hip_status(oomb::launch_copy_pages(a, static_cast<hipStream_t>(stream)), "copy_pages");
}

// A copy-engine page list may break into at most max(kSdmaMaxShortRuns, n / kSdmaMinRun)
// runs of consecutive pages: runs average at least kSdmaMinRun pages, or there are few.
constexpr int64_t kSdmaMinRun = 16;
constexpr int64_t kSdmaMaxShortRuns = 16;

int oomb_copy_pages_sdma(const void* src, void* dst, int64_t page_bytes, int64_t n_src_pages,
                         int64_t n_dst_pages, const int32_t* src_ids, const int32_t* dst_ids,
                         int32_t n, void* stream) {
  if (page_bytes <= 0) return fail(OOMB_ERR_INVALID, "page size must be positive");
  if (n < 0) return fail(OOMB_ERR_INVALID, "n must be >= 0 (got %d)", n);
  if (n_src_pages <= 0 || n_dst_pages <= 0) return fail(OOMB_ERR_INVALID, "page counts must be positive");
  if (n > 0 && (src_ids == nullptr || dst_ids == nullptr))
    return fail(OOMB_ERR_INVALID, "id lists are NULL");
  // Runs of consecutive pages on both sides become one copy-engine transfer each. Each
  // transfer has a fixed cost of several microseconds, so a list that breaks into many
  // short runs (scattered pages) would crawl: such lists belong to oomb_copy_pages,
  // whose kernel gathers scattered pages at the link's speed. Refused before any HIP call.
  {
    int64_t runs = 0;
    for (int32_t i = 0; i < n; ++i)
      if (i == 0 || src_ids[i] != src_ids[i - 1] + 1 || dst_ids[i] != dst_ids[i - 1] + 1) ++runs;
    const int64_t allowed = n / kSdmaMinRun > kSdmaMaxShortRuns ? n / kSdmaMinRun : kSdmaMaxShortRuns;
    if (runs > allowed)
      return fail(OOMB_ERR_INVALID,
                  "copy_pages_sdma: %d pages in %lld runs (more than %lld); copy scattered pages "
                  "with oomb_copy_pages", n, static_cast<long long>(runs),
                  static_cast<long long>(allowed));
  }
  const void* s_dev = nullptr;
  const void* d_dev = nullptr;
  int st;
  // both ends must be device memory or pinned host memory (pageable memory would make
  // the copy synchronous); the copies themselves use the pointers as given
  if ((st = device_address(src, 1, "src", &s_dev))) return st;
  if ((st = device_address(static_cast<const void*>(dst), 1, "dst", &d_dev))) return st;
  std::vector<void*> dsts, srcs;
  std::vector<size_t> sizes;
  for (int32_t i = 0; i < n;) {
    const int64_t s0 = src_ids[i], d0 = dst_ids[i];
    if (s0 < 0 || s0 >= n_src_pages || d0 < 0 || d0 >= n_dst_pages) {
      ++i;
      continue;
    }
    int32_t len = 1;
    while (i + len < n && src_ids[i + len] == s0 + len && dst_ids[i + len] == d0 + len &&
           s0 + len < n_src_pages && d0 + len < n_dst_pages)
      ++len;
    srcs.push_back(const_cast<char*>(static_cast<const char*>(src)) + s0 * page_bytes);
    dsts.push_back(static_cast<char*>(dst) + d0 * page_bytes);
    sizes.push_back(static_cast<size_t>(len) * page_bytes);
    i += len;
  }
  // One asynchronous copy per run (the batched-copy call needs a newer HIP runtime than
  // the one PyTorch loads).
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  for (size_t r = 0; r < dsts.size(); ++r) {
    const hipError_t e = hipMemcpyAsync(dsts[r], srcs[r], sizes[r], hipMemcpyDefault, hs);
    if (e != hipSuccess) return hip_status(e, "copy_pages_sdma");
  }
  return OOMB_OK;
}

int oomb_add_pages_f32(const float* src, float* dst, int64_t page_elems, int64_t n_src_pages,
                       int64_t n_dst_pages, const int32_t* src_ids, const int32_t* dst_ids,
                       int32_t n, const int32_t* n_dev, int32_t zero_src, void* stream) {
  oomb::PageCopyArgs a{};
  if (page_elems <= 0 || page_elems % 4 != 0)
    return fail(OOMB_ERR_INVALID, "page size %lld floats must be a positive multiple of 4",
                static_cast<long long>(page_elems));
  const int st = check_page_list(src, dst, page_elems * 4, n_src_pages, n_dst_pages, src_ids,
                                 dst_ids, n, n_dev, &a);
  if (st) return st;
  if (n == 0) return OOMB_OK;
  return hip_status(oomb::launch_add_pages(a, zero_src != 0, static_cast<hipStream_t>(stream)),
                    "add_pages");
}

int oomb_fetch_selected(const oomb_pool* pool, int32_t* table, int64_t table_stride,
                        const void* host_k, const void* host_v, int64_t host_pages,
                        const int32_t* host_table, int64_t host_table_stride, const int32_t* sel,
                        int64_t sel_stride, const int32_t* count, const int32_t* stage,
                        int64_t stage_stride, int64_t n_logical, void* stream) {
  oomb::FetchArgs a{};
  oomb::PoolView v;
  int st = check_pool(pool, &v, false, false);
  if (st) return st;
  if (host_pages <= 0) return fail(OOMB_ERR_INVALID, "host_pages must be positive");
  if (sel_stride < 0) return fail(OOMB_ERR_INVALID, "sel_stride must be >= 0");
  if (stage_stride < sel_stride)
    return fail(OOMB_ERR_INVALID, "stage_stride %lld < sel_stride %lld",
                static_cast<long long>(stage_stride), static_cast<long long>(sel_stride));
  if (n_logical < 0 || table_stride < n_logical || host_table_stride < n_logical)
    return fail(OOMB_ERR_INVALID, "table strides must cover the %lld logical pages",
                static_cast<long long>(n_logical));
  if ((st = device_address(host_k, 16, "host_k", &a.host_k))) return st;
  if ((st = device_address(host_v, 16, "host_v", &a.host_v))) return st;
  if ((st = device_address(host_table, 4, "host_table", &a.host_table))) return st;
  if ((st = device_address(table, 4, "table", &a.table))) return st;
  if ((st = device_address(sel, 4, "sel", &a.sel))) return st;
  if ((st = device_address(count, 4, "count", &a.count))) return st;
  if ((st = device_address(stage, 4, "stage", &a.stage))) return st;
  if (sel_stride == 0 || n_logical == 0) return OOMB_OK;
  a.host_pages = host_pages;
  a.host_tstride = host_table_stride;
  a.k_pool = v.k_pool_w;
  a.v_pool = v.v_pool_w;
  a.dev_pages = v.N;
  a.tstride = table_stride;
  a.sel_stride = sel_stride;
  a.stage_stride = stage_stride;
  a.n_logical = n_logical;
  a.page_bytes = static_cast<int64_t>(v.P) * v.D * elem_size(v);
  a.n_heads = v.Hkv;
  return hip_status(oomb::launch_fetch_selected(a, static_cast<hipStream_t>(stream)),
                    "fetch_selected");
}

}  // extern "C"
