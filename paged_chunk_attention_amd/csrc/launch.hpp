// Host-side interface between the C ABI (api.cpp) and the kernel files.
// Every launcher only enqueues work on `stream`; argument checking is done by the
// caller (api.cpp) before any of these is reached.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

namespace oomb {

struct PoolView {
  int dtype;        // 0 = bf16, 1 = fp32
  int P, log2p, D, Hq, Hkv;
  int64_t N, Ng;
  const void* k_pool;
  const void* v_pool;
  void* k_pool_w;   // writable aliases (append / summarize)
  void* v_pool_w;
  void* k_summary;
  float* dk_pool;
  float* dv_pool;
};

struct AppendArgs {
  PoolView pool;
  const int32_t* table;
  int64_t tstride;
  const void* k_new;
  const void* v_new;
  int64_t hs, ts;
  int n_tok;
  int64_t start;
};

struct SummarizeArgs {
  PoolView pool;
  const int32_t* table;
  int64_t tstride;
  int64_t first_page, n_pages, seq_len;
  float* kmean;     // mean-key summaries [N][D] fp32 (page_mean only)
};

struct SelectArgs {
  PoolView pool;
  const int32_t* table;
  int64_t tstride;
  const void* q;
  int64_t q_hs, q_ts;
  int n_q;
  int64_t t0;
  int top_k;
  int32_t* sel;
  int64_t sel_stride;
  int32_t* count;
  float* partial;   // [Hkv][nb][D]
  float* qbar;      // [Hkv][D]
  float* score;     // [Hkv][score_stride]
  int64_t score_stride;
  int n_cand;
  int nb;           // query blocks of 64 rows (of one tile)
  float inv;        // fp32(1 / (G * tile)), rounded once from fp64
  const float* kmean;  // mean-key summaries [N][D] (score = qbar . kmean), or nullptr (min/max)
  // Query tiles: the chunk's queries in tiles of `tile` (the last one n_q - (n_tiles - 1)
  // * tile long, whose reciprocal is inv_last); unit u = j * Hkv + g (tile j, KV head g)
  // owns partial[u], qbar[u], score[u], sel[u] and count[u]. One tile of n_q queries is
  // the per-chunk selection. After a tile's top-k ids its selection row lists the
  // chunk's pages wholly before the tile's first query (none for tile 0).
  int n_tiles;
  int tile;
  float inv_last;
};

struct AttnArgs {
  PoolView pool;
  const int32_t* table;
  int64_t tstride;
  const int32_t* gtable;
  int64_t gtstride;
  const void* q;
  int64_t q_hs, q_ts;
  int n_q;
  int t0;
  int n_cand;        // prior pages a dense call attends: t0 / P - prior0
  int prior0;        // first prior page a dense call attends: 0, or the window's first page
  int window;        // local attention: query p sees keys t with p - window < t; 0 = unbounded
  int first_local;   // t0 / P
  int n_local;       // local pages
  const int32_t* sel;  // nullptr = dense
  int64_t sel_stride;
  const int32_t* count;
  float scale;
  void* o;
  int64_t o_hs, o_ts;
  const void* dout;
  int64_t do_hs, do_ts;
  float* lse;        // forward output
  const float* lse_in;
  float* dq;
  int64_t dq_hs, dq_ts;
  float* delta;      // [Hq][n_q] workspace
  int max_att_pages; // upper bound of attended pages per head (grid sizing)
};

// A page list between two page arrays (device memory or the device mapping of pinned
// host memory): page i of the list goes from src page src_ids[i] to dst page
// dst_ids[i]; ids outside [0, n_src) / [0, n_dst) are skipped. The list length is n,
// or min(n, *n_dev) when n_dev (a device int32) is given.
struct PageCopyArgs {
  const void* src;
  void* dst;
  int64_t page_bytes;  // multiple of 16
  const int32_t* src_ids;
  const int32_t* dst_ids;
  int n;
  const int32_t* n_dev;
  int64_t n_src, n_dst;
};

// Fetch of the selected pages of every KV head from host pages into device staging pages.
struct FetchArgs {
  const void* host_k;
  const void* host_v;
  int64_t host_pages;
  const int32_t* host_table;  // [n_heads][host_tstride]: logical page -> host page
  int64_t host_tstride;
  void* k_pool;
  void* v_pool;
  int64_t dev_pages;
  int32_t* table;             // [n_heads][tstride]: logical page -> device page (updated)
  int64_t tstride;
  const int32_t* sel;
  int64_t sel_stride;
  const int32_t* count;
  const int32_t* stage;       // [n_heads][stage_stride]: device staging page of entry j
  int64_t stage_stride;
  int64_t n_logical;          // logical pages that may be selected (table widths)
  int64_t page_bytes;
  int n_heads;
};

hipError_t launch_copy_pages(const PageCopyArgs& a, hipStream_t s);
hipError_t launch_add_pages(const PageCopyArgs& a, int zero_src, hipStream_t s);
hipError_t launch_fetch_selected(const FetchArgs& a, hipStream_t s);

// Rotary embedding of n_tok tokens of n_heads heads ([head][token][D] views x, y; y may
// alias x), positions pos0 .. pos0 + n_tok - 1.
struct RopeArgs {
  const void* x;
  int64_t x_hs, x_ts;
  void* y;
  int64_t y_hs, y_ts;
  int n_heads, n_tok, D, dtype;
  int64_t pos0;
  float theta;
  int inverse;
};
hipError_t launch_rope(const RopeArgs& a, hipStream_t s);

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t s);
hipError_t launch_page_summarize(const SummarizeArgs& a, hipStream_t s);
hipError_t launch_page_mean(const SummarizeArgs& a, hipStream_t s);
hipError_t launch_select(const SelectArgs& a, hipStream_t s);

// Scalar kernels: any supported dtype / head_dim / page size.
hipError_t launch_fwd_scalar(const AttnArgs& a, hipStream_t s);
hipError_t launch_bwd_scalar(const AttnArgs& a, hipStream_t s);
// Matrix-core kernels: bf16, head_dim 128, page size >= 16.

// The split counts below are chosen for load balance; OOMB_FWD_SPLITS, OOMB_DQ_SPLITS
// and OOMB_DKDV_SPLITS (1..16) fix them instead (with OOMB_FWD_WHOLE, OOMB_DQ_WHOLE
// and OOMB_DKDV_WHOLE for the tiles or key blocks per KV head that stay whole), read
// at every call, so the workspace query and the call agree while the variables do not
// change. Every choice gives the same results up to rounding order; the variables
// exist so that each code path can be tested at small sizes. Returns 0 when the
// variable is unset or out of range.
inline int split_override(const char* var) {
  const char* v = getenv(var);
  if (v == nullptr) return 0;
  const int n = atoi(v);
  return n >= 1 && n <= 16 ? n : 0;
}
// How the forward and dQ passes cut query tiles into key ranges: per KV head, the
// first `whole` tiles in longest-first order run whole, every later one as n_ks
// ranges (whole = 0: all tiles cut; n_ks = 1: none). Partials are laid out for n_ks
// ranges of every row; rows of whole tiles never use theirs.
struct SplitPlan {
  int n_ks;
  int whole;
};
// Workgroups per KV head under plan p with `tiles` query tiles per head.
inline int plan_units(SplitPlan p, int tiles) {
  return p.n_ks <= 1 ? tiles : p.whole + (tiles - p.whole) * p.n_ks;
}
// The plan fixed by the environment: `var_n` as in split_override, and `var_whole`
// (default 0, clamped to the tiles per head) for the tiles that stay whole.
inline bool plan_override(const char* var_n, const char* var_whole, int tiles, SplitPlan* out) {
  const int n = split_override(var_n);
  if (n == 0) return false;
  int w = 0;
  if (const char* v = getenv(var_whole)) w = atoi(v);
  w = w < 0 ? 0 : (w > tiles ? tiles : w);
  *out = SplitPlan{n, n > 1 ? w : 0};
  return true;
}
// Refines a uniform cut into n_uniform > 1 key ranges. When the Hkv * tiles tiles are
// not a multiple of the 256 CUs (one workgroup per CU), cutting every tile is more
// than balance needs: the longest 256 * floor(T / 256) tiles run whole (the same number
// on every CU) and only the remaining r = T mod 256 are cut, into n ranges with n in
// {2, 4, 8} minimising the rounds ceil(r n / 256) / n the pieces take (smaller n on
// ties; ranges of at least 16 key blocks), so the pieces spread over all CUs and
// fewer rows need partials and a merge. Needs 256 % Hkv == 0, so that every head has a
// whole number of whole tiles; otherwise (or with no gain) the uniform cut stays.
inline SplitPlan mixed_plan(int tiles, int hkv, double smallest_blocks, int n_uniform) {
  const SplitPlan uniform{n_uniform, 0};
  const int T = tiles * hkv;
  if (n_uniform <= 1 || 256 % hkv != 0 || T <= 256 || T % 256 == 0) return uniform;
  const int r = T % 256;
  int best = 0;
  double best_rounds = 1.0;  // the remainder left whole: one more round of whole tiles
  for (int n = 2; n <= 8; n *= 2) {
    if (smallest_blocks / n < 16.0) break;
    const double rounds = static_cast<double>((r * n + 255) / 256) / n;
    if (rounds < best_rounds - 1e-9) {
      best = n;
      best_rounds = rounds;
    }
  }
  if (best == 0) return uniform;
  return SplitPlan{best, (T / 256) * 256 / hkv};
}
// Key blocks (of kb keys) that the query tile [q_first, q_first + len) visits: from
// the block its first query's window starts in (block 0 without a window) to the one
// holding its last query's own key. With a selection the prior keys count at their
// upper bound (sel_stride pages).
inline int64_t tile_key_blocks(const AttnArgs& a, int q_first, int len, int kb) {
  const int64_t P = a.pool.P;
  const int64_t prior_keys = static_cast<int64_t>(a.max_att_pages - a.n_local) * P;
  const int64_t off = a.t0 - static_cast<int64_t>(a.first_local) * P;  // chunk keys before query 0
  const int64_t q_last = (q_first + len < a.n_q ? q_first + len : a.n_q) - 1;
  const int64_t hi = prior_keys + off + q_last;  // attended index of the last query's own key
  int64_t lo = 0;
  if (a.window > 0) {
    lo = static_cast<int64_t>(a.t0) + q_first - a.window + 1 - static_cast<int64_t>(a.prior0) * P;
    if (lo < 0) lo = 0;
  }
  return hi / kb - lo / kb + 1;
}
// Matrix-core forward. A plan with n_ks > 1 cuts query tiles into key ranges; `part`
// then holds fwd_partial_bytes(a, plan) bytes of fp32 partials.
hipError_t launch_fwd_mfma(const AttnArgs& a, SplitPlan p, float* part, hipStream_t s);
SplitPlan fwd_plan(const AttnArgs& a);
size_t fwd_partial_bytes(const AttnArgs& a, SplitPlan p);
// A dK/dV plan with n_ks > 1 splits key blocks' query streams (per KV head the first
// `whole` blocks stay whole); `part` then holds dkdv_partial_bytes(a, plan) bytes of
// fp32 partials. A dQ plan with n_ks > 1 cuts query tiles into key ranges; `dq_part`
// then holds dq_partial_bytes(a, plan) bytes.
// With ds (ds_spill_bytes(a) bytes) the dK/dV pass spills its bf16 dS tiles there and
// the dQ pass reads them (Delta from launch_delta first); without, the dQ pass runs
// first and recomputes S and dP.
hipError_t launch_bwd_mfma(const AttnArgs& a, SplitPlan kv, float* part, SplitPlan dq,
                           float* dq_part, uint16_t* ds, hipStream_t s);
// dQ pass of the matrix-core backward. Without ds it recomputes dS and also computes
// Delta = rowsum(dO * O) into a.delta for the dK/dV pass (so it runs first); with ds it
// reads the dK/dV pass's spilled dS (so it runs after that pass).
hipError_t launch_dq_mfma(const AttnArgs& a, SplitPlan p, float* part, const uint16_t* ds,
                          hipStream_t s);
SplitPlan dkdv_plan(const AttnArgs& a);
size_t dkdv_partial_bytes(const AttnArgs& a, SplitPlan p);
// Workspace bytes of the dS spill for this call, or 0 when the spill is not used.
size_t ds_spill_bytes(const AttnArgs& a);
// Delta for the spilling backward, bit-identical to the one the recomputing dQ pass forms.
hipError_t launch_delta_mfma(const AttnArgs& a, hipStream_t s);
SplitPlan dq_plan(const AttnArgs& a);
size_t dq_partial_bytes(const AttnArgs& a, SplitPlan p);
// Delta_i = dO_i . O_i for the scalar backward (the matrix-core dQ pass forms its own).
hipError_t launch_delta(const AttnArgs& a, hipStream_t s);

}  // namespace oomb
