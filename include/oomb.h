/*
 * oomb.h - C ABI of the paged chunk-attention library (MI355X / gfx950).
 *
 * The library computes the per-chunk attention step of OOMB's chunk-recurrent
 * long-context training (arXiv 2602.02108): one chunk of queries attends, causally,
 * to a key/value cache kept in fixed-size pages; the backward pass recomputes the
 * attention probabilities and adds the key/value gradients, in place, into a paged
 * gradient pool; optionally only the top-k most relevant prior pages are attended.
 *   - chunking and recomputation: gist.science explainer of the paper, 2.A
 *     "Chunk-Recurrent Training with Activation Recomputation";
 *   - paged K/V and paged K/V gradients, in-place accumulation, no autograd:
 *     explainer 2.B "Paged KV Cache and Gradient Management"; the mlsanity page's
 *     abstract (pages managed for the key/value cache and for its gradients alike);
 *   - top-k page retrieval: explainer 2.D "Page-Level Sparse Attention".
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every buffer argument is a DEVICE pointer owned by the caller. The library never
 *    allocates, frees or synchronises; every call only enqueues kernels on `stream`
 *    (a hipStream_t passed as void*, NULL = the default stream) and returns.
 *  - Return value: OOMB_OK, or an error code. On an error no kernel was launched,
 *    except OOMB_ERR_HIP, which reports a failed launch (hipGetLastError). A short
 *    description of the last error of the calling thread: oomb_last_error().
 *  - Calls are stateless and reentrant. Two calls that write the same memory race
 *    unless they are ordered (same stream, or events).
 *  - Element strides are counted in elements of the tensor's dtype. The last
 *    dimension (head_dim) is always contiguous. Q/O/dO/dQ are viewed as
 *    [head][token][head_dim] with (head_stride, tok_stride), which accepts both
 *    [H, C, D] and [C, H, D] storage. For bf16 tensors, pointers must be 16-byte
 *    aligned and strides multiples of 8; for fp32, 16-byte aligned and multiples of 4.
 *  - Token positions are absolute positions in the sequence. Token t of KV head g
 *    lives in logical page t / P, slot t % P, i.e. physical page table[g][t / P].
 *  - Page-table CONTENTS are not read on the host. Kernels skip (never touch) a row
 *    whose physical id is outside [0, num_pages) or whose selected logical id is
 *    outside the candidate range, so a bad table gives wrong results, not a fault.
 *    A well-formed table is injective within a call: no physical page appears twice.
 */
#ifndef OOMB_H
#define OOMB_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  OOMB_OK = 0,
  OOMB_ERR_INVALID = 1,      /* bad argument: null pointer, bad size, stride or alignment */
  OOMB_ERR_UNSUPPORTED = 2,  /* dtype / head_dim / page_size combination not built */
  OOMB_ERR_HIP = 3,          /* a kernel launch failed */
  OOMB_ERR_WORKSPACE = 4     /* workspace missing or smaller than the query function says */
};

enum { OOMB_DTYPE_BF16 = 0, OOMB_DTYPE_FP32 = 1 };

/* One layer's paged storage (host-side descriptor; the arrays are device memory).
 *   k_pool, v_pool : [num_pages, page_size, head_dim]       in `dtype`
 *   k_summary      : [num_pages, 2, head_dim]                in `dtype`
 *                    row 0 = per-dimension minimum of the page's keys, row 1 = maximum
 *                    (needed by oomb_page_summarize and oomb_select_pages only)
 *   dk_pool,dv_pool: [num_grad_pages, page_size, head_dim]  fp32
 *                    (needed by oomb_paged_chunk_attn_bwd only)
 * Supported: dtype BF16 or FP32; head_dim 64 or 128; page_size a power of two in
 * [16, 256]. The matrix-core kernels serve bf16 with head_dim 128; every other
 * supported combination runs on the scalar kernels. */
typedef struct oomb_pool {
  int32_t dtype;
  int32_t page_size;
  int32_t head_dim;
  int32_t num_q_heads;     /* Hq, a multiple of num_kv_heads (grouped-query attention) */
  int32_t num_kv_heads;    /* Hkv; query head h reads KV head h / (Hq / Hkv) */
  int32_t reserved;        /* must be 0 */
  int64_t num_pages;
  int64_t num_grad_pages;
  void* k_pool;
  void* v_pool;
  void* k_summary;
  float* dk_pool;
  float* dv_pool;
} oomb_pool;

const char* oomb_status_string(int status);
/* Description of the last error returned on the calling thread ("" if none). */
const char* oomb_last_error(void);
/* ABI version: bumped whenever a signature or a layout changes, or a call is added. */
int oomb_abi_version(void);

/* KV append - write a chunk's keys and values into their pages (explainer 2.B:
 * the paged cache grows by filling the next page slots, never by reallocation).
 * For every KV head g and token t in [start_pos, start_pos + n_tok):
 *   k_pool[table[g*table_stride + t/P]][t%P][:] = k_new[g*head_stride + (t-start_pos)*tok_stride + :]
 * and the same for V. A bitwise copy; no other slot is touched.
 * table: int32 [Hkv][table_stride]; (start_pos + n_tok - 1) / P must be < table_stride.
 * n_tok == 0 is a no-op. */
int oomb_kv_append(const oomb_pool* pool, const int32_t* table, int64_t table_stride,
                   const void* k_new, const void* v_new, int64_t head_stride,
                   int64_t tok_stride, int32_t n_tok, int64_t start_pos, void* stream);

/* Page summarize - per-page key summary used to rank pages (explainer 2.D retrieves
 * pages by scoring them against an averaged stand-in vector; the min/max form follows
 * Quest, cited by the paper). For KV head g and logical page j in
 * [first_page, first_page+n_pages):
 *   k_summary[phys][0][d] = min, k_summary[phys][1][d] = max of K[t][d] over the
 *   page's tokens t with t < seq_len,
 * under the total order of values in which -0 < +0 (result independent of the
 * reduction order). Pages with no token below seq_len are left unchanged.
 * first_page + n_pages must be <= table_stride. */
int oomb_page_summarize(const oomb_pool* pool, const int32_t* table, int64_t table_stride,
                        int64_t first_page, int64_t n_pages, int64_t seq_len, void* stream);

/* Bytes of device workspace oomb_select_pages needs for n_q queries after t0 prior
 * tokens (256-byte aligned pointer). */
size_t oomb_select_workspace_bytes(const oomb_pool* pool, int32_t n_q, int64_t t0);

/* Page select - top-k page retrieval (explainer 2.D), one selection per KV head
 * shared by all its query heads and all n_q queries. In IEEE fp32, no fused
 * multiply-add, in this fixed order (bit-reproducible):
 *   1. qbar[d]: the mean of x_m = q[g*G + m/n_q][m%n_q][d], m in [0, G*n_q)
 *      (G = Hq/Hkv): sequential sums from +0 over blocks of 64 consecutive m, then a
 *      stride-halving tree over the block sums zero-padded to a power of two, then
 *      one multiply by fp32(1/(G*n_q)) (reciprocal taken in fp64).
 *   2. For candidate logical pages j in [0, t0/P) (complete pages before the chunk):
 *      e[d] = qbar[d]*kmax[d] if that product is greater than qbar[d]*kmin[d],
 *      else qbar[d]*kmin[d]; score_j = stride-halving tree sum of e over d.
 *   3. Keep the min(top_k, t0/P) pages with the largest score, ties to the lower
 *      logical id (-0 and +0 compare equal; a NaN score ranks below every number,
 *      -inf included, NaNs tying with each other), written in ascending id order to
 *      sel[g*sel_stride + 0..count[g]).
 * The chunk's own pages (including one straddling t0) are never candidates: the
 * attention calls always add them. q: [Hq][n_q][D] view. sel_stride >=
 * min(top_k, t0/P). qbar_out ([Hkv][D] fp32) and score_out ([Hkv][score_stride]
 * fp32, score_stride >= t0/P) are optional diagnostics (NULL to skip).
 * top_k >= 0; top_k >= t0/P selects every candidate. */
int oomb_select_pages(const oomb_pool* pool, const int32_t* table, int64_t table_stride,
                      const void* q, int64_t q_head_stride, int64_t q_tok_stride,
                      int32_t n_q, int64_t t0, int32_t top_k, int32_t* sel,
                      int64_t sel_stride, int32_t* count, float* qbar_out,
                      float* score_out, int64_t score_stride, void* workspace,
                      size_t workspace_bytes, void* stream);

/* Page select per query tile, a finer selection granularity (the explainer, 2.D, leaves
 * the unit of selection open): the chunk's n_q queries are cut into n_tiles =
 * ceil(n_q / tile) tiles of `tile` queries (the last one shorter when tile does not
 * divide n_q), and each (tile, KV head) selects its own top-k candidate pages by the
 * steps of oomb_select_pages, with qbar taken over the tile's rows only: in step 1 read
 * n_q as the tile's length and m over the tile's queries, in the same block, tree and
 * reciprocal order. Candidates are still the complete pages before the chunk (t0/P).
 * Outputs are tile-major, unit u = j * Hkv + g for tile j and KV head g:
 *   sel [n_tiles][Hkv][sel_stride]: tile j's top-k ids ascending, then the chunk's
 *       pages that lie wholly before the tile's first query, logical ids t0/P ..
 *       (t0 + j*tile)/P - 1 (none for tile 0);
 *   count [n_tiles][Hkv]: how many ids the row holds;
 *   qbar_out [n_tiles][Hkv][D], score_out [n_tiles][Hkv][score_stride]: optional.
 * sel_stride >= min(top_k, t0/P) + (t0 + (n_tiles - 1)*tile)/P - t0/P.
 * Tile j's attention is then the forward / backward call on its queries (first
 * position t0 + j*tile, n_q = its length) with sel + j*Hkv*sel_stride and count + j*Hkv
 * as the selection: the tile attends its own prior pages and every chunk page up to
 * each query. tile >= n_q gives exactly oomb_select_pages' results. The workspace holds
 * oomb_select_tiled_workspace_bytes(pool, n_q, t0, tile) bytes (256-byte aligned). */
size_t oomb_select_tiled_workspace_bytes(const oomb_pool* pool, int32_t n_q, int64_t t0,
                                         int32_t tile);
int oomb_select_pages_tiled(const oomb_pool* pool, const int32_t* table, int64_t table_stride,
                            const void* q, int64_t q_head_stride, int64_t q_tok_stride,
                            int32_t n_q, int64_t t0, int32_t tile, int32_t top_k, int32_t* sel,
                            int64_t sel_stride, int32_t* count, float* qbar_out,
                            float* score_out, int64_t score_stride, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Page select without any allocation, for callers that cannot allocate device memory
 * (code being captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc): oomb_select_pages with the same arguments and results, minus the
 * workspace, which is instead a static device array of 8 MiB (8388608 bytes) inside
 * the library, one per device, held until the process ends. The call needs the bytes
 * oomb_select_workspace_bytes reports; above 8 MiB it returns OOMB_ERR_INVALID before
 * any launch (the 4M-token chunk of 8192 queries with 28/4 heads of 128 needs
 * 2.4 MiB). It calls no allocator. Every call on one device uses that device's array,
 * so calls that may overlap on one device (different streams, no ordering between
 * them) race on it: order them. Nothing in the array needs to be zero on entry. */
int oomb_select_pages_noalloc(const oomb_pool* pool, const int32_t* table, int64_t table_stride,
                              const void* q, int64_t q_head_stride, int64_t q_tok_stride,
                              int32_t n_q, int64_t t0, int32_t top_k, int32_t* sel,
                              int64_t sel_stride, int32_t* count, float* qbar_out,
                              float* score_out, int64_t score_stride, void* stream);

/* Rotary position embedding of a chunk's queries or keys by their absolute positions
 * pos0 + i (the chunk-recurrent layer keeps every token's global position, explainer
 * 2.A). x and y are [n_heads][n_tok][head_dim] views (element strides; y may equal x)
 * of dtype OOMB_DTYPE_BF16 or _FP32; head_dim even. Pairs (d, d + head_dim/2):
 *   y_d = x_d cos a - x_{d+h} sin a,  y_{d+h} = x_{d+h} cos a + x_d sin a,
 *   a = (pos0 + i) * theta^(-2d/head_dim)   (h = head_dim/2; inverse != 0: a -> -a,
 * the transpose, which is what the backward applies to gradients). Angles in fp64,
 * rotation in fp32, one rounding to the dtype. */
int oomb_rope(const void* x, int64_t x_head_stride, int64_t x_tok_stride, void* y,
              int64_t y_head_stride, int64_t y_tok_stride, int32_t n_heads, int32_t n_tok,
              int32_t head_dim, int32_t dtype, int64_t pos0, float theta, int32_t inverse,
              void* stream);

/* Selector variant: the page representative read as a plain average of the page's keys
 * (the explainer's averaged stand-in vector, 2.D, read the other way).
 * oomb_page_summarize_mean writes kmean[phys] (fp32 [N][D], 16-byte aligned, caller
 * owned) for logical pages [first_page, first_page + n_pages) of every KV head: the
 * keys widened to fp32 and summed from +0 in token order over the tokens below
 * seq_len, then multiplied by fp32(1 / n_valid) (reciprocal in fp64); pages with no
 * such token are left unchanged. oomb_select_pages_mean is oomb_select_pages with
 *   score_j = stride-halving tree over d of fp32(qbar[d] * kmean[phys_j][d])
 * (same qbar, same tree, same top-k rule, same workspace size); k_summary is not
 * used, and kmean must be the 16-byte aligned array the summary call writes. */
int oomb_page_summarize_mean(const oomb_pool* pool, const int32_t* table, int64_t table_stride,
                             int64_t first_page, int64_t n_pages, int64_t seq_len, float* kmean,
                             void* stream);
int oomb_select_pages_mean(const oomb_pool* pool, const int32_t* table, int64_t table_stride,
                           const void* q, int64_t q_head_stride, int64_t q_tok_stride,
                           int32_t n_q, int64_t t0, int32_t top_k, const float* kmean,
                           int32_t* sel, int64_t sel_stride, int32_t* count, float* qbar_out,
                           float* score_out, int64_t score_stride, void* workspace,
                           size_t workspace_bytes, void* stream);

/* Chunk attention forward (explainer 2.A/2.B/2.D). Query i of the chunk sits at
 * position t0 + i; q head h uses KV head g = h / (Hq/Hkv). It attends to key t iff
 *   t <= t0 + i  and  page(t) is in  Sel_g U Local  (and t > t0 + i - window),
 * where Local = [t0/P, (t0+n_q-1)/P] (the chunk's own pages, appended beforehand)
 * and Sel_g = sel[g*sel_stride + 0..count[g]) (count clamped to [0, sel_stride] and
 * to t0/P), or every page before t0/P when sel == NULL (dense).
 * window > 0 is local attention, the attention of the sparse layers of sparse-native
 * models (explainer 2.D): each query sees only the `window` most recent positions up
 * to its own. It requires sel == NULL; only the pages the windows reach are read.
 * window == 0: no window; window < 0 is invalid.
 *   s_t = scale * q.k_t ;  LSE = ln sum_t exp(s_t) ;  O = sum_t exp(s_t - LSE) v_t
 * Writes o ([Hq][n_q][D] view, dtype of the pool) and lse (fp32 [Hq][n_q],
 * contiguous). Keys beyond t0 + n_q are never read into the result. The workspace
 * must hold oomb_fwd_workspace_bytes(pool, n_q, t0, sel ? sel_stride : -1, window) bytes at a
 * 256-byte aligned address (it may be NULL when that is 0); its contents on entry do
 * not matter. */
int oomb_paged_chunk_attn_fwd(const oomb_pool* pool, const int32_t* table,
                              int64_t table_stride, const void* q, int64_t q_head_stride,
                              int64_t q_tok_stride, int32_t n_q, int64_t t0,
                              const int32_t* sel, int64_t sel_stride, const int32_t* count,
                              int32_t window, float scale, void* o, int64_t o_head_stride,
                              int64_t o_tok_stride, float* lse, void* workspace,
                              size_t workspace_bytes, void* stream);

/* Bytes of device workspace oomb_paged_chunk_attn_fwd needs (256-byte aligned) for
 * n_q queries after t0 prior tokens, with at most sel_stride selected prior pages per
 * KV head (sel_stride < 0: dense) and the call's window. It holds fp32 partial
 * outputs when the query tiles' key blocks are cut into ranges so that the work
 * spreads evenly over the GPU (an in-order merge then combines them: results stay
 * bit-reproducible). May be 0. Returns 0 for invalid arguments. */
size_t oomb_fwd_workspace_bytes(const oomb_pool* pool, int32_t n_q, int64_t t0,
                                int64_t sel_stride, int32_t window);

/* Bytes of device workspace oomb_paged_chunk_attn_bwd needs (256-byte aligned) for
 * n_q queries after t0 prior tokens, with at most sel_stride selected prior pages
 * per KV head (sel_stride < 0: dense, every prior page). It holds Delta and, when
 * the dK/dV pass is split over the query stream or the dQ pass over key ranges (so
 * that the work spreads evenly over the GPU), their fp32 partials; and, on the
 * matrix-core path without a window, the bf16 dS of every (64-query tile, 128-key
 * block) the key pass visits: Hq * ceil(keys / 128) * ceil(n_q / 64) * 16 KiB, with
 * keys = (selected + local pages) * page_size. The dQ pass then reads dS instead of
 * recomputing it (27.4 GiB for a 4096-query chunk over a 128K-token dense context,
 * 2.6 GiB over 64 selected pages). That part is included only while it stays within
 * the environment variable OOMB_DS_SPILL_MAX_MIB (MiB, default 32768; 0 = never),
 * read at every call like the split variables: the backward then recomputes dS in
 * the dQ pass instead, with the same dK/dV bits and dQ within rounding.
 * Returns 0 for invalid arguments. */
size_t oomb_bwd_workspace_bytes(const oomb_pool* pool, int32_t n_q, int64_t t0,
                                int64_t sel_stride, int32_t window);

/* How the forward and backward calls of this geometry (arguments as for the workspace
 * queries) spread their work over the GPU, for inspection and tests; the calls compute
 * the same themselves. out[0], out[1]: key ranges per query tile of the forward, and
 * query tiles per KV head (the longest first) that stay whole; out[2], out[3]: the same
 * for the dQ pass; out[4], out[5]: parts of each key block's query stream in the dK/dV
 * pass, and key blocks per KV head (in attended order) that stay whole. The scalar
 * kernels (fp32, head_dim 64) do not split: 1, 0 for each pass. The choice depends on
 * the geometry and the OOMB_*_SPLITS / OOMB_*_WHOLE environment variables only, never
 * on the device. Returns OOMB_OK, or OOMB_ERR_INVALID (out untouched). */
int oomb_split_plan(const oomb_pool* pool, int32_t n_q, int64_t t0, int64_t sel_stride,
                    int32_t window, int32_t* out);

/* Chunk attention backward, with the attention probabilities recomputed from the
 * saved LSE (explainer 2.A: activations are recomputed just before use) and the
 * key/value gradients added in place into the paged gradient pool (explainer 2.B:
 * in-place accumulation without intermediate buffers). Same q / table / sel / count /
 * window / scale as the forward call it differentiates; o and lse are that call's
 * outputs.
 * For the loss sum(dout * O):
 *   Delta_i = dO_i . O_i ; P_it = exp(s_it - LSE_i) ; dS_it = P_it (dO_i . v_t - Delta_i)
 *   dq[h][i]  = scale * sum_t dS_it k_t                        (fp32, OVERWRITTEN)
 *   dk_pool[gtable[g][t/P]][t%P] += scale * sum_{h in g, i} dS_it q_hi   (fp32, ADDED)
 *   dv_pool[gtable[g][t/P]][t%P] += sum_{h in g, i} P_it dO_hi           (fp32, ADDED)
 * Every gradient row is written by exactly one workgroup (a plain read-modify-write,
 * no atomics, no races; when the key pass is split over the query stream, the split
 * partials go through the workspace and one merge kernel adds them in split order),
 * so results are bit-reproducible. The caller zeroes the gradient pool when a step
 * starts. The workspace must hold oomb_bwd_workspace_bytes(pool, n_q, t0,
 * sel ? sel_stride : -1, window) bytes. gtable: int32 [Hkv][gtable_stride], may alias
 * table. dq: fp32 [Hq][n_q][D] view. */
int oomb_paged_chunk_attn_bwd(const oomb_pool* pool, const int32_t* table,
                              int64_t table_stride, const int32_t* gtable,
                              int64_t gtable_stride, const void* q, int64_t q_head_stride,
                              int64_t q_tok_stride, int32_t n_q, int64_t t0,
                              const int32_t* sel, int64_t sel_stride, const int32_t* count,
                              int32_t window, float scale, const void* o,
                              int64_t o_head_stride, int64_t o_tok_stride, const void* dout,
                              int64_t do_head_stride, int64_t do_tok_stride,
                              const float* lse, float* dq, int64_t dq_head_stride,
                              int64_t dq_tok_stride, void* workspace, size_t workspace_bytes,
                              void* stream);

/* ---- Page movement between the device and pinned host memory ----------------------
 * The asynchronous CPU offload of the KV cache and its gradients (explainer 2.C): pages
 * move between the device pools and host copies while other work runs on other
 * streams (for dense and local layers, the next layer's pages are fetched while the
 * current layer computes; for sparse layers only the selected pages move). Every
 * buffer below is device memory or pinned host memory (hipHostMalloc, or a torch
 * tensor made with pin_memory=True), which the kernels read and write directly
 * through its device mapping; pageable memory is rejected with OOMB_ERR_INVALID before
 * any launch. Page-id lists are int32 arrays in such memory, read on the device, so a
 * list computed on the GPU (a selection) needs no host round trip. Ids outside their
 * page array are skipped. The calls are asynchronous on `stream`; the caller keeps
 * the buffers alive and orders other streams with events. */

/* dst page dst_ids[i] = src page src_ids[i], for i < n (or i < min(n, *n_dev) when
 * n_dev, a device int32, is given). src holds n_src_pages pages of page_bytes bytes
 * (a positive multiple of 16) and dst n_dst_pages; src and dst must not overlap.
 * Copies are bitwise. */
int oomb_copy_pages(const void* src, void* dst, int64_t page_bytes, int64_t n_src_pages,
                    int64_t n_dst_pages, const int32_t* src_ids, const int32_t* dst_ids,
                    int32_t n, const int32_t* n_dev, void* stream);

/* As oomb_copy_pages, on the copy engines (SDMA) instead of compute units, for lists the
 * host knows that consist of long runs of consecutive pages (a whole layer's pages, a
 * chunk's new pages): src_ids / dst_ids are HOST int32 arrays, read during the call;
 * each run of consecutive pages on both sides becomes one transfer, enqueued on
 * `stream`. page_bytes > 0. Every transfer has a fixed cost of several microseconds,
 * so a list that breaks into more than max(16, n / 16) runs is refused with
 * OOMB_ERR_INVALID before any HIP call: scattered pages go through oomb_copy_pages or
 * oomb_fetch_selected, whose kernels gather them at the link's speed. While attention
 * kernels run on other streams, copy-engine transfers leave them at full speed; copies
 * by kernels share the compute units' memory path and slow them by ~10%, in exchange
 * for device-side lists. */
int oomb_copy_pages_sdma(const void* src, void* dst, int64_t page_bytes, int64_t n_src_pages,
                         int64_t n_dst_pages, const int32_t* src_ids, const int32_t* dst_ids,
                         int32_t n, void* stream);

/* fp32 pages of page_elems floats (a multiple of 4): dst page dst_ids[i] += src page
 * src_ids[i] (one fp32 rounding per element), then, if zero_src, src page src_ids[i]
 * = 0; for i < n (or min(n, *n_dev)). For moving key/value gradient pages into an fp32
 * pool elsewhere (explainer 2.B/2.C: gradients accumulate in paged storage and are
 * offloaded too). The dst ids of one call must be distinct. */
int oomb_add_pages_f32(const float* src, float* dst, int64_t page_elems, int64_t n_src_pages,
                       int64_t n_dst_pages, const int32_t* src_ids, const int32_t* dst_ids,
                       int32_t n, const int32_t* n_dev, int32_t zero_src, void* stream);

/* Fetch of the selected pages (sparse layers, explainer 2.C/2.D): for every KV head g
 * and j < count[g] (j < sel_stride), with lp = sel[g*sel_stride + j] (skipped unless
 * 0 <= lp < n_logical) and s = stage[g*stage_stride + j]: device page s of the pool's
 * K and V = host page host_table[g*host_table_stride + lp] of host_k / host_v (each
 * [host_pages][P][D] in the pool dtype), and table[g*table_stride + lp] = s. After it,
 * the attention calls read the selected pages from the staging pages through `table`.
 * The selection and counts come straight from oomb_select_pages. */
int oomb_fetch_selected(const oomb_pool* pool, int32_t* table, int64_t table_stride,
                        const void* host_k, const void* host_v, int64_t host_pages,
                        const int32_t* host_table, int64_t host_table_stride, const int32_t* sel,
                        int64_t sel_stride, const int32_t* count, const int32_t* stage,
                        int64_t stage_stride, int64_t n_logical, void* stream);

/* Kernel timing for profiling tools; not needed for normal use. While enabled on
 * the calling thread, each kernel that a call above launches is bracketed by two
 * HIP events on that call's stream (a small cost per launch). oomb_profile_collect
 * waits for the recorded events, writes up to `max` (kernel name, milliseconds)
 * pairs in launch order, releases the events and returns how many it wrote. Names
 * are static strings owned by the library. */
int oomb_profile_enable(int on);
int oomb_profile_collect(const char** names, float* ms, int max);

#ifdef __cplusplus
}
#endif

#endif /* OOMB_H */
