"""Plain, slow CPU oracle for OOMB-style paged chunk attention.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg may use this module; the HIP library never does. It shares no code
with the HIP path: it builds its own page pool by scatter, gathers pages back into
contiguous key/value arrays, and evaluates every quantity from its definition.

Sources (the OOMB pages; "explainer" = the gist.science explainer of arXiv 2602.02108):
  * chunk-recurrent training with recomputation: explainer, 2.A "Chunk-Recurrent
    Training with Activation Recomputation"; mlsanity page, "Abstract (arXiv)".
  * paged KV cache and paged KV gradients, in-place accumulation: explainer, 2.B
    "Paged KV Cache and Gradient Management"; mlsanity abstract.
  * top-K page retrieval scored through an averaged stand-in vector: explainer, 2.D "Page-Level
    Sparse Attention".
  * CPU offload of pages and gradient pages: explainer, 2.C "Asynchronous KV Cache CPU
    Offloading" (moving pages is a copy; moving gradient pages adds them in).
  * local attention for the sparse layers of sparse-native models: explainer, 2.D
    ("Native Support"). The pages do not define it further; it is read here as the
    usual sliding window: a query at position p sees the keys at p - W < t <= p.
The pages give no formula. Attention itself is the textbook definition (softmax of
scaled dot products, causal), so the forward/backward below is that definition
written out in fp64. Page selection is a heuristic the pages leave open; it is
specified here step by step (Quest-style min/max page summaries, a fixed fp32
summation order) and implemented in float32 exactly as specified.

Precision: attention in float64 from inputs widened exactly (bf16 and fp32 are
subsets of fp64); selection arithmetic in IEEE float32, round-to-nearest, no fused
multiply-add, in the order documented on each function.

Pins (tests marked "not gpu"): finite differences; equality of the chunk sweep with
full-sequence causal attention from torch's SDPA; an explicitly masked SDPA call for
sparse selections and for windows; window 1 (each query sees only itself) and a
window covering the whole context (equal to none); closed forms (single visible key,
all-zero keys, row sums of P,
column sums of dK and dV); page-permutation invariance; hand-derived values for the
summation orders (tests/golden/); brute-force order statistics for the top-k.
No function here is parity-unpinned.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence

import numpy as np
import torch

__all__ = [
    "append", "gather", "summarize", "total_order_key",
    "query_summary", "page_scores", "top_k_pages", "select_pages",
    "attended_pages", "key_positions", "fwd", "bwd", "sweep",
    "copy_pages", "add_pages", "fetch_selected",
    "summarize_mean", "page_scores_mean", "select_pages_mean", "rope", "layer_reference",
    "query_tiles", "select_pages_tiled", "tile_selection_row", "fwd_tiled", "bwd_tiled",
]


# ---------------------------------------------------------------------------
# Paging (explainer 2.B: K/V and their gradients live in fixed-size pages).
# A pool is [N, P, D]; a table row maps logical page j of one KV head to a
# physical page id. Token t of head g lives at pool[table[g, t // P], t % P].
# ---------------------------------------------------------------------------

def append(pool: torch.Tensor, table: torch.Tensor, new: torch.Tensor, start: int) -> None:
    """Scatter tokens [start, start+n) of every KV head into their pages (a copy)."""
    P = pool.shape[1]
    hkv, n, _ = new.shape
    t = torch.arange(start, start + n)
    for g in range(hkv):
        phys = table[g].long()[t // P]
        pool[phys, t % P] = new[g]


def gather(pool: torch.Tensor, table: torch.Tensor, g: int, pages: Sequence[int]) -> torch.Tensor:
    """Contiguous [len(pages) * P, D] copy of the listed logical pages of head g."""
    idx = table[g].long()[torch.as_tensor(list(pages), dtype=torch.long)]
    return pool[idx].reshape(-1, pool.shape[2])


def total_order_key(x: torch.Tensor) -> torch.Tensor:
    """Integer key that orders finite floats by value and puts -0 below +0."""
    if x.dtype == torch.bfloat16:
        b = x.view(torch.int16).to(torch.int32)
        mag = b & 0x7FFF
    elif x.dtype == torch.float32:
        b = x.view(torch.int32).to(torch.int64)
        mag = b & 0x7FFFFFFF
    else:
        raise TypeError(x.dtype)
    return torch.where(b >= 0, b, -mag - 1)


def summarize(k_pool, table, summary, first_page: int, n_pages: int, seq_len: int) -> None:
    """Per-page key summary (the representative of a page for retrieval, explainer 2.D;
    min/max form as in Quest, which the mlsanity page lists among OOMB's sources).

    summary[phys, 0, d] = min over the page's tokens with position < seq_len of K[., d]
    summary[phys, 1, d] = max over the same tokens.
    min/max use the total order of the values in which -0 < +0 (so the result never
    depends on evaluation order). Pages without a valid token are left unchanged."""
    P = k_pool.shape[1]
    for g in range(table.shape[0]):
        pages = torch.arange(first_page, first_page + n_pages)
        n_valid = torch.clamp(seq_len - pages * P, max=P)
        # pages whose every token is valid, a batch at a time
        full = pages[n_valid == P]
        for b0 in range(0, len(full), 2048):
            phys = table[g].long()[full[b0:b0 + 2048]]
            x = k_pool[phys]                                   # [n, P, D]
            key = total_order_key(x)
            summary[phys, 0] = torch.gather(x, 1, key.argmin(dim=1, keepdim=True))[:, 0]
            summary[phys, 1] = torch.gather(x, 1, key.argmax(dim=1, keepdim=True))[:, 0]
        # partially filled pages, one at a time
        for j, nv in zip(pages.tolist(), n_valid.tolist()):
            if nv <= 0 or nv == P:
                continue
            phys = int(table[g, j])
            x = k_pool[phys, :nv]
            key = total_order_key(x)
            summary[phys, 0] = torch.gather(x, 0, key.argmin(dim=0, keepdim=True))[0]
            summary[phys, 1] = torch.gather(x, 0, key.argmax(dim=0, keepdim=True))[0]


# ---------------------------------------------------------------------------
# Page selection (explainer 2.D "Top-K Page Retrieval": keep the K most relevant key
# pages, scored through an averaged stand-in vector). Float32, fixed order.
# ---------------------------------------------------------------------------

BLOCK = 64  # queries summed sequentially before the pairwise stage


def _as_f32(x: torch.Tensor) -> np.ndarray:
    return x.detach().to("cpu", torch.float32).numpy()


def query_summary(q: torch.Tensor, g: int, group: int) -> np.ndarray:
    """qbar for KV head g: the mean of the chunk's queries over its `group` heads.

    q is [Hq, C, D]. Let x_m = q[g*group + m // C, m % C, :] for m in [0, group*C)
    (head-major, then query order). Within each block of 64 consecutive m, sum
    sequentially in float32 starting from +0. Pad the block sums with +0 to a power
    of two and combine them by stride-halving pairs: for s = n/2, n/4, .., 1:
    a[i] = a[i] + a[i + s] for i < s. Multiply a[0] by fp32(1 / (group*C)), where
    the reciprocal is taken in float64 and rounded once."""
    C = q.shape[1]
    x = _as_f32(q[g * group:(g + 1) * group]).reshape(group * C, -1)
    M, D = x.shape
    nb = -(-M // BLOCK)
    padded = np.zeros((nb * BLOCK, D), np.float32)
    padded[:M] = x
    blocks = padded.reshape(nb, BLOCK, D)
    acc = np.zeros((nb, D), np.float32)
    for j in range(BLOCK):           # sequential within every block (all blocks at once)
        acc = acc + blocks[:, j]
    n2 = 1
    while n2 < nb:
        n2 *= 2
    a = np.zeros((n2, D), np.float32)
    a[:nb] = acc
    s = n2 // 2
    while s >= 1:
        a[:s] = a[:s] + a[s:2 * s]
        s //= 2
    inv = np.float32(1.0 / (group * C))
    return (a[0] * inv).astype(np.float32)


def page_scores(qbar: np.ndarray, summary: torch.Tensor, table: torch.Tensor, g: int,
                n_cand: int) -> np.ndarray:
    """score_j = sum_d max(qbar_d * kmax_jd, qbar_d * kmin_jd) for logical pages j < n_cand.

    Products are rounded to float32; max keeps qbar*kmax only when it is strictly
    greater. The sum over d is a stride-halving tree: for s = D/2, .., 1:
    a[d] = a[d] + a[d + s] for d < s."""
    if n_cand == 0:
        return np.zeros(0, np.float32)
    phys = table[g, :n_cand].long()
    smry = _as_f32(summary[phys])            # [n, 2, D]
    kmin, kmax = smry[:, 0], smry[:, 1]
    qb = qbar.astype(np.float32)[None, :]
    p_hi = qb * kmax
    p_lo = qb * kmin
    a = np.where(p_hi > p_lo, p_hi, p_lo).astype(np.float32)
    s = a.shape[1] // 2
    with np.errstate(invalid="ignore"):      # inf + -inf is NaN by IEEE rules: intended
        while s >= 1:
            a[:, :s] = a[:, :s] + a[:, s:2 * s]
            s //= 2
    return a[:, 0].copy()


def summarize_mean(k_pool, table, kmean: np.ndarray, first_page: int, n_pages: int,
                   seq_len: int) -> None:
    """Mean-key summary (the other plain reading of the page representative, explainer
    2.D: an average of the page's keys) of logical pages [first_page, first_page +
    n_pages) of every KV head, into kmean[phys] (float32 [N, D]): the keys widened to
    float32 and summed from +0 in token order, one float32 rounding per addition, then
    multiplied by float32(1 / n_valid) (the reciprocal taken in float64). Pages with no
    token below seq_len are left unchanged."""
    P = k_pool.shape[1]
    for g in range(table.shape[0]):
        for lp in range(first_page, first_page + n_pages):
            n_valid = min(P, seq_len - lp * P)
            if n_valid <= 0:
                continue
            ph = int(table[g, lp])
            rows = _as_f32(k_pool[ph, :n_valid])          # [n_valid, D] float32
            s = np.zeros(rows.shape[1], np.float32)
            for t in range(n_valid):
                s = (s + rows[t]).astype(np.float32)
            kmean[ph] = (s * np.float32(1.0 / n_valid)).astype(np.float32)


def page_scores_mean(qbar: np.ndarray, kmean: np.ndarray, table: torch.Tensor, g: int,
                     n_cand: int) -> np.ndarray:
    """score_j = sum_d float32(qbar_d * kmean_jd) for logical pages j < n_cand, summed
    by the same stride-halving tree over d as page_scores."""
    if n_cand == 0:
        return np.zeros(0, np.float32)
    phys = table[g, :n_cand].long().numpy()
    a = (qbar.astype(np.float32)[None, :] * kmean[phys].astype(np.float32)).astype(np.float32)
    s = a.shape[1] // 2
    while s >= 1:
        a[:, :s] = a[:, :s] + a[:, s:2 * s]
        s //= 2
    return a[:, 0].copy()


def top_k_pages(scores: np.ndarray, k: int) -> List[int]:
    """The k best pages by (score descending, logical id ascending), in ascending id
    order. Scores compare as IEEE values (-0 equals +0). A NaN score (keys holding
    infinities of both signs, say) ranks below every number, -inf included; NaN pages
    tie with each other, so among them the lower ids come first. k >= n keeps every
    page."""
    n = len(scores)

    def rank(j):
        x = float(scores[j])
        return (1, 0.0, j) if math.isnan(x) else (0, -x, j)

    order = sorted(range(n), key=rank)
    return sorted(order[:max(0, min(k, n))])


def select_pages(q, summary, table, t0: int, page: int, group: int, top_k: int):
    """Per KV head: (qbar, scores, selected logical ids). Candidates are the complete
    pages strictly before the chunk, [0, t0 // page); the chunk's own pages (and a
    page straddling t0) are attended anyway and never compete."""
    n_cand = t0 // page
    out = []
    for g in range(table.shape[0]):
        qb = query_summary(q, g, group)
        sc = page_scores(qb, summary, table, g, n_cand)
        out.append((qb, sc, top_k_pages(sc, top_k)))
    return out


def select_pages_mean(q, kmean: np.ndarray, table, t0: int, page: int, group: int, top_k: int):
    """As select_pages, with the scores of page_scores_mean."""
    n_cand = t0 // page
    out = []
    for g in range(table.shape[0]):
        qb = query_summary(q, g, group)
        sc = page_scores_mean(qb, kmean, table, g, n_cand)
        out.append((qb, sc, top_k_pages(sc, top_k)))
    return out


# ---------------------------------------------------------------------------
# Finer selection granularity (explainer 2.D leaves the unit of selection open): the
# chunk's queries are cut into tiles of `tile` consecutive queries (the last tile may
# be shorter), and every (KV head, tile) pair selects its own top-k prior pages by the
# same rule, from the mean of that tile's queries over the head group. The candidates
# are still the complete pages before the chunk, and the chunk's own pages are still
# attended by every query.
# ---------------------------------------------------------------------------

def query_tiles(n_q: int, tile: int) -> List[range]:
    """Query index ranges of the tiles of a chunk of n_q queries."""
    if tile <= 0:
        raise ValueError("tile must be positive")
    return [range(i0, min(n_q, i0 + tile)) for i0 in range(0, n_q, tile)]


def select_pages_tiled(q, summary, table, t0: int, page: int, group: int, top_k: int,
                       tile: int):
    """out[g][j] = (qbar, scores, selected logical ids) of KV head g and query tile j:
    select_pages' steps with qbar taken over the tile's queries only (the same fixed
    order: blocks of 64 consecutive rows of the tile, head-major then query order, the
    stride-halving tree, one multiply by fp32(1 / (group * tile length)))."""
    n_cand = t0 // page
    out = []
    for g in range(table.shape[0]):
        row = []
        for r in query_tiles(q.shape[1], tile):
            qb = query_summary(q[:, r.start:r.stop], g, group)
            sc = page_scores(qb, summary, table, g, n_cand)
            row.append((qb, sc, top_k_pages(sc, top_k)))
        out.append(row)
    return out


def tile_selection_row(chosen: Sequence[int], t0: int, page: int, tile: int, j: int) -> List[int]:
    """The pages that query tile j attends besides its own local pages, as one ascending
    list: its chosen prior pages, then the chunk's pages that lie wholly before the
    tile's first query (logical [t0 // page, (t0 + j * tile) // page)). Attention of the
    tile is then the chunk attention of its queries, first position t0 + j * tile, with
    this list as the selection."""
    return sorted(int(c) for c in chosen) + list(range(t0 // page, (t0 + j * tile) // page))


def fwd_tiled(q, k_pool, v_pool, table, t0: int, chosen, scale: float, tile: int):
    """O, LSE of a chunk whose query tiles attend their own selections: chosen[g][j] are
    tile j's prior pages for KV head g; each tile is fwd over its queries at t0 + j*tile
    with tile_selection_row as its selection."""
    hq, C, D = q.shape
    P = k_pool.shape[1]
    O = torch.zeros(hq, C, D, dtype=torch.float64)
    L = torch.zeros(hq, C, dtype=torch.float64)
    for j, r in enumerate(query_tiles(C, tile)):
        sel = [tile_selection_row(chosen[g][j], t0, P, tile, j) for g in range(table.shape[0])]
        O[:, r.start:r.stop], L[:, r.start:r.stop] = fwd(q[:, r.start:r.stop], k_pool, v_pool,
                                                         table, t0 + r.start, sel, scale)
    return O, L


def bwd_tiled(q, k_pool, v_pool, table, t0: int, chosen, scale: float, tile: int, dout,
              dk_pool=None, dv_pool=None, gtable=None):
    """dQ of the tiled attention (tile by tile, as bwd), adding every tile's dK/dV into
    the gradient pools when given."""
    hq, C, D = q.shape
    P = k_pool.shape[1]
    dQ = torch.zeros(hq, C, D, dtype=torch.float64)
    for j, r in enumerate(query_tiles(C, tile)):
        sel = [tile_selection_row(chosen[g][j], t0, P, tile, j) for g in range(table.shape[0])]
        dQ[:, r.start:r.stop], _ = bwd(q[:, r.start:r.stop], k_pool, v_pool, table,
                                       t0 + r.start, sel, scale, dout[:, r.start:r.stop],
                                       dk_pool, dv_pool, gtable)
    return dQ


# ---------------------------------------------------------------------------
# Attention of one chunk over the paged cache (explainer 2.A-2.B, 2.D).
# Query i of the chunk sits at absolute position t0 + i and sees key t iff
# page(t) is selected or local and t <= t0 + i; with a window W (local attention,
# dense calls only) also t > t0 + i - W.
# ---------------------------------------------------------------------------

def attended_pages(t0: int, n_q: int, page: int, sel: Optional[Sequence[int]]) -> List[int]:
    """Selected prior pages (all of [0, t0//page) when sel is None), then local pages."""
    first_local = t0 // page
    last_local = (t0 + n_q - 1) // page
    prior = list(range(first_local)) if sel is None else sorted(int(j) for j in sel)
    return prior + list(range(first_local, last_local + 1))


def key_positions(pages: Sequence[int], page: int, end: int) -> torch.Tensor:
    """Absolute positions of the tokens of the listed pages that lie before `end`."""
    pos = (torch.as_tensor(list(pages), dtype=torch.long)[:, None] * page
           + torch.arange(page)[None, :]).reshape(-1)
    return pos[pos < end]


def _keys(k_pool, v_pool, table, g, pages, page, end):
    pos_all = (torch.as_tensor(list(pages), dtype=torch.long)[:, None] * page
               + torch.arange(page)[None, :]).reshape(-1)
    keep = pos_all < end
    K = gather(k_pool, table, g, pages)[keep].to(torch.float64)
    V = gather(v_pool, table, g, pages)[keep].to(torch.float64)
    return pos_all[keep], K, V


def _rows(n, rb):
    for i0 in range(0, n, rb):
        yield i0, min(n, i0 + rb)


def _probs(Qb, K, pos, qpos, scale, window=0):
    """P = softmax over visible keys of scale * Q K^T, and the natural-log LSE."""
    S = scale * torch.matmul(Qb, K.T)
    hidden = pos[None, :] > qpos[:, None]
    if window > 0:
        hidden = hidden | (pos[None, :] <= qpos[:, None] - window)
    S = S.masked_fill(hidden[None], -math.inf)
    m = S.amax(dim=-1, keepdim=True)
    E = torch.exp(S - m)
    Z = E.sum(dim=-1, keepdim=True)
    return E / Z, (m + torch.log(Z))[..., 0]


def _check_window(sel, window):
    if window < 0 or (window > 0 and sel is not None):
        raise ValueError("window must be >= 0, and a window (local attention) takes no selection")


def fwd(q, k_pool, v_pool, table, t0: int, sel, scale: float, row_block: int = 256,
        window: int = 0):
    """O [Hq, C, D] and LSE [Hq, C] in float64.

    sel: None for dense, else one list of selected logical pages per KV head.
    window > 0: local attention (sel None), only keys t > p - window are visible.
    For q head h (KV head g = h // G) and query i at p = t0 + i, over the visible
    keys t: s_t = scale * q.k_t, LSE = log sum_t exp(s_t), P_t = exp(s_t - LSE),
    O = sum_t P_t v_t."""
    _check_window(sel, window)
    hq, C, D = q.shape
    hkv = table.shape[0]
    G = hq // hkv
    P = k_pool.shape[1]
    O = torch.zeros(hq, C, D, dtype=torch.float64)
    L = torch.zeros(hq, C, dtype=torch.float64)
    qpos_all = t0 + torch.arange(C)
    for g in range(hkv):
        pages = attended_pages(t0, C, P, None if sel is None else sel[g])
        pos, K, V = _keys(k_pool, v_pool, table, g, pages, P, t0 + C)
        Qg = q[g * G:(g + 1) * G].to(torch.float64)
        for i0, i1 in _rows(C, row_block):
            Pm, lse = _probs(Qg[:, i0:i1], K, pos, qpos_all[i0:i1], scale, window)
            O[g * G:(g + 1) * G, i0:i1] = torch.matmul(Pm, V)
            L[g * G:(g + 1) * G, i0:i1] = lse
    return O, L


def bwd(q, k_pool, v_pool, table, t0: int, sel, scale: float, dout,
        dk_pool=None, dv_pool=None, gtable=None, row_block: int = 256, window: int = 0,
        with_fwd: bool = False):
    """Analytic backward of fwd for the loss sum(dout * O), with O and LSE recomputed
    here (explainer 2.A: activations are recomputed just before the gradient).

    Returns dQ [Hq, C, D] float64. With dk_pool/dv_pool (float64 [Ng, P, D]) and
    gtable, adds dK/dV of every attended key into its gradient page (explainer 2.B:
    gradients accumulate in place in paged storage). Also returns the per-head
    key-gradient arrays as a list of (positions, dK, dV). with_fwd=True appends the
    recomputed O and LSE (the same values fwd returns) to the result.
        Delta_i = dO_i . O_i
        dP_it   = dO_i . v_t
        dS_it   = P_it (dP_it - Delta_i)
        dQ_i    = scale * sum_t dS_it k_t
        dK_t    = scale * sum_{h in group, i} dS_it q_i
        dV_t    = sum_{h in group, i} P_it dO_i
    """
    _check_window(sel, window)
    hq, C, D = q.shape
    hkv = table.shape[0]
    G = hq // hkv
    P = k_pool.shape[1]
    dQ = torch.zeros(hq, C, D, dtype=torch.float64)
    O = torch.zeros(hq, C, D, dtype=torch.float64) if with_fwd else None
    L = torch.zeros(hq, C, dtype=torch.float64) if with_fwd else None
    per_head = []
    qpos_all = t0 + torch.arange(C)
    for g in range(hkv):
        pages = attended_pages(t0, C, P, None if sel is None else sel[g])
        pos, K, V = _keys(k_pool, v_pool, table, g, pages, P, t0 + C)
        Qg = q[g * G:(g + 1) * G].to(torch.float64)
        dOg = dout[g * G:(g + 1) * G].to(torch.float64)
        dK = torch.zeros_like(K)
        dV = torch.zeros_like(V)
        for i0, i1 in _rows(C, row_block):
            Qb, dOb = Qg[:, i0:i1], dOg[:, i0:i1]
            Pm, lse = _probs(Qb, K, pos, qpos_all[i0:i1], scale, window)
            Ob = torch.matmul(Pm, V)
            if with_fwd:
                O[g * G:(g + 1) * G, i0:i1] = Ob
                L[g * G:(g + 1) * G, i0:i1] = lse
            delta = (dOb * Ob).sum(dim=-1, keepdim=True)
            dP = torch.matmul(dOb, V.T)
            dS = Pm * (dP - delta)
            dQ[g * G:(g + 1) * G, i0:i1] = scale * torch.matmul(dS, K)
            dK += scale * torch.einsum("hik,hid->kd", dS, Qb)
            dV += torch.einsum("hik,hid->kd", Pm, dOb)
        per_head.append((pos, dK, dV))
        if dk_pool is not None:
            phys = gtable[g].long()[pos // P]
            dk_pool.index_put_((phys, pos % P), dK, accumulate=True)
            dv_pool.index_put_((phys, pos % P), dV, accumulate=True)
    if with_fwd:
        return dQ, per_head, O, L
    return dQ, per_head


def sweep(q_all, k_all, v_all, do_all, table, gtable, n_pool: int, page: int, chunk: int,
          scale: float, top_k: Optional[int] = None, window: int = 0):
    """Chunk-recurrent pass over a whole sequence (explainer 2.A).

    Forward, chunk c = 0..S-1: append chunk c's K/V into the pool, summarize its
    pages, select pages (when top_k is set), attend. Reverse, c = S-1..0: recompute
    chunk c's attention with the selection made in the forward pass, then its
    backward; dQ is per chunk and dK/dV accumulate across chunks in the paged
    float64 gradient pools. Returns O, LSE, dQ over the whole sequence, the gradient
    pools and the selections."""
    hq, T, D = q_all.shape
    hkv = k_all.shape[0]
    G = hq // hkv
    S = T // chunk
    k_pool = torch.zeros(n_pool, page, D, dtype=k_all.dtype)
    v_pool = torch.zeros(n_pool, page, D, dtype=v_all.dtype)
    summary = torch.zeros(n_pool, 2, D, dtype=k_all.dtype)
    dk_pool = torch.zeros(n_pool, page, D, dtype=torch.float64)
    dv_pool = torch.zeros(n_pool, page, D, dtype=torch.float64)
    O = torch.zeros(hq, T, D, dtype=torch.float64)
    L = torch.zeros(hq, T, dtype=torch.float64)
    dQ = torch.zeros(hq, T, D, dtype=torch.float64)
    sels = []
    for c in range(S):
        t0 = c * chunk
        sl = slice(t0, t0 + chunk)
        append(k_pool, table, k_all[:, sl], t0)
        append(v_pool, table, v_all[:, sl], t0)
        first = t0 // page
        summarize(k_pool, table, summary, first, (t0 + chunk - 1) // page - first + 1, t0 + chunk)
        sel = None
        if top_k is not None:
            sel = [s for (_, _, s) in select_pages(q_all[:, sl], summary, table, t0, page, G, top_k)]
        sels.append(sel)
        O[:, sl], L[:, sl] = fwd(q_all[:, sl], k_pool, v_pool, table, t0, sel, scale,
                                 window=window)
    for c in reversed(range(S)):
        t0 = c * chunk
        sl = slice(t0, t0 + chunk)
        dQ[:, sl], _ = bwd(q_all[:, sl], k_pool, v_pool, table, t0, sels[c], scale,
                           do_all[:, sl], dk_pool, dv_pool, gtable, window=window)
    return {"O": O, "LSE": L, "dQ": dQ, "dk_pool": dk_pool, "dv_pool": dv_pool,
            "sels": sels, "k_pool": k_pool, "v_pool": v_pool, "summary": summary}


# ---------------------------------------------------------------------------
# Page movement (explainer 2.C: the KV cache and its gradients move between GPU
# and CPU memory). A page array is [N, ...]; page ids outside it are skipped.
# ---------------------------------------------------------------------------

def _valid(i: int, n: int) -> bool:
    return 0 <= i < n


def copy_pages(src: torch.Tensor, dst: torch.Tensor, src_ids, dst_ids, n: Optional[int] = None) -> None:
    """dst[dst_ids[i]] = src[src_ids[i]] for i < n, in list order."""
    n = len(src_ids) if n is None else n
    for i in range(n):
        s, d = int(src_ids[i]), int(dst_ids[i])
        if _valid(s, src.shape[0]) and _valid(d, dst.shape[0]):
            dst[d] = src[s]


def add_pages(src: torch.Tensor, dst: torch.Tensor, src_ids, dst_ids, n: Optional[int] = None,
              zero_src: bool = False) -> None:
    """fp32 pages: dst[dst_ids[i]] = fp32(dst + src) element by element (one rounding),
    then src[src_ids[i]] = 0 when zero_src; for i < n."""
    n = len(src_ids) if n is None else n
    for i in range(n):
        s, d = int(src_ids[i]), int(dst_ids[i])
        if _valid(s, src.shape[0]) and _valid(d, dst.shape[0]):
            total = src[s].to(torch.float64) + dst[d].to(torch.float64)
            dst[d] = total.to(torch.float32)  # the exact sum, rounded once
            if zero_src:
                src[s] = 0.0


def fetch_selected(k_pool, v_pool, table, host_k, host_v, host_table, sel, count, stage,
                   n_logical: int) -> None:
    """For KV head g and j < count[g]: lp = sel[g][j] (skipped unless 0 <= lp < n_logical),
    s = stage[g][j]: device page s of K and V = host page host_table[g][lp], and
    table[g][lp] = s (in head order, then j)."""
    for g in range(table.shape[0]):
        for j in range(min(int(count[g]), sel.shape[1])):
            lp = int(sel[g, j])
            if not _valid(lp, n_logical):
                continue
            hp, s = int(host_table[g, lp]), int(stage[g, j])
            if not (_valid(hp, host_k.shape[0]) and _valid(s, k_pool.shape[0])):
                continue
            k_pool[s] = host_k[hp]
            v_pool[s] = host_v[hp]
            table[g, lp] = s


# ---------------------------------------------------------------------------
# Rotary position embedding of the chunk-recurrent layer (positions are global: a
# chunk's tokens keep their absolute positions, explainer 2.A).
# ---------------------------------------------------------------------------

def rope(x: torch.Tensor, pos0: int, theta: float = 10000.0, inverse: bool = False) -> torch.Tensor:
    """float64 rotation of x [heads, tokens, D] by a = (pos0 + i) * theta^(-2d/D) on the
    pairs (d, d + D/2): y_d = x_d cos a - x_{d+D/2} sin a, y_{d+D/2} = x_{d+D/2} cos a
    + x_d sin a; inverse rotates by -a."""
    H, n, D = x.shape
    half = D // 2
    d = torch.arange(half, dtype=torch.float64)
    inv_freq = torch.tensor(float(theta), dtype=torch.float64) ** (-2.0 * d / D)
    ang = (pos0 + torch.arange(n, dtype=torch.float64))[:, None] * inv_freq[None, :]
    c, s = torch.cos(ang), torch.sin(ang)
    if inverse:
        s = -s
    xd = x.to(torch.float64)
    lo, hi = xd[..., :half], xd[..., half:]
    return torch.cat([lo * c - hi * s, hi * c + lo * s], dim=-1)



# ---------------------------------------------------------------------------
# One chunk-recurrent attention layer as a single full-sequence computation
# (explainer 2.A: chunking with recomputation must give the gradients of the whole
# sequence; 2.D: top-k layers attend the pages each chunk selected, local layers a
# window).
# ---------------------------------------------------------------------------

def layer_reference(x, wq, wk, wv, wo, n_q_heads: int, n_kv_heads: int, head_dim: int,
                    page: int, chunk: int, scale: float, theta: float, dy,
                    top_k: Optional[int] = None, window: int = 0,
                    sel_dtype: torch.dtype = torch.bfloat16):
    """y = o Wo with o = attention(q, k, v), q = rope(x Wq), k = rope(x Wk), v = x Wv
    (positions 0..T-1), over the whole sequence at once in float64, and the gradients
    of sum(dy * y) with respect to x, Wq, Wk, Wv, Wo by autograd.

    Query i attends key t iff t <= i, and with a window also t > i - window; for a
    top-k layer also iff page(t) is one of the pages the chunk holding i selected, or
    one of that chunk's own pages. The selection of chunk c is select_pages applied to
    the chunk's queries and the keys before it, each rounded once to sel_dtype (the
    dtype the layer keeps its activations in), with the summaries of complete pages.

    Returns (y, dx, [dWq, dWk, dWv, dWo], sels) with sels[c] = one list of selected
    logical pages per KV head (None for layers without selection)."""
    f64 = torch.float64
    xs = x.detach().to("cpu", f64).requires_grad_()
    ws = [w.detach().to("cpu", f64).requires_grad_() for w in (wq, wk, wv, wo)]
    T = xs.shape[0]
    hq, hkv, D = n_q_heads, n_kv_heads, head_dim
    G = hq // hkv
    q = rope((xs @ ws[0]).view(T, hq, D).transpose(0, 1), 0, theta)
    k = rope((xs @ ws[1]).view(T, hkv, D).transpose(0, 1), 0, theta)
    v = (xs @ ws[2]).view(T, hkv, D).transpose(0, 1)
    pos = torch.arange(T)
    allowed = pos[None, :] <= pos[:, None]
    if window:
        allowed = allowed & (pos[None, :] > pos[:, None] - window)
    allowed = allowed[None].expand(hq, T, T).clone()
    sels = [None] * (T // chunk)
    if top_k is not None:
        n_pages = -(-T // page)
        ident = torch.arange(hkv * n_pages, dtype=torch.int32).reshape(hkv, n_pages)
        kr = k.detach().to(sel_dtype)
        kpool = torch.zeros(hkv * n_pages, page, D, dtype=sel_dtype)
        append(kpool, ident, kr, 0)
        summ = torch.zeros(hkv * n_pages, 2, D, dtype=sel_dtype)
        summarize(kpool, ident, summ, 0, n_pages, T)
        page_of = pos // page
        for c in range(T // chunk):
            t0 = c * chunk
            qc = q.detach()[:, t0:t0 + chunk].to(sel_dtype)
            chosen = [s_ for (_, _, s_) in select_pages(qc, summ, ident, t0, page, G, top_k)]
            sels[c] = chosen
            for h in range(hq):
                ok = torch.zeros(n_pages, dtype=torch.bool)
                ok[torch.as_tensor(chosen[h // G], dtype=torch.long)] = True
                ok[t0 // page:] = True
                allowed[h, t0:t0 + chunk] &= ok[page_of][None, :]
    kk = k.repeat_interleave(G, dim=0)
    vv = v.repeat_interleave(G, dim=0)
    S = (q @ kk.transpose(1, 2)) * scale
    S = S.masked_fill(~allowed, -math.inf)
    o = torch.softmax(S, dim=-1) @ vv
    y = o.transpose(0, 1).reshape(T, hq * D) @ ws[3]
    (y * dy.detach().to("cpu", f64)).sum().backward()
    return y.detach(), xs.grad, [w.grad for w in ws], (sels if top_k is not None else None)
