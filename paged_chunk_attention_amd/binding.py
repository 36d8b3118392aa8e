"""Thin Python binding of the C ABI (include/oomb.h), over torch device tensors.

Each function has the C name, checks tensor devices/dtypes/shapes, allocates
outputs and workspace with torch when the caller passes none, and calls the
library on the given stream (torch's current stream by default). What a function
allocates or fills is allocated and filled on that same stream, so the fills are
ordered before the library's kernels and the caching allocator reuses the memory
only for later work on that stream. No step of the computation happens here.

Setting OOMB_CHECK_TABLES=1 makes every call check, on the host, that the page
tables it reads are injective over the pages the call touches and that selections
are strictly ascending candidate ids (check_page_tables, check_selection). The
check copies the tables to the host and synchronises, so it is for debugging.

`PagedPool` owns one layer's page pool (K, V, key summaries, fp32 dK/dV) as torch
tensors and describes it to the library. The page tables are plain int32 tensors
[num_kv_heads, pages_per_head] mapping logical pages to physical ones; the
gradient table may be the same tensor or a separate one. The cache and its
gradients are not tracked by autograd: callers invoke forward and backward
explicitly (gist.science explainer of OOMB, 2.B: the KV cache is decoupled from
the autograd graph).
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

from ._lib import OOMB_DTYPE_BF16, OOMB_DTYPE_FP32, OombPool, call, lib

_DTYPES = {torch.bfloat16: OOMB_DTYPE_BF16, torch.float32: OOMB_DTYPE_FP32}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on(stream):
    """Context in which the binding allocates and fills: the call's stream when one is
    given (torch.cuda.stream makes it current), else torch's current stream as is."""
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _new(kind: str, shape, dtype, device, fill=None) -> torch.Tensor:
    """Every tensor the binding creates for a call comes from here (inside _on)."""
    if kind == "full":
        return torch.full(shape, fill, dtype=dtype, device=device)
    if kind == "zeros":
        return torch.zeros(shape, dtype=dtype, device=device)
    return torch.empty(shape, dtype=dtype, device=device)


def _checks_on() -> bool:
    return os.environ.get("OOMB_CHECK_TABLES", "0") not in ("", "0")


def check_page_tables(table: torch.Tensor, pages, n_pages: int, name: str = "table") -> None:
    """Raise ValueError unless the logical pages a call touches map to distinct physical
    pages in [0, n_pages).

    table: int32 [Hkv, stride]; pages: the number of leading logical pages in use per KV
    head, or one list of logical ids per KV head. All the (head, page) entries together
    must be distinct, since the KV heads share one page array. Two logical pages on one
    physical page would make the forward count those keys twice and two backward
    workgroups add into one gradient row at once."""
    t = table.detach().to("cpu", torch.int64)
    if isinstance(pages, int):
        if pages > t.shape[1]:
            raise ValueError(f"{name}: {pages} pages in use but only {t.shape[1]} columns")
        ids = t[:, :pages].reshape(-1)
    else:
        rows = []
        for g, lp in enumerate(pages):
            lp = torch.as_tensor(list(lp), dtype=torch.int64)
            if lp.numel() and (int(lp.min()) < 0 or int(lp.max()) >= t.shape[1]):
                raise ValueError(f"{name}: logical page outside the table of KV head {g}")
            rows.append(t[g, lp])
        ids = torch.cat(rows) if rows else torch.zeros(0, dtype=torch.int64)
    bad = (ids < 0) | (ids >= n_pages)
    if bool(bad.any()):
        raise ValueError(f"{name}: physical id {int(ids[bad][0])} outside [0, {n_pages})")
    uniq, counts = torch.unique(ids, return_counts=True)
    if bool((counts > 1).any()):
        raise ValueError(f"{name}: physical page {int(uniq[counts > 1][0])} is mapped "
                         f"{int(counts.max())} times")


def check_selection(sel: torch.Tensor, count: torch.Tensor, n_cand: int) -> None:
    """Raise ValueError unless, for every KV head g, sel[g, :count[g]] (count clamped to
    the row length and to n_cand, as the kernels clamp it) are strictly ascending
    candidate ids in [0, n_cand)."""
    s = sel.detach().to("cpu", torch.int64)
    c = count.detach().to("cpu", torch.int64)
    for g in range(s.shape[0]):
        row = s[g, :max(0, min(int(c[g]), s.shape[1], n_cand))]
        if row.numel() and (int(row.min()) < 0 or int(row.max()) >= n_cand):
            raise ValueError(f"selection of KV head {g}: id outside [0, {n_cand})")
        if row.numel() > 1 and not bool((row[1:] > row[:-1]).all()):
            raise ValueError(f"selection of KV head {g} is not strictly ascending")


def attended_logical_pages(hkv: int, P: int, t0: int, n_q: int, sel=None, count=None,
                           window: int = 0):
    """Per KV head, the logical pages an attention call reads: the selected (or, dense,
    all) prior pages, or with a window the prior pages it reaches, then the chunk's own."""
    first_local, last_local = t0 // P, (t0 + max(n_q, 1) - 1) // P
    local = list(range(first_local, last_local + 1))
    if sel is not None:
        s = sel.detach().to("cpu", torch.int64)
        c = count.detach().to("cpu", torch.int64)
        out = []
        for g in range(hkv):
            n = max(0, min(int(c[g]), s.shape[1], first_local))
            out.append(sorted(set(s[g, :n].tolist())) + local)
        return out
    lo = 0 if window <= 0 else max(0, t0 - window + 1) // P
    return [list(range(lo, first_local)) + local for _ in range(hkv)]


def _debug_check(pool, table, t0: int, n_q: int, sel=None, count=None, window: int = 0,
                 gtable=None) -> None:
    """The OOMB_CHECK_TABLES checks of one attention call (no-op when unset)."""
    if not _checks_on() or n_q == 0:
        return
    n_cand = t0 // pool.page_size
    if sel is not None:
        check_selection(sel, count, n_cand)
    pages = attended_logical_pages(pool.num_kv_heads, pool.page_size, t0, n_q, sel, count, window)
    check_page_tables(table, pages, pool.num_pages, "table")
    if gtable is not None:
        check_page_tables(gtable, pages, pool.dk.shape[0], "gtable")


class PagedPool:
    """K/V page pool of one layer, plus its key summaries and fp32 gradient pool."""

    def __init__(self, num_pages: int, page_size: int, head_dim: int, num_q_heads: int,
                 num_kv_heads: int, dtype: torch.dtype = torch.bfloat16, device="cuda",
                 num_grad_pages: Optional[int] = None, with_summary: bool = True,
                 with_grad: bool = True):
        if dtype not in _DTYPES:
            raise TypeError(f"unsupported dtype {dtype}")
        self.page_size, self.head_dim = page_size, head_dim
        self.num_q_heads, self.num_kv_heads = num_q_heads, num_kv_heads
        self.dtype, self.device = dtype, torch.device(device)
        self.k = torch.zeros(num_pages, page_size, head_dim, dtype=dtype, device=device)
        self.device = self.k.device  # concrete index, e.g. cuda:0
        self.v = torch.zeros_like(self.k)
        self.summary = (torch.zeros(num_pages, 2, head_dim, dtype=dtype, device=device)
                        if with_summary else None)
        ng = num_pages if num_grad_pages is None else num_grad_pages
        self.dk = torch.zeros(ng, page_size, head_dim, dtype=torch.float32, device=device) \
            if with_grad else None
        self.dv = torch.zeros_like(self.dk) if with_grad else None
        self.desc = OombPool(
            dtype=_DTYPES[dtype], page_size=page_size, head_dim=head_dim,
            num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, reserved=0,
            num_pages=num_pages, num_grad_pages=ng if with_grad else 0,
            k_pool=self.k.data_ptr(), v_pool=self.v.data_ptr(),
            k_summary=self.summary.data_ptr() if with_summary else None,
            dk_pool=self.dk.data_ptr() if with_grad else None,
            dv_pool=self.dv.data_ptr() if with_grad else None)

    @classmethod
    def from_tensors(cls, k: torch.Tensor, v: torch.Tensor, summary: Optional[torch.Tensor],
                     dk: Optional[torch.Tensor], dv: Optional[torch.Tensor], num_q_heads: int,
                     num_kv_heads: int, num_pages: Optional[int] = None) -> "PagedPool":
        """A pool over existing tensors (nothing is allocated): k, v [N, P, D] in one dtype,
        summary [>= num_pages, 2, D] or None, dk, dv fp32 [Ng, P, D] or None. num_pages
        (default N) is what the descriptor declares; a larger value suits calls that only
        read the summaries (the page selection), indexed by ids up to num_pages."""
        if k.dtype not in _DTYPES or v.dtype != k.dtype or v.shape != k.shape or k.dim() != 3:
            raise ValueError("k and v must be [pages, page_size, head_dim] tensors of one dtype")
        self = cls.__new__(cls)
        self.page_size, self.head_dim = k.shape[1], k.shape[2]
        self.num_q_heads, self.num_kv_heads = num_q_heads, num_kv_heads
        self.dtype, self.device = k.dtype, k.device
        self.k, self.v, self.summary, self.dk, self.dv = k, v, summary, dk, dv
        n = k.shape[0] if num_pages is None else num_pages
        if summary is not None and summary.shape[0] < n:
            raise ValueError("summary holds fewer pages than declared")
        ng = 0 if dk is None else dk.shape[0]
        self.desc = OombPool(
            dtype=_DTYPES[k.dtype], page_size=k.shape[1], head_dim=k.shape[2],
            num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, reserved=0,
            num_pages=n, num_grad_pages=ng, k_pool=k.data_ptr(), v_pool=v.data_ptr(),
            k_summary=None if summary is None else summary.data_ptr(),
            dk_pool=None if dk is None else dk.data_ptr(),
            dv_pool=None if dv is None else dv.data_ptr())
        return self

    @property
    def num_pages(self) -> int:
        return int(self.desc.num_pages)

    def zero_grad(self):
        if self.dk is not None:
            self.dk.zero_()
            self.dv.zero_()

    def ref(self):
        return ctypes.byref(self.desc)


def _check_table(t: torch.Tensor, pool: PagedPool, name: str):
    if t.dtype != torch.int32 or t.device != pool.device or t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be an int32 [num_kv_heads, pages] tensor on {pool.device}")
    if t.shape[0] != pool.num_kv_heads:
        raise ValueError(f"{name} has {t.shape[0]} rows, expected {pool.num_kv_heads}")


def _view(x: torch.Tensor, pool: PagedPool, heads: int, name: str, dtype=None):
    dtype = pool.dtype if dtype is None else dtype
    if x.dtype != dtype or x.device != pool.device or x.dim() != 3:
        raise ValueError(f"{name} must be a [heads, tokens, {pool.head_dim}] {dtype} tensor "
                         f"on {pool.device}")
    if x.shape[0] != heads or x.shape[2] != pool.head_dim or x.stride(2) != 1:
        raise ValueError(f"{name} has shape {tuple(x.shape)} / strides {x.stride()}")
    return x.stride(0), x.stride(1)


def oomb_kv_append(pool: PagedPool, table: torch.Tensor, k_new: torch.Tensor,
                   v_new: torch.Tensor, start_pos: int, stream=None) -> None:
    """Write tokens [start_pos, start_pos + n) of every KV head into their pages."""
    _check_table(table, pool, "table")
    hs, ts = _view(k_new, pool, pool.num_kv_heads, "k_new")
    if _view(v_new, pool, pool.num_kv_heads, "v_new") != (hs, ts) or v_new.shape != k_new.shape:
        raise ValueError("k_new and v_new must have the same shape and strides")
    n = k_new.shape[1]
    if _checks_on() and n > 0:
        P = pool.page_size
        written = list(range(start_pos // P, (start_pos + n - 1) // P + 1))
        check_page_tables(table, [written] * pool.num_kv_heads, pool.num_pages, "table")
    call("oomb_kv_append", pool.ref(), _ptr(table), table.stride(0), _ptr(k_new), _ptr(v_new),
         hs, ts, k_new.shape[1], start_pos, _stream(stream))


def oomb_page_summarize(pool: PagedPool, table: torch.Tensor, first_page: int, n_pages: int,
                        seq_len: int, stream=None) -> None:
    """Per-page key min/max for logical pages [first_page, first_page + n_pages)."""
    _check_table(table, pool, "table")
    call("oomb_page_summarize", pool.ref(), _ptr(table), table.stride(0), first_page, n_pages,
         seq_len, _stream(stream))


def split_plan(pool: PagedPool, n_q: int, t0: int, sel_stride: int = -1, window: int = 0) -> dict:
    """How the forward and backward calls of this geometry spread their work over the
    GPU (oomb_split_plan): per pass, the key ranges or query-stream parts and the tiles
    or key blocks per KV head that stay whole."""
    out = (ctypes.c_int32 * 6)()
    call("oomb_split_plan", pool.ref(), n_q, t0, sel_stride, window, out)
    return {"fwd": (out[0], out[1]), "dq": (out[2], out[3]), "dkdv": (out[4], out[5])}


def select_workspace_bytes(pool: PagedPool, n_q: int, t0: int) -> int:
    return int(lib().oomb_select_workspace_bytes(pool.ref(), n_q, t0))


def bwd_workspace_bytes(pool: PagedPool, n_q: int, t0: int, sel_stride: int = -1,
                        window: int = 0) -> int:
    """Workspace of oomb_paged_chunk_attn_bwd (sel_stride = -1 for dense calls)."""
    return int(lib().oomb_bwd_workspace_bytes(pool.ref(), n_q, t0, sel_stride, window))


def fwd_workspace_bytes(pool: PagedPool, n_q: int, t0: int, sel_stride: int = -1,
                        window: int = 0) -> int:
    """Workspace of oomb_paged_chunk_attn_fwd (sel_stride = -1 for dense calls)."""
    return int(lib().oomb_fwd_workspace_bytes(pool.ref(), n_q, t0, sel_stride, window))


def _workspace(nbytes: int, device, ws: Optional[torch.Tensor]):
    if ws is None:
        ws = _new("empty", max(nbytes, 256), torch.uint8, device)
    if ws.numel() < nbytes or ws.data_ptr() % 256:
        raise ValueError(f"workspace must hold {nbytes} bytes at a 256-byte aligned address")
    return ws


def oomb_select_pages(pool: PagedPool, table: torch.Tensor, q: torch.Tensor, t0: int, top_k: int,
                      sel: Optional[torch.Tensor] = None, count: Optional[torch.Tensor] = None,
                      qbar_out: Optional[torch.Tensor] = None,
                      score_out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None,
                      stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Top-k prior pages per KV head. Returns (sel int32 [Hkv, k], count int32 [Hkv])."""
    _check_table(table, pool, "table")
    hs, ts = _view(q, pool, pool.num_q_heads, "q")
    n_q = q.shape[1]
    n_cand = t0 // pool.page_size
    k = max(0, min(top_k, n_cand))
    with _on(stream):
        if sel is None:
            sel = _new("full", (pool.num_kv_heads, max(k, 1)), torch.int32, q.device, -1)
        if count is None:
            count = _new("zeros", pool.num_kv_heads, torch.int32, q.device)
        ws = _workspace(select_workspace_bytes(pool, n_q, t0), q.device, workspace)
        score_stride = 0 if score_out is None else score_out.stride(0)
        if _checks_on():
            check_page_tables(table, n_cand, pool.num_pages, "table")
        call("oomb_select_pages", pool.ref(), _ptr(table), table.stride(0), _ptr(q), hs, ts, n_q,
             t0, top_k, _ptr(sel), sel.stride(0), _ptr(count), _ptr(qbar_out), _ptr(score_out),
             score_stride, _ptr(ws), ws.numel(), _stream(stream))
    return sel, count


def select_tiled_workspace_bytes(pool: PagedPool, n_q: int, t0: int, tile: int) -> int:
    return int(lib().oomb_select_tiled_workspace_bytes(pool.ref(), n_q, t0, tile))


def tile_row_length(pool: PagedPool, n_q: int, t0: int, top_k: int, tile: int) -> int:
    """Ids a row of oomb_select_pages_tiled holds at most: top-k plus the chunk's pages
    before the last tile."""
    P = pool.page_size
    n_tiles = max(1, -(-n_q // tile))
    return max(0, min(top_k, t0 // P)) + (t0 + (n_tiles - 1) * tile) // P - t0 // P


def oomb_select_pages_tiled(pool: PagedPool, table: torch.Tensor, q: torch.Tensor, t0: int,
                            top_k: int, tile: int, sel: Optional[torch.Tensor] = None,
                            count: Optional[torch.Tensor] = None,
                            qbar_out: Optional[torch.Tensor] = None,
                            score_out: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None,
                            stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Top-k prior pages per (query tile, KV head). Returns (sel int32 [n_tiles, Hkv,
    stride], count int32 [n_tiles, Hkv]); sel[j] and count[j] are the selection of tile j
    for the attention calls on its queries at position t0 + j * tile."""
    _check_table(table, pool, "table")
    hs, ts = _view(q, pool, pool.num_q_heads, "q")
    n_q = q.shape[1]
    n_tiles = max(1, -(-n_q // tile)) if tile < n_q else 1
    width = max(1, tile_row_length(pool, n_q, t0, top_k, tile))
    with _on(stream):
        if sel is None:
            sel = _new("full", (n_tiles, pool.num_kv_heads, width), torch.int32, q.device, -1)
        if count is None:
            count = _new("zeros", (n_tiles, pool.num_kv_heads), torch.int32, q.device)
        if sel.dim() != 3 or sel.stride(2) != 1 or sel.stride(0) != sel.shape[1] * sel.stride(1):
            raise ValueError("sel must be [n_tiles, Hkv, stride] with contiguous rows")
        if not count.is_contiguous():
            raise ValueError("count must be contiguous [n_tiles, Hkv]")
        ws = _workspace(select_tiled_workspace_bytes(pool, n_q, t0, tile), q.device, workspace)
        score_stride = 0 if score_out is None else score_out.stride(-2)
        call("oomb_select_pages_tiled", pool.ref(), _ptr(table), table.stride(0), _ptr(q), hs, ts,
             n_q, t0, tile, top_k, _ptr(sel), sel.stride(1), _ptr(count), _ptr(qbar_out),
             _ptr(score_out), score_stride, _ptr(ws), ws.numel(), _stream(stream))
    return sel, count


def oomb_select_pages_noalloc(pool: PagedPool, table: torch.Tensor, q: torch.Tensor, t0: int,
                              top_k: int, sel: torch.Tensor, count: torch.Tensor,
                              qbar_out: Optional[torch.Tensor] = None,
                              score_out: Optional[torch.Tensor] = None, stream=None) -> None:
    """oomb_select_pages into the caller's sel [Hkv, >= k] and count [Hkv] (int32, on the
    pool's device), with the library's static scratch instead of a workspace: nothing is
    allocated, here or in the library."""
    _check_table(table, pool, "table")
    hs, ts = _view(q, pool, pool.num_q_heads, "q")
    for name, t in (("sel", sel), ("count", count)):
        if t.dtype != torch.int32 or t.device != pool.device:
            raise ValueError(f"{name} must be an int32 tensor on {pool.device}")
    if sel.dim() != 2 or sel.stride(1) != 1 or count.dim() != 1 or not count.is_contiguous():
        raise ValueError("sel must be [Hkv, k] with contiguous rows, count [Hkv] contiguous")
    score_stride = 0 if score_out is None else score_out.stride(0)
    call("oomb_select_pages_noalloc", pool.ref(), _ptr(table), table.stride(0), _ptr(q), hs, ts,
         q.shape[1], t0, top_k, _ptr(sel), sel.stride(0), _ptr(count), _ptr(qbar_out),
         _ptr(score_out), score_stride, _stream(stream))


def oomb_rope(x: torch.Tensor, pos0: int, theta: float = 10000.0, inverse: bool = False,
              out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Rotary embedding of x [heads, tokens, head_dim] (bf16 or fp32, on the GPU) at
    positions pos0 .. pos0 + tokens - 1; out may be x (in place)."""
    if x.dim() != 3 or x.stride(2) != 1 or not x.is_cuda or x.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("x must be a [heads, tokens, head_dim] bf16/fp32 GPU tensor, last dim contiguous")
    with _on(stream):
        if out is None:
            out = _new("empty", x.shape, x.dtype, x.device)
        if out.shape != x.shape or out.dtype != x.dtype or out.stride(2) != 1:
            raise ValueError("out must match x")
        dt = OOMB_DTYPE_BF16 if x.dtype == torch.bfloat16 else OOMB_DTYPE_FP32
        call("oomb_rope", _ptr(x), x.stride(0), x.stride(1), _ptr(out), out.stride(0),
             out.stride(1), x.shape[0], x.shape[1], x.shape[2], dt, pos0, float(theta),
             int(bool(inverse)), _stream(stream))
    return out


def oomb_page_summarize_mean(pool: PagedPool, table: torch.Tensor, first_page: int, n_pages: int,
                             seq_len: int, kmean: torch.Tensor, stream=None) -> None:
    """Mean-key summaries (fp32 [num_pages, head_dim]) of the listed logical pages."""
    _check_table(table, pool, "table")
    if (kmean.dtype != torch.float32 or kmean.device != pool.device or not kmean.is_contiguous()
            or tuple(kmean.shape) != (pool.num_pages, pool.head_dim)):
        raise ValueError(f"kmean must be a contiguous fp32 [{pool.num_pages}, {pool.head_dim}] "
                         f"tensor on {pool.device}")
    call("oomb_page_summarize_mean", pool.ref(), _ptr(table), table.stride(0), first_page, n_pages,
         seq_len, _ptr(kmean), _stream(stream))


def oomb_select_pages_mean(pool: PagedPool, table: torch.Tensor, q: torch.Tensor, t0: int,
                           top_k: int, kmean: torch.Tensor, sel: Optional[torch.Tensor] = None,
                           count: Optional[torch.Tensor] = None,
                           qbar_out: Optional[torch.Tensor] = None,
                           score_out: Optional[torch.Tensor] = None,
                           workspace: Optional[torch.Tensor] = None,
                           stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """As oomb_select_pages, scoring pages by qbar . kmean (the mean-key summaries)."""
    _check_table(table, pool, "table")
    hs, ts = _view(q, pool, pool.num_q_heads, "q")
    if kmean.dtype != torch.float32 or kmean.device != pool.device or not kmean.is_contiguous():
        raise ValueError("kmean must be a contiguous fp32 tensor on the pool's device")
    n_q = q.shape[1]
    n_cand = t0 // pool.page_size
    k = max(0, min(top_k, n_cand))
    with _on(stream):
        if sel is None:
            sel = _new("full", (pool.num_kv_heads, max(k, 1)), torch.int32, q.device, -1)
        if count is None:
            count = _new("zeros", pool.num_kv_heads, torch.int32, q.device)
        ws = _workspace(select_workspace_bytes(pool, n_q, t0), q.device, workspace)
        score_stride = 0 if score_out is None else score_out.stride(0)
        if _checks_on():
            check_page_tables(table, n_cand, pool.num_pages, "table")
        call("oomb_select_pages_mean", pool.ref(), _ptr(table), table.stride(0), _ptr(q), hs, ts,
             n_q, t0, top_k, _ptr(kmean), _ptr(sel), sel.stride(0), _ptr(count), _ptr(qbar_out),
             _ptr(score_out), score_stride, _ptr(ws), ws.numel(), _stream(stream))
    return sel, count


def oomb_paged_chunk_attn_fwd(pool: PagedPool, table: torch.Tensor, q: torch.Tensor, t0: int,
                              sel: Optional[torch.Tensor] = None,
                              count: Optional[torch.Tensor] = None,
                              scale: Optional[float] = None, o: Optional[torch.Tensor] = None,
                              lse: Optional[torch.Tensor] = None,
                              workspace: Optional[torch.Tensor] = None,
                              window: int = 0,
                              stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Attention of the chunk q [Hq, n_q, D] (first query at position t0) over the
    selected (or all, when sel is None) prior pages and its own pages; with
    window > 0 (sel None), local attention over the `window` most recent positions.
    Returns (O [Hq, n_q, D] in the pool dtype, LSE fp32 [Hq, n_q])."""
    _check_table(table, pool, "table")
    hs, ts = _view(q, pool, pool.num_q_heads, "q")
    n_q = q.shape[1]
    if scale is None:
        scale = pool.head_dim ** -0.5
    with _on(stream):
        if o is None:
            o = _new("empty", q.shape, q.dtype, q.device)
        ohs, ots = _view(o, pool, pool.num_q_heads, "o")
        if lse is None:
            lse = _new("empty", (pool.num_q_heads, n_q), torch.float32, q.device)
        if not lse.is_contiguous() or lse.shape != (pool.num_q_heads, n_q):
            raise ValueError("lse must be a contiguous fp32 [Hq, n_q] tensor")
        sel_stride = 0 if sel is None else sel.stride(0)
        need = fwd_workspace_bytes(pool, n_q, t0, -1 if sel is None else sel_stride, window)
        ws = _workspace(need, q.device, workspace) if need > 0 or workspace is not None else None
        _debug_check(pool, table, t0, n_q, sel, count, window)
        call("oomb_paged_chunk_attn_fwd", pool.ref(), _ptr(table), table.stride(0), _ptr(q), hs,
             ts, n_q, t0, _ptr(sel), sel_stride, _ptr(count), int(window), float(scale), _ptr(o),
             ohs, ots, _ptr(lse), _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
    return o, lse


def oomb_paged_chunk_attn_bwd(pool: PagedPool, table: torch.Tensor, gtable: torch.Tensor,
                              q: torch.Tensor, t0: int, sel: Optional[torch.Tensor],
                              count: Optional[torch.Tensor], o: torch.Tensor, dout: torch.Tensor,
                              lse: torch.Tensor, scale: Optional[float] = None,
                              dq: Optional[torch.Tensor] = None,
                              workspace: Optional[torch.Tensor] = None,
                              window: int = 0,
                              stream=None) -> torch.Tensor:
    """Backward of oomb_paged_chunk_attn_fwd: returns dQ (fp32 [Hq, n_q, D]) and adds
    dK/dV into pool.dk / pool.dv at the pages gtable maps to."""
    _check_table(table, pool, "table")
    _check_table(gtable, pool, "gtable")
    if pool.dk is None:
        raise ValueError("pool has no gradient storage")
    hs, ts = _view(q, pool, pool.num_q_heads, "q")
    n_q = q.shape[1]
    if scale is None:
        scale = pool.head_dim ** -0.5
    ohs, ots = _view(o, pool, pool.num_q_heads, "o")
    dhs, dts = _view(dout, pool, pool.num_q_heads, "dout")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.shape != (pool.num_q_heads, n_q):
        raise ValueError("lse must be a contiguous fp32 [Hq, n_q] tensor")
    sel_stride = 0 if sel is None else sel.stride(0)
    with _on(stream):
        if dq is None:
            dq = _new("empty", (pool.num_q_heads, n_q, pool.head_dim), torch.float32, q.device)
        qhs, qts = _view(dq, pool, pool.num_q_heads, "dq", torch.float32)
        ws = _workspace(bwd_workspace_bytes(pool, n_q, t0, -1 if sel is None else sel_stride,
                                            window), q.device, workspace)
        _debug_check(pool, table, t0, n_q, sel, count, window, gtable)
        call("oomb_paged_chunk_attn_bwd", pool.ref(), _ptr(table), table.stride(0), _ptr(gtable),
             gtable.stride(0), _ptr(q), hs, ts, n_q, t0, _ptr(sel), sel_stride, _ptr(count),
             int(window), float(scale), _ptr(o), ohs, ots, _ptr(dout), dhs, dts, _ptr(lse),
             _ptr(dq), qhs, qts, _ptr(ws), ws.numel(), _stream(stream))
    return dq


def oomb_paged_chunk_attn_fwd_tiled(pool: PagedPool, table: torch.Tensor, q: torch.Tensor,
                                    t0: int, sel: torch.Tensor, count: torch.Tensor, tile: int,
                                    scale: Optional[float] = None,
                                    o: Optional[torch.Tensor] = None, stream=None):
    """Attention of a chunk whose query tiles attend their own selections (sel, count
    from oomb_select_pages_tiled): one forward call per tile, on its queries at position
    t0 + j * tile with sel[j], count[j]. Returns (O [Hq, n_q, D], one LSE [Hq, tile
    length] per tile)."""
    n_q = q.shape[1]
    with _on(stream):
        if o is None:
            o = _new("empty", q.shape, q.dtype, q.device)
    lses = []
    for j, i0 in enumerate(range(0, n_q, tile)):
        i1 = min(n_q, i0 + tile)
        _, lse = oomb_paged_chunk_attn_fwd(pool, table, q[:, i0:i1], t0 + i0, sel[j], count[j],
                                           scale, o=o[:, i0:i1], stream=stream)
        lses.append(lse)
    return o, lses


def oomb_paged_chunk_attn_bwd_tiled(pool: PagedPool, table: torch.Tensor, gtable: torch.Tensor,
                                    q: torch.Tensor, t0: int, sel: torch.Tensor,
                                    count: torch.Tensor, tile: int, o: torch.Tensor,
                                    dout: torch.Tensor, lses, scale: Optional[float] = None,
                                    dq: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Backward of oomb_paged_chunk_attn_fwd_tiled: one backward call per tile (dQ of its
    rows; dK/dV of every tile added into the pool)."""
    n_q = q.shape[1]
    with _on(stream):
        if dq is None:
            dq = _new("empty", (pool.num_q_heads, n_q, pool.head_dim), torch.float32, q.device)
    for j, i0 in enumerate(range(0, n_q, tile)):
        i1 = min(n_q, i0 + tile)
        oomb_paged_chunk_attn_bwd(pool, table, gtable, q[:, i0:i1], t0 + i0, sel[j], count[j],
                                  o[:, i0:i1], dout[:, i0:i1], lses[j], scale, dq=dq[:, i0:i1],
                                  stream=stream)
    return dq


def _pages(x: torch.Tensor, name: str) -> torch.Tensor:
    """A page array [N, ...]: contiguous, on a GPU or in pinned host memory (the kernels
    read and write host pages directly; pageable memory would be rejected by the call)."""
    if not x.is_contiguous() or x.dim() < 2:
        raise ValueError(f"{name} must be a contiguous [pages, ...] tensor")
    if not x.is_cuda and not x.is_pinned():
        raise ValueError(f"{name} is in pageable host memory: allocate it with pin_memory=True")
    return x


def _ids(x: torch.Tensor, name: str) -> torch.Tensor:
    if x.dtype != torch.int32 or not x.is_contiguous() or not (x.is_cuda or x.is_pinned()):
        raise ValueError(f"{name} must be a contiguous int32 tensor on the GPU or pinned")
    return x


def oomb_copy_pages(src: torch.Tensor, dst: torch.Tensor, src_ids: torch.Tensor,
                    dst_ids: torch.Tensor, n: Optional[int] = None,
                    n_dev: Optional[torch.Tensor] = None, stream=None) -> None:
    """dst[dst_ids[i]] = src[src_ids[i]] for i < n (default len(src_ids); or < n_dev[0]),
    pages in device or pinned host memory (the CPU offload of K/V pages)."""
    _pages(src, "src")
    _pages(dst, "dst")
    if src.dtype != dst.dtype or src.shape[1:] != dst.shape[1:]:
        raise ValueError("src and dst pages differ in dtype or shape")
    _ids(src_ids, "src_ids")
    _ids(dst_ids, "dst_ids")
    n = min(src_ids.numel(), dst_ids.numel()) if n is None else n
    if n > min(src_ids.numel(), dst_ids.numel()):
        raise ValueError("n exceeds the id lists")
    page_bytes = src[0].numel() * src.element_size()
    call("oomb_copy_pages", _ptr(src), _ptr(dst), page_bytes, src.shape[0], dst.shape[0],
         _ptr(src_ids), _ptr(dst_ids), n, _ptr(None if n_dev is None else _ids(n_dev, "n_dev")),
         _stream(stream))


def oomb_copy_pages_sdma(src: torch.Tensor, dst: torch.Tensor, src_ids, dst_ids,
                         stream=None) -> None:
    """As oomb_copy_pages, by the copy engines, for id lists the host holds (sequences of
    ints or int32 CPU tensors)."""
    _pages(src, "src")
    _pages(dst, "dst")
    if src.dtype != dst.dtype or src.shape[1:] != dst.shape[1:]:
        raise ValueError("src and dst pages differ in dtype or shape")
    s_ids = torch.as_tensor(src_ids, dtype=torch.int32).contiguous()
    d_ids = torch.as_tensor(dst_ids, dtype=torch.int32).contiguous()
    if s_ids.is_cuda or d_ids.is_cuda or s_ids.numel() != d_ids.numel():
        raise ValueError("id lists must be host int32 lists of equal length")
    page_bytes = src[0].numel() * src.element_size()
    call("oomb_copy_pages_sdma", _ptr(src), _ptr(dst), page_bytes, src.shape[0], dst.shape[0],
         _ptr(s_ids), _ptr(d_ids), s_ids.numel(), _stream(stream))


def oomb_add_pages_f32(src: torch.Tensor, dst: torch.Tensor, src_ids: torch.Tensor,
                       dst_ids: torch.Tensor, n: Optional[int] = None,
                       n_dev: Optional[torch.Tensor] = None, zero_src: bool = False,
                       stream=None) -> None:
    """dst[dst_ids[i]] += src[src_ids[i]] (fp32 pages), then src[src_ids[i]] = 0 if
    zero_src: gradient pages into an fp32 pool elsewhere (e.g. pinned host memory)."""
    _pages(src, "src")
    _pages(dst, "dst")
    if src.dtype != torch.float32 or dst.dtype != torch.float32 or src.shape[1:] != dst.shape[1:]:
        raise ValueError("src and dst must be fp32 page arrays of one page shape")
    _ids(src_ids, "src_ids")
    _ids(dst_ids, "dst_ids")
    n = min(src_ids.numel(), dst_ids.numel()) if n is None else n
    if n > min(src_ids.numel(), dst_ids.numel()):
        raise ValueError("n exceeds the id lists")
    call("oomb_add_pages_f32", _ptr(src), _ptr(dst), src[0].numel(), src.shape[0], dst.shape[0],
         _ptr(src_ids), _ptr(dst_ids), n, _ptr(None if n_dev is None else _ids(n_dev, "n_dev")),
         int(bool(zero_src)), _stream(stream))


def oomb_fetch_selected(pool: PagedPool, table: torch.Tensor, host_k: torch.Tensor,
                        host_v: torch.Tensor, host_table: torch.Tensor, sel: torch.Tensor,
                        count: torch.Tensor, stage: torch.Tensor, n_logical: Optional[int] = None,
                        stream=None) -> None:
    """Copy the selected pages of every KV head from the host copies host_k / host_v
    ([pages, P, D], pinned) into the device staging pages `stage` [Hkv, >= k] and point
    `table` at them, so that the attention calls read them there."""
    _check_table(table, pool, "table")
    for name, x in (("host_k", host_k), ("host_v", host_v)):
        _pages(x, name)
        if x.dtype != pool.dtype or tuple(x.shape[1:]) != (pool.page_size, pool.head_dim):
            raise ValueError(f"{name} must be [pages, {pool.page_size}, {pool.head_dim}] "
                             f"{pool.dtype}")
    if host_k.shape != host_v.shape:
        raise ValueError("host_k and host_v differ in shape")
    for name, x in (("host_table", host_table), ("sel", sel), ("count", count), ("stage", stage)):
        _ids(x, name)
    if host_table.dim() != 2 or sel.dim() != 2 or stage.dim() != 2:
        raise ValueError("host_table, sel and stage must be [Hkv, stride] tensors")
    n_logical = min(table.shape[1], host_table.shape[1]) if n_logical is None else n_logical
    call("oomb_fetch_selected", pool.ref(), _ptr(table), table.stride(0), _ptr(host_k),
         _ptr(host_v), host_k.shape[0], _ptr(host_table), host_table.stride(0), _ptr(sel),
         sel.stride(0), _ptr(count), _ptr(stage), stage.stride(0), n_logical, _stream(stream))


class kernel_timer:
    """Context manager: time every kernel the library launches on this thread with
    HIP events. After exit, `records` holds (kernel name, milliseconds) pairs."""

    def __init__(self, max_records: int = 1 << 16):
        self.max_records = max_records
        self.records = []

    def __enter__(self):
        lib().oomb_profile_enable(1)
        return self

    def __exit__(self, *exc):
        lib().oomb_profile_enable(0)
        names = (ctypes.c_char_p * self.max_records)()
        ms = (ctypes.c_float * self.max_records)()
        n = lib().oomb_profile_collect(names, ms, self.max_records)
        self.records = [(names[i].decode(), float(ms[i])) for i in range(n)]
        return False
