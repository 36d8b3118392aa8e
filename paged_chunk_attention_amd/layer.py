"""One attention layer of a chunk-recurrent transformer, on the paged library.

The sequence is processed in chunks (gist.science explainer of OOMB, 2.A "Chunk-Recurrent
Training with Activation Recomputation"): the forward runs chunk by chunk, appending each
chunk's keys and values into the paged cache (2.B) and attending to the cache (optionally
to the top-k prior pages, 2.D, or within a local window), and keeps no activations but the
layer input. The backward walks the chunks in reverse, recomputes each chunk's Q/K/V and
attention output just before use, adds the key/value gradients into the paged fp32
gradient pool in place, and reads a chunk's own key/value gradients back once every later
chunk has contributed to them. The cache is outside PyTorch's autograd graph (2.B,
"Autograd Bypass"): it is state of the layer, not a saved tensor.

Projections are plain library GEMMs (torch matmul on hipBLASLt); rotary embedding,
paging, selection and attention run in the library's kernels. Weights are synthetic.
"""
from __future__ import annotations

import math
from typing import List, Optional, Tuple

import torch

from .binding import (
    PagedPool,
    bwd_workspace_bytes,
    fwd_workspace_bytes,
    oomb_copy_pages,
    oomb_kv_append,
    oomb_page_summarize,
    oomb_paged_chunk_attn_bwd,
    oomb_paged_chunk_attn_fwd,
    oomb_rope,
    oomb_select_pages,
)


_MM_OUT_F32: Optional[bool] = None


def _mm_f32(a: torch.Tensor, b: torch.Tensor) -> torch.Tensor:
    """a @ b with bf16 operands, fp32 accumulation and an fp32 result (the plain bf16
    product widened where the fp32-output form is not available). b is contiguous."""
    global _MM_OUT_F32
    if _MM_OUT_F32 is not False:
        try:
            c = torch.mm(a, b, out_dtype=torch.float32)
            _MM_OUT_F32 = True
            return c
        except (NotImplementedError, RuntimeError, TypeError):
            _MM_OUT_F32 = False
    return torch.mm(a, b).float()


class ChunkRecurrentAttention(torch.nn.Module):
    """Grouped-query self-attention over `max_tokens` tokens, trained chunk by chunk.

    x [T, hidden] -> y [T, hidden]; T a multiple of `chunk`, `chunk` a multiple of
    `page`. q = RoPE(x Wq), k = RoPE(x Wk), v = x Wv (positions are the tokens' absolute
    positions), o = attention(q, k, v) over the cache, y = o Wo."""

    def __init__(self, hidden: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 page: int, chunk: int, max_tokens: int, top_k: Optional[int] = None,
                 window: int = 0, rope_theta: float = 1.0e6, dtype=torch.bfloat16,
                 device="cuda", seed: int = 0):
        super().__init__()
        if chunk % page or max_tokens % chunk:
            raise ValueError("chunk must be a multiple of page, max_tokens of chunk")
        if top_k is not None and window:
            raise ValueError("a layer is top-k or local, not both")
        self.hq, self.hkv, self.d = num_q_heads, num_kv_heads, head_dim
        self.page, self.chunk, self.max_tokens = page, chunk, max_tokens
        self.top_k, self.window, self.theta = top_k, window, rope_theta
        self.scale = 1.0 / math.sqrt(head_dim)
        g = torch.Generator(device="cpu").manual_seed(seed)

        def w(rows, cols):
            t = torch.randn(rows, cols, generator=g) / math.sqrt(rows)
            return torch.nn.Parameter(t.to(device=device, dtype=dtype))

        self.wq = w(hidden, num_q_heads * head_dim)
        self.wk = w(hidden, num_kv_heads * head_dim)
        self.wv = w(hidden, num_kv_heads * head_dim)
        self.wo = w(num_q_heads * head_dim, hidden)
        pages_per_head = max_tokens // page
        # the allocator: each KV head owns a contiguous run of physical pages, in a
        # seeded order (pages need not be in logical order)
        perm = torch.randperm(pages_per_head, generator=g).to(torch.int32)
        table = torch.stack([perm + h * pages_per_head for h in range(num_kv_heads)])
        self.table = table.to(device)
        self.pool = PagedPool(num_kv_heads * pages_per_head, page, head_dim, num_q_heads,
                              num_kv_heads, dtype, device)
        self.sels: List[Tuple[Optional[torch.Tensor], Optional[torch.Tensor]]] = []

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return _ChunkRecurrentFn.apply(x, self.wq, self.wk, self.wv, self.wo, self)

    # ---- pieces of one chunk -------------------------------------------------------------
    def _heads(self, t: torch.Tensor, n: int) -> torch.Tensor:
        """[C, n * D] -> [n, C, D] contiguous."""
        return t.view(t.shape[0], n, self.d).transpose(0, 1).contiguous()

    def _qkv(self, xc: torch.Tensor, t0: int):
        q = oomb_rope(self._heads(xc @ self.wq, self.hq), t0, self.theta)
        k = oomb_rope(self._heads(xc @ self.wk, self.hkv), t0, self.theta)
        v = self._heads(xc @ self.wv, self.hkv)
        return q, k, v

    def _attend(self, q, t0, sel, count, o=None, lse=None):
        sstride = -1 if sel is None else sel.stride(0)
        ws = torch.empty(max(256, fwd_workspace_bytes(self.pool, self.chunk, t0, sstride,
                                                      self.window)),
                         dtype=torch.uint8, device=q.device)
        return oomb_paged_chunk_attn_fwd(self.pool, self.table, q, t0, sel, count, self.scale,
                                         o=o, lse=lse, workspace=ws, window=self.window)

    def _chunk_rows(self, t0: int) -> torch.Tensor:
        """Physical pages of the chunk's tokens, head by head: [Hkv * C/P] int32."""
        lp0 = t0 // self.page
        return self.table[:, lp0:lp0 + self.chunk // self.page].contiguous().flatten()


class _ChunkRecurrentFn(torch.autograd.Function):
    """Forward: chunks in order, nothing saved but x and the weights (plus each chunk's
    page selection, k ids per KV head). Backward: chunks in reverse with recomputation;
    key/value gradients accumulate in the paged pool in place."""

    @staticmethod
    def forward(ctx, x, wq, wk, wv, wo, layer: ChunkRecurrentAttention):
        T, C, P = x.shape[0], layer.chunk, layer.page
        if T % C or T > layer.max_tokens:
            raise ValueError(f"sequence of {T} tokens does not fit chunks of {C} up to "
                             f"{layer.max_tokens}")
        layer.sels = []
        y = torch.empty(T, wo.shape[1], dtype=x.dtype, device=x.device)
        with torch.no_grad():
            for t0 in range(0, T, C):
                xc = x[t0:t0 + C]
                q, k, v = layer._qkv(xc, t0)
                oomb_kv_append(layer.pool, layer.table, k, v, t0)
                oomb_page_summarize(layer.pool, layer.table, t0 // P, C // P, t0 + C)
                sel = count = None
                if layer.top_k is not None:
                    sel, count = oomb_select_pages(layer.pool, layer.table, q, t0, layer.top_k)
                o, _ = layer._attend(q, t0, sel, count)
                layer.sels.append((sel, count))
                y[t0:t0 + C] = o.transpose(0, 1).reshape(C, -1) @ wo
        ctx.layer = layer
        ctx.save_for_backward(x, wq, wk, wv, wo)
        return y

    @staticmethod
    def backward(ctx, dy):
        x, wq, wk, wv, wo = ctx.saved_tensors
        layer: ChunkRecurrentAttention = ctx.layer
        T, C, P, D = x.shape[0], layer.chunk, layer.page, layer.d
        pool = layer.pool
        pool.dk.zero_()
        pool.dv.zero_()
        f32, cdt = torch.float32, x.dtype
        dx = torch.empty(T, x.shape[1], dtype=f32, device=x.device)
        dwq, dwk, dwv, dwo = (torch.zeros(w.shape, dtype=f32, device=x.device)
                              for w in (wq, wk, wv, wo))
        # transposed weights, contiguous, once: every right operand below is contiguous
        wqT, wkT, wvT, woT = (w.t().contiguous() for w in (wq, wk, wv, wo))
        mm = _mm_f32 if cdt == torch.bfloat16 else torch.mm
        n_pg = C // P
        gk = torch.empty(layer.hkv * n_pg, P, D, dtype=f32, device=x.device)
        gv = torch.empty_like(gk)
        dst = torch.arange(layer.hkv * n_pg, dtype=torch.int32, device=x.device)
        with torch.no_grad():
            for ci in reversed(range(T // C)):
                t0 = ci * C
                xc = x[t0:t0 + C]
                sel, count = layer.sels[ci]
                # recompute the chunk's activations just before they are needed
                q, _, _ = layer._qkv(xc, t0)
                o, lse = layer._attend(q, t0, sel, count)
                dyc = dy[t0:t0 + C].contiguous()
                o2 = o.transpose(0, 1).reshape(C, -1)
                dwo += mm(o2.t(), dyc)
                do = layer._heads(dyc @ woT, layer.hq)
                sstride = -1 if sel is None else sel.stride(0)
                ws = torch.empty(bwd_workspace_bytes(pool, C, t0, sstride, layer.window),
                                 dtype=torch.uint8, device=x.device)
                dq = oomb_paged_chunk_attn_bwd(pool, layer.table, layer.table, q, t0, sel, count,
                                               o, do, lse, layer.scale, workspace=ws,
                                               window=layer.window)
                # the chunk's own keys now hold every contribution (later chunks came first)
                rows = layer._chunk_rows(t0)
                oomb_copy_pages(pool.dk, gk, rows, dst)
                oomb_copy_pages(pool.dv, gv, rows, dst)
                # through the rotary embedding (a rotation: its transpose is the inverse)
                dq = oomb_rope(dq, t0, layer.theta, inverse=True)
                dk = oomb_rope(gk.view(layer.hkv, C, D), t0, layer.theta, inverse=True)
                dq2 = dq.transpose(0, 1).reshape(C, -1).to(cdt)
                dk2 = dk.transpose(0, 1).reshape(C, -1).to(cdt)
                dv2 = gv.view(layer.hkv, C, D).transpose(0, 1).reshape(C, -1).to(cdt)
                xt = xc.t()
                dwq += mm(xt, dq2)
                dwk += mm(xt, dk2)
                dwv += mm(xt, dv2)
                dx[t0:t0 + C] = mm(dq2, wqT) + mm(dk2, wkT) + mm(dv2, wvT)
        return (dx.to(x.dtype), dwq.to(wq.dtype), dwk.to(wk.dtype), dwv.to(wv.dtype),
                dwo.to(wo.dtype), None)
