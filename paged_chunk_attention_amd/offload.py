"""A stack of attention layers whose paged key/value caches live in pinned host memory,
run one chunk at a time with the transfers hidden behind compute (gist.science explainer
of OOMB, 2.C "Asynchronous KV Cache CPU Offloading": the cache and its gradients are kept
on the CPU; for dense and local layers the next layer's pages are fetched while the
current layer computes, for sparse layers only the selected pages move).

One step is the forward of the chunk through layers 0..L-1, then its backward through
layers L-1..0 (the attention part of a chunk-recurrent training step; the queries,
chunk keys/values and output gradients of every layer are inputs). Per layer:
  forward:  [fetch stream] bring the layer's attended pages into one of two device
            staging buffers, one layer ahead; [compute stream] append the chunk's keys
            and values, attend; [write-back stream] write the chunk's new pages back to
            the host cache.
  backward: [fetch stream] bring the layer's attended pages again, one layer ahead;
            [compute stream] attention backward into the staging gradient pages;
            [write-back stream] move those gradient pages into the host gradient pool.
Dense layers fetch every page of the layer (one copy-engine transfer per KV head, the
host pages of a head being consecutive), and for the backward also the layer's host
gradient pages: the backward adds into them and the copy kernel writes them back.
Fetches use the copy engines and write-backs the copy kernel because two copy-engine
streams share one direction's bandwidth (57 GB/s in all), while a copy engine and a
kernel moving data the opposite way use both directions of the link at once (95 GB/s
measured on one MI355X). Sparse layers select first (the selection reads
page summaries kept on the device), gather only the selected pages with the fetch
kernel, and add their gradient pages into the host pool with the add kernel. In this
stack every layer's queries are given, so a sparse layer's selection and fetch can
also run one layer ahead; in a full model, where a layer's queries depend on the layer
below, they would overlap the layer's own key/value projection instead.

Buffers are reused only after the events that order them: a staging buffer is
refilled once the compute that read it and the write-backs out of it have finished,
and a layer's pages are fetched for the backward once its chunk pages have reached
the host. The events persist across steps, so consecutive chunk steps overlap.

The overlap needs each of the three streams on its own hardware queue: with HIP's
default of four queues per process, streams made earlier can leave a copy stream on
the compute stream's queue, where it waits behind the attention kernels. Run with
GPU_MAX_HW_QUEUES=8 (bench.py sets it). Copy kernels cannot run beside the attention
kernels (those fill the register file of every SIMD), so on the compute units they run
only in the gaps between kernels; the copy engines run beside them. The results equal those of the same calls
on an all-resident cache bit for bit (the kernels' results do not depend on where the
pages sit), which `resident_step` computes for comparison and timing.
"""
from __future__ import annotations

from typing import List, Optional

import torch

from .binding import (
    PagedPool,
    bwd_workspace_bytes,
    fwd_workspace_bytes,
    oomb_add_pages_f32,
    oomb_copy_pages,
    oomb_copy_pages_sdma,
    oomb_fetch_selected,
    oomb_kv_append,
    oomb_page_summarize,
    oomb_paged_chunk_attn_bwd,
    oomb_paged_chunk_attn_fwd,
    oomb_select_pages,
    select_workspace_bytes,
)


class OffloadedAttentionStack:
    """L attention layers over one shared geometry: Hq/Hkv heads of D, pages of P
    tokens, a prior context of `prior` tokens and chunks of `chunk` queries; dense
    (top_k None) or top-k sparse. Host memory per layer: K and V pages plus fp32 dK
    and dV pages for the whole context, all pinned; host page of (KV head g, logical
    page j) is g * pages_per_head + j. With grads_on_host False the gradient pools stay
    in device memory (same layout) and only keys and values move."""

    def __init__(self, n_layers: int, hq: int, hkv: int, d: int, page: int, prior: int,
                 chunk: int, top_k: Optional[int] = None, dtype=torch.bfloat16,
                 device="cuda", grads_on_host: bool = True):
        if prior % page:
            raise ValueError("the prior context must fill whole pages")
        self.L, self.hq, self.hkv, self.d, self.P = n_layers, hq, hkv, d, page
        self.prior, self.chunk, self.top_k, self.dtype = prior, chunk, top_k, dtype
        self.dev = torch.device(device)
        self.t0 = prior
        self.n_prior = prior // page
        self.first_local = self.n_prior
        self.n_local = (prior + chunk - 1) // page - self.first_local + 1
        self.npph = self.first_local + self.n_local             # pages per head
        self.scale = d ** -0.5
        n_host = hkv * self.npph
        shape = (n_host, page, d)
        self.hk = [torch.zeros(shape, dtype=dtype, pin_memory=True) for _ in range(n_layers)]
        self.hv = [torch.zeros(shape, dtype=dtype, pin_memory=True) for _ in range(n_layers)]
        # fp32 gradient pools: pinned host memory, or (grads_on_host False) device memory,
        # where the backward adds into them directly and only keys and values move
        self.grads_on_host = grads_on_host
        gkw = dict(pin_memory=True) if grads_on_host else dict(device=device)
        self.hdk = [torch.zeros(shape, dtype=torch.float32, **gkw) for _ in range(n_layers)]
        self.hdv = [torch.zeros(shape, dtype=torch.float32, **gkw) for _ in range(n_layers)]
        dv = self.dev
        ident = torch.arange(n_host, dtype=torch.int32).reshape(hkv, self.npph)
        self.host_table = ident.pin_memory()                   # (g, j) -> host page
        self.ident = ident.to(dv)
        self.summary: List[Optional[torch.Tensor]] = [None] * n_layers
        # staging: two buffers, each with its own gradient pages
        if top_k is None:
            n_stage = n_host                                   # the whole layer
            self.k_sel = 0
        else:
            self.k_sel = max(1, min(top_k, self.n_prior))
            n_stage = hkv * (self.k_sel + self.n_local)
        self.stage = [PagedPool(n_stage, page, d, hq, hkv, dtype, dv, with_summary=False)
                      for _ in range(2)]
        if top_k is None:
            self.tables = [self.ident, self.ident]
        else:
            # staging page of selection slot s of head g: g * (k + n_local) + s; of the
            # chunk's r-th page: g * (k + n_local) + k + r
            per = self.k_sel + self.n_local
            self.stage_ids = (torch.arange(hkv, dtype=torch.int32)[:, None] * per
                              + torch.arange(self.k_sel, dtype=torch.int32)[None, :]).to(dv)
            self.tables = []
            for _ in range(2):
                t = torch.full((hkv, self.npph), -1, dtype=torch.int32)
                for g in range(hkv):
                    for r in range(self.n_local):
                        t[g, self.first_local + r] = g * per + self.k_sel + r
                self.tables.append(t.to(dv))
            self.sel = [torch.zeros(hkv, self.k_sel, dtype=torch.int32, device=dv)
                        for _ in range(n_layers)]
            self.count = [torch.zeros(hkv, dtype=torch.int32, device=dv) for _ in range(n_layers)]
            self.ws_sel = torch.empty(select_workspace_bytes(self.stage[0], chunk, prior),
                                      dtype=torch.uint8, device=dv)
        sstride = -1 if top_k is None else self.k_sel
        self.ws_fwd = torch.empty(max(256, fwd_workspace_bytes(self.stage[0], chunk, prior,
                                                               sstride)),
                                  dtype=torch.uint8, device=dv)
        self.ws_bwd = torch.empty(bwd_workspace_bytes(self.stage[0], chunk, prior, sstride),
                                  dtype=torch.uint8, device=dv)
        # Three streams made one after the other: HIP gives streams its hardware queues in
        # turn (four by default), so consecutive ones never share a queue, and a copy
        # stream sharing the compute stream's queue would wait behind its kernels. Steps
        # therefore compute on their own stream, ordered after and before the caller's.
        self.compute_stream = torch.cuda.Stream(device=dv)
        self.copy_stream = torch.cuda.Stream(device=dv)    # host -> device
        self.wb_stream = torch.cuda.Stream(device=dv)      # device -> host
        self._ev = None
        # page id lists of the transfers (device int32)
        self.local_host = torch.cat([g * self.npph + self.first_local +
                                     torch.arange(self.n_local, dtype=torch.int32)
                                     for g in range(hkv)])
        if top_k is None:
            self.local_stage = self.local_host
        else:
            per = self.k_sel + self.n_local
            self.local_stage = torch.cat([g * per + self.k_sel +
                                          torch.arange(self.n_local, dtype=torch.int32)
                                          for g in range(hkv)])
        self.local_host_dev = self.local_host.to(dv)
        # first host page of each KV head, for the write-back of selected gradient pages
        self.head_base = (torch.arange(hkv, dtype=torch.int32) * self.npph)[:, None].to(dv)
        self.local_stage_dev = self.local_stage.to(dv)
        # the id lists and tables above were written on the current stream; the step reads
        # them on its own streams
        torch.cuda.synchronize(dv)

    # ---- setup ------------------------------------------------------------------------
    def load_prior(self, layer: int, k: torch.Tensor, v: torch.Tensor) -> None:
        """Write the prior context [Hkv, prior, D] of one layer into its host cache, and
        (sparse) keep its page summaries on the device: built through the library on a
        temporary device pool, then copied out."""
        tmp = PagedPool(self.hkv * self.npph, self.P, self.d, self.hq, self.hkv, self.dtype,
                        self.dev, with_summary=self.top_k is not None, with_grad=False)
        oomb_kv_append(tmp, self.ident, k.to(self.dev), v.to(self.dev), 0)
        if self.top_k is not None:
            oomb_page_summarize(tmp, self.ident, 0, self.n_prior, self.prior)
            self.summary[layer] = tmp.summary
        self.hk[layer].copy_(tmp.k)
        self.hv[layer].copy_(tmp.v)
        torch.cuda.synchronize(self.dev)

    def zero_grad(self) -> None:
        for t in self.hdk + self.hdv:
            t.zero_()

    # ---- pieces -----------------------------------------------------------------------
    def _att_pool(self, b: int) -> PagedPool:
        return self.stage[b]

    def _sel_pool(self, layer: int) -> PagedPool:
        """Descriptor for the selection of `layer`: its summaries, indexed by host page."""
        s = self.stage[0]
        return PagedPool.from_tensors(s.k, s.v, self.summary[layer], None, None, self.hq,
                                      self.hkv, num_pages=self.hkv * self.npph)

    def _select(self, layer: int, q: torch.Tensor, stream) -> None:
        oomb_select_pages(self._sel_pool(layer), self.ident, q, self.t0, self.top_k,
                          sel=self.sel[layer], count=self.count[layer], workspace=self.ws_sel,
                          stream=stream)

    def _fetch(self, layer: int, b: int, with_local: bool, stream) -> None:
        """Bring layer `layer`'s attended pages into staging buffer b (on `stream`)."""
        pool = self.stage[b]
        if self.top_k is None:
            n = self.npph if with_local else self.n_prior
            for g in range(self.hkv):
                ids = list(range(g * self.npph, g * self.npph + n))
                oomb_copy_pages_sdma(self.hk[layer], pool.k, ids, ids, stream=stream)
                oomb_copy_pages_sdma(self.hv[layer], pool.v, ids, ids, stream=stream)
            return
        oomb_fetch_selected(pool, self.tables[b], self.hk[layer], self.hv[layer],
                            self.host_table, self.sel[layer], self.count[layer],
                            self.stage_ids, n_logical=self.n_prior, stream=stream)
        if with_local:
            for g in range(self.hkv):
                src = [g * self.npph + self.first_local + r for r in range(self.n_local)]
                per = self.k_sel + self.n_local
                dst = [g * per + self.k_sel + r for r in range(self.n_local)]
                oomb_copy_pages_sdma(self.hk[layer], pool.k, src, dst, stream=stream)
                oomb_copy_pages_sdma(self.hv[layer], pool.v, src, dst, stream=stream)

    def _write_back_local(self, layer: int, b: int, stream) -> None:
        """The chunk's new pages of `layer` from staging buffer b into the host cache (by
        the copy kernel: write-backs run on compute units, fetches on the copy engines,
        so the two directions of the link are used at once)."""
        pool = self.stage[b]
        oomb_copy_pages(pool.k, self.hk[layer], self.local_stage_dev, self.local_host_dev,
                        stream=stream)
        oomb_copy_pages(pool.v, self.hv[layer], self.local_stage_dev, self.local_host_dev,
                        stream=stream)

    def _write_back_grads(self, layer: int, b: int, stream) -> None:
        """Add the staging gradient pages of `layer`'s attended pages into its host
        gradient pool (fp32, one rounding per element)."""
        pool = self.stage[b]
        if self.top_k is None:
            ids = self.ident.reshape(-1)
            src = dst = ids
        else:
            # selected pages: staging slot -> host page g * npph + selected id; the
            # chunk's own pages: fixed staging pages -> their host pages
            with torch.cuda.stream(stream):
                sel_host = (self.sel[layer] + self.head_base).reshape(-1)
                src = torch.cat([self.stage_ids.reshape(-1), self.local_stage_dev])
                dst = torch.cat([sel_host, self.local_host_dev])
        oomb_add_pages_f32(pool.dk, self.hdk[layer], src, dst, stream=stream)
        oomb_add_pages_f32(pool.dv, self.hdv[layer], src, dst, stream=stream)

    # ---- the step ---------------------------------------------------------------------
    def _fetch_grads(self, layer: int, b: int, stream) -> None:
        """Dense layers: bring the layer's host gradient pages into staging buffer b (the
        backward adds into them; the write-back then copies them out whole)."""
        pool = self.stage[b]
        for g in range(self.hkv):
            ids = list(range(g * self.npph, (g + 1) * self.npph))
            oomb_copy_pages_sdma(self.hdk[layer], pool.dk, ids, ids, stream=stream)
            oomb_copy_pages_sdma(self.hdv[layer], pool.dv, ids, ids, stream=stream)

    def _copy_out_grads(self, layer: int, b: int, stream) -> None:
        """Dense layers: the staging gradient pages (host values plus this step's) back into
        the host gradient pool, by the copy kernel (see _write_back_local)."""
        pool = self.stage[b]
        ids = self.ident.reshape(-1)
        oomb_copy_pages(pool.dk, self.hdk[layer], ids, ids, stream=stream)
        oomb_copy_pages(pool.dv, self.hdv[layer], ids, ids, stream=stream)

    def _events(self):
        if getattr(self, "_ev", None) is None:
            cs = self.compute_stream
            ev = {}
            for name, n in (("kv_free", 2), ("local_out", 2), ("grads_out", 2), ("home", self.L)):
                ev[name] = [torch.cuda.Event() for _ in range(n)]
                for e in ev[name]:
                    e.record(cs)
            self._ev = ev
            self._base = 0
        return self._ev

    def step(self, q: List[torch.Tensor], k_new: List[torch.Tensor], v_new: List[torch.Tensor],
             dout: List[torch.Tensor], o: List[torch.Tensor], lse: List[torch.Tensor],
             dq: List[torch.Tensor], join: bool = True) -> None:
        """Forward then backward of one chunk through every layer, transfers overlapped.
        Writes o, lse, dq per layer; adds dK/dV into the host gradient pools and the
        chunk's keys and values into the host caches. Fetches run on one copy stream,
        write-backs on another. With join, the current stream waits for every transfer
        at the end; without, the next step's first transfers overlap this step's last
        compute and write-backs (the events that order the staging buffers and the host
        caches persist across steps, and each step starts in the buffer the previous
        one finished with least recently)."""
        L = self.L
        caller = torch.cuda.current_stream(self.dev)
        cs = self.compute_stream
        cs.wait_stream(caller)                                 # the step's inputs are ready
        h2d, d2h = self.copy_stream, self.wb_stream
        sparse = self.top_k is not None
        E = self._events()
        kv_free, local_out, grads_out, home = E["kv_free"], E["local_out"], E["grads_out"], E["home"]
        new = lambda: torch.cuda.Event()                      # noqa: E731
        fetched = [new() for _ in range(L)]
        base = self._base

        def fbuf(i):
            return (base + i) % 2

        # ---------------- forward: layer i on buffer fbuf(i)
        def issue_fetch_fwd(i):
            b = fbuf(i)
            if sparse:
                sel_done = new()
                self._select(i, q[i], cs)
                sel_done.record(cs)
                h2d.wait_event(sel_done)
            h2d.wait_event(kv_free[b])
            h2d.wait_event(home[i])          # the layer's host cache holds its last chunk
            self._fetch(i, b, with_local=False, stream=h2d)
            fetched[i].record(h2d)

        issue_fetch_fwd(0)
        for i in range(L):
            b = fbuf(i)
            if i + 1 < L:
                issue_fetch_fwd(i + 1)
            pool, table = self.stage[b], self.tables[b]
            cs.wait_event(fetched[i])
            cs.wait_event(local_out[b])     # the local pages' last write-back has read them
            oomb_kv_append(pool, table, k_new[i], v_new[i], self.t0, stream=cs)
            s_, c_ = (self.sel[i], self.count[i]) if sparse else (None, None)
            oomb_paged_chunk_attn_fwd(pool, table, q[i], self.t0, s_, c_, self.scale, o=o[i],
                                      lse=lse[i], workspace=self.ws_fwd, stream=cs)
            done = new()
            done.record(cs)
            kv_free[b] = done
            d2h.wait_event(done)
            self._write_back_local(i, b, d2h)
            lo = new()
            lo.record(d2h)
            local_out[b] = lo
            home[i] = lo

        # ---------------- backward: layer L-1 stays in its buffer (its keys and values are
        # still there), then the buffers alternate
        last_b = fbuf(L - 1)
        fetched_b = [new() for _ in range(L)]

        def bbuf(i):
            return (last_b + (L - 1 - i)) % 2

        def issue_fetch_bwd(i, kv):
            b = bbuf(i)
            if kv:   # keys and values: once the buffer's readers are done
                h2d.wait_event(kv_free[b])
                h2d.wait_event(local_out[b])
                h2d.wait_event(home[i])
                self._fetch(i, b, with_local=True, stream=h2d)
            if not sparse and self.grads_on_host:
                # gradient pages: once the last write-back out of them is done
                h2d.wait_event(grads_out[b])
                self._fetch_grads(i, b, h2d)
            fetched_b[i].record(h2d)

        issue_fetch_bwd(L - 1, kv=False)
        for i in reversed(range(L)):
            b = bbuf(i)
            if i - 1 >= 0:
                issue_fetch_bwd(i - 1, kv=True)
            pool, table = self.stage[b], self.tables[b]
            cs.wait_event(fetched_b[i])
            gtable = table
            if not self.grads_on_host:
                # gradients straight into the layer's device pool (logical page layout)
                pool = PagedPool.from_tensors(pool.k, pool.v, None, self.hdk[i], self.hdv[i],
                                              self.hq, self.hkv)
                gtable = self.ident
            elif sparse:
                cs.wait_event(grads_out[b])
                with torch.cuda.stream(cs):
                    pool.dk.zero_()
                    pool.dv.zero_()
            s_, c_ = (self.sel[i], self.count[i]) if sparse else (None, None)
            oomb_paged_chunk_attn_bwd(pool, table, gtable, q[i], self.t0, s_, c_, o[i],
                                      dout[i], lse[i], self.scale, dq=dq[i],
                                      workspace=self.ws_bwd, stream=cs)
            done = new()
            done.record(cs)
            kv_free[b] = done
            if self.grads_on_host:
                d2h.wait_event(done)
                if sparse:
                    self._write_back_grads(i, b, d2h)
                else:
                    self._copy_out_grads(i, b, d2h)
                go = new()
                go.record(d2h)
                grads_out[b] = go
        # the next step starts in the buffer the last backward layer did not use
        self._base = 1 - bbuf(0)
        caller.wait_stream(cs)
        if join:
            caller.wait_stream(h2d)
            caller.wait_stream(d2h)

    def resident_step(self, pools: List[PagedPool], q, k_new, v_new, dout, o, lse, dq) -> None:
        """The same chunk step on all-resident caches (pools[i]: the layer's whole cache
        on the device, identity table, zeroed gradient pages), on one stream."""
        sparse = self.top_k is not None
        for i in range(self.L):
            oomb_kv_append(pools[i], self.ident, k_new[i], v_new[i], self.t0)
            s_ = c_ = None
            if sparse:
                s_, c_ = self.sel[i], self.count[i]
                oomb_select_pages(pools[i], self.ident, q[i], self.t0, self.top_k, sel=s_,
                                  count=c_, workspace=self.ws_sel)
            oomb_paged_chunk_attn_fwd(pools[i], self.ident, q[i], self.t0, s_, c_, self.scale,
                                      o=o[i], lse=lse[i], workspace=self.ws_fwd)
        for i in reversed(range(self.L)):
            s_, c_ = (self.sel[i], self.count[i]) if sparse else (None, None)
            oomb_paged_chunk_attn_bwd(pools[i], self.ident, self.ident, q[i], self.t0, s_, c_,
                                      o[i], dout[i], lse[i], self.scale, dq=dq[i],
                                      workspace=self.ws_bwd)

    def resident_pools(self) -> List[PagedPool]:
        """All-resident copies of the host caches (for comparison and timing)."""
        pools = []
        for i in range(self.L):
            p = PagedPool(self.hkv * self.npph, self.P, self.d, self.hq, self.hkv, self.dtype,
                          self.dev, with_summary=self.top_k is not None)
            p.k.copy_(self.hk[i])
            p.v.copy_(self.hv[i])
            if self.top_k is not None:
                p.summary.copy_(self.summary[i])
            pools.append(p)
        return pools
