"""Shared pieces of the GPU parity tests: run one chunk (or a chunk sweep) through
the HIP library via its C-ABI binding and through the CPU oracle on identical
inputs, and compare.

Nothing here computes the method: inputs come from `workloads`, expected values
from `oracle`, results from `paged_chunk_attention_amd`.
"""
from __future__ import annotations

import math
import sys
from typing import Optional

import numpy as np
import torch

import oracle as orc
import paged_chunk_attention_amd as pca
import workloads as wl

DEV = "cuda"
TOL = {torch.bfloat16: (2e-2, 1e-2), torch.float32: (1e-5, 1e-5)}
SENTINEL = {torch.bfloat16: 0x7FC1, torch.float32: 0x7FC00001}


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def bits(t: torch.Tensor) -> torch.Tensor:
    t = t.detach().cpu().contiguous()
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def fill_sentinel(t: torch.Tensor) -> None:
    iv = torch.int16 if t.element_size() == 2 else torch.int32
    t.view(iv).fill_(SENTINEL[t.dtype])


def compare(name: str, got: torch.Tensor, ref: torch.Tensor, dtype) -> dict:
    """max-abs and relative-L2 (fp64) of got vs ref, asserted against the dtype's bar."""
    atol, rtol = TOL[dtype]
    g = got.detach().to("cpu", torch.float64)
    r = ref.detach().to("cpu", torch.float64)
    assert g.shape == r.shape, (name, g.shape, r.shape)
    assert torch.isfinite(g).all(), f"{name}: non-finite values"
    diff = g - r
    maxabs = diff.abs().max().item() if diff.numel() else 0.0
    rn = r.norm().item()
    rel = diff.norm().item() / rn if rn > 0 else diff.norm().item()
    log(f"    {name:6s} max_abs={maxabs:.3e} rel_l2={rel:.3e} (bar {atol:g}/{rtol:g})")
    assert maxabs <= atol, f"{name}: max_abs {maxabs} > {atol}"
    assert rel <= rtol, f"{name}: rel_l2 {rel} > {rtol}"
    return {"max_abs": maxabs, "rel_l2": rel}


class GpuLayer:
    """One layer's pool + tables on the GPU, filled through the library's own calls."""

    def __init__(self, w: wl.Workload, x: dict, spare_pages: int = 3):
        self.w = w
        n = w.pool_pages + spare_pages
        self.pool = pca.PagedPool(n, w.page, w.d, w.hq, w.hkv, w.dtype, DEV)
        fill_sentinel(self.pool.k)
        fill_sentinel(self.pool.v)
        fill_sentinel(self.pool.summary)
        g = torch.Generator(device="cpu").manual_seed(1234)
        self.grad_init = torch.randn(n, w.page, w.d, generator=g)
        self.pool.dk.copy_(self.grad_init)
        self.pool.dv.copy_(self.grad_init * 0.5)
        self.table = x["table"].to(DEV)
        self.gtable = x["gtable"].to(DEV)

    def append(self, k, v, start):
        pca.oomb_kv_append(self.pool, self.table, k.to(DEV), v.to(DEV), start)


def oracle_layer(w: wl.Workload, x: dict, upto: int, spare_pages: int = 3):
    """Oracle pool (built by scatter) holding tokens [0, upto)."""
    n = w.pool_pages + spare_pages
    kp = torch.zeros(n, w.page, w.d, dtype=w.dtype)
    vp = torch.zeros(n, w.page, w.d, dtype=w.dtype)
    orc.append(kp, x["table"], x["k"][:, :upto], 0)
    orc.append(vp, x["table"], x["v"][:, :upto], 0)
    summ = torch.zeros(n, 2, w.d, dtype=w.dtype)
    orc.summarize(kp, x["table"], summ, 0, -(-upto // w.page), upto)
    return kp, vp, summ


def run_chunk_parity(w: wl.Workload, x: Optional[dict] = None, label: str = "",
                     pieces=(0.37, 0.71)) -> dict:
    """Append the prior context (in uneven pieces) and the chunk, summarize, select
    (if w.top_k), forward and backward on the GPU; the same on the oracle; compare
    everything. Returns the measured errors."""
    if x is None:
        x = wl.make_inputs(w)
    t0, C, P = w.t0, w.chunk, w.page
    log(f"[case {label or w.name}] hq={w.hq} hkv={w.hkv} d={w.d} page={P} chunk={C} t0={t0} "
        f"dtype={w.dtype} top_k={w.top_k} window={w.window}")
    L = GpuLayer(w, x)
    cuts = sorted({0, *[int(f * t0) for f in pieces], t0})
    for a, b in zip(cuts[:-1], cuts[1:]):
        if b > a:
            L.append(x["k"][:, a:b], x["v"][:, a:b], a)
    L.append(x["k"][:, t0:t0 + C], x["v"][:, t0:t0 + C], t0)
    n_pages_used = -(-(t0 + C) // P)
    pca.oomb_page_summarize(L.pool, L.table, 0, n_pages_used, t0 + C)
    q = x["q"].to(DEV)
    do = x["do"].to(DEV)
    sel = count = None
    n_cand = t0 // P
    res = {}
    if w.top_k is not None:
        qbar = torch.empty(w.hkv, w.d, dtype=torch.float32, device=DEV)
        score = torch.empty(w.hkv, max(n_cand, 1), dtype=torch.float32, device=DEV)
        sel, count = pca.oomb_select_pages(L.pool, L.table, q, t0, w.top_k, qbar_out=qbar,
                                           score_out=score)
    o, lse = pca.oomb_paged_chunk_attn_fwd(L.pool, L.table, q, t0, sel, count, w.scale,
                                           window=w.window)
    dq = pca.oomb_paged_chunk_attn_bwd(L.pool, L.table, L.gtable, q, t0, sel, count, o, do, lse,
                                       w.scale, window=w.window)
    torch.cuda.synchronize()
    log("    gpu done")

    # ---- oracle
    kp, vp, summ = oracle_layer(w, x, t0 + C)
    used = torch.zeros(kp.shape[0], dtype=torch.bool)
    for g in range(w.hkv):
        used[x["table"][g, :n_pages_used].long()] = True
    # paging: stored pages equal the oracle's bitwise (only the written slots),
    # every other slot still holds the sentinel
    gk, gv, gs = L.pool.k.cpu(), L.pool.v.cpu(), L.pool.summary.cpu()
    slot_written = torch.zeros(kp.shape[0], P, dtype=torch.bool)
    for g in range(w.hkv):
        t = torch.arange(t0 + C)
        slot_written[x["table"][g].long()[t // P], t % P] = True
    assert torch.equal(bits(gk)[slot_written], bits(kp)[slot_written]), "K pool differs"
    assert torch.equal(bits(gv)[slot_written], bits(vp)[slot_written]), "V pool differs"
    assert bool((bits(gk)[~slot_written] == SENTINEL[w.dtype]).all()), "K sentinel overwritten"
    assert bool((bits(gv)[~slot_written] == SENTINEL[w.dtype]).all()), "V sentinel overwritten"
    assert torch.equal(bits(gs)[used], bits(summ)[used]), "page summaries differ"
    assert bool((bits(gs)[~used] == SENTINEL[w.dtype]).all()), "summary sentinel overwritten"
    log("    paging + summaries bitwise ok")

    osel = None
    if w.top_k is not None:
        ref = orc.select_pages(x["q"], summ, x["table"], t0, P, w.group, w.top_k)
        gq, gsc = qbar.cpu(), score.cpu()
        gsel, gcnt = sel.cpu(), count.cpu()
        osel = []
        for g, (qb, sc, chosen) in enumerate(ref):
            assert torch.equal(bits(gq[g]), torch.from_numpy(qb).view(torch.int32)), f"qbar head {g}"
            assert torch.equal(bits(gsc[g, :n_cand]), torch.from_numpy(sc).view(torch.int32)), \
                f"scores head {g}"
            assert int(gcnt[g]) == len(chosen), f"count head {g}"
            assert gsel[g, :len(chosen)].tolist() == chosen, f"selection head {g}"
            osel.append(chosen)
        log(f"    selection bit-exact ({[len(s) for s in osel]} pages per head)")

    O, LSE = orc.fwd(x["q"], kp, vp, x["table"], t0, osel, w.scale, window=w.window)
    res["O"] = compare("O", o, O, w.dtype)
    lse_err = (lse.cpu().double() - LSE).abs().max().item()
    log(f"    LSE    max_abs={lse_err:.3e}")
    assert lse_err <= (1e-2 if w.dtype == torch.bfloat16 else 1e-5)
    gpk = torch.zeros(kp.shape, dtype=torch.float64)
    gpv = torch.zeros(kp.shape, dtype=torch.float64)
    dQ, _ = orc.bwd(x["q"], kp, vp, x["table"], t0, osel, w.scale, x["do"], gpk, gpv, x["gtable"],
                    window=w.window)
    res["dQ"] = compare("dQ", dq, dQ, w.dtype)
    # gradient pool: touched rows hold init + dK, everything else is bit-unchanged
    touched = torch.zeros(kp.shape[0], P, dtype=torch.bool)
    for g in range(w.hkv):
        pages = orc.attended_pages(t0, C, P, None if osel is None else osel[g])
        pos = orc.key_positions(pages, P, t0 + C)
        touched[x["gtable"][g].long()[pos // P], pos % P] = True
    gdk, gdv = L.pool.dk.cpu(), L.pool.dv.cpu()
    assert torch.equal(bits(gdk)[~touched], bits(L.grad_init)[~touched]), "dK pool rows touched"
    assert torch.equal(bits(gdv)[~touched], bits(L.grad_init * 0.5)[~touched]), "dV pool rows touched"
    res["dK"] = compare("dK", (gdk.double() - L.grad_init.double())[touched], gpk[touched], w.dtype)
    res["dV"] = compare("dV", (gdv.double() - (L.grad_init * 0.5).double())[touched], gpv[touched],
                        w.dtype)
    return res
