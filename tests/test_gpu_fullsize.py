"""GPU parity at full workload sizes, in the launch configuration bench.py times,
and the chunk-recurrent sweep.

Full sizes: page selection is compared bit for bit for every KV head; O, LSE and dQ
on sampled query rows that the oracle evaluates one by one (each over exactly the
keys that row attends); dK/dV elementwise for one whole KV group where the oracle
can afford it (1M context), else through identities that hold at any size:
  sum_t dV_t = sum_{h in group, i} dO_hi      (rows of P sum to one)
  sum_t dK_t = 0                              (sum_t dS_it = dO_i.O_i - Delta_i = 0)
"""
import numpy as np
import pytest
import torch

import oracle as orc
import paged_chunk_attention_amd as pca
import workloads as wl
from tests.gpu_harness import DEV, SENTINEL, bits, compare, fill_sentinel, log

pytestmark = pytest.mark.gpu


def _gpu_step(w, x, spare=3):
    """The step bench.py times (append prior + chunk, summarize, select, fwd, bwd)."""
    t0, C, P = w.t0, w.chunk, w.page
    pool = pca.PagedPool(w.pool_pages + spare, P, w.d, w.hq, w.hkv, w.dtype, DEV)
    fill_sentinel(pool.k)
    fill_sentinel(pool.v)
    table, gtable = x["table"].to(DEV), x["gtable"].to(DEV)
    pca.oomb_kv_append(pool, table, x["k"][:, :t0], x["v"][:, :t0], 0)
    pca.oomb_page_summarize(pool, table, 0, t0 // P, t0)
    pca.oomb_kv_append(pool, table, x["k"][:, t0:t0 + C].contiguous(),
                       x["v"][:, t0:t0 + C].contiguous(), t0)
    pca.oomb_page_summarize(pool, table, t0 // P, (t0 + C - 1) // P - t0 // P + 1, t0 + C)
    sel = count = qbar = score = None
    if w.top_k is not None:
        n_cand = t0 // P
        qbar = torch.empty(w.hkv, w.d, dtype=torch.float32, device=DEV)
        score = torch.empty(w.hkv, n_cand, dtype=torch.float32, device=DEV)
        sel, count = pca.oomb_select_pages(pool, table, x["q"], t0, w.top_k, qbar_out=qbar,
                                           score_out=score)
    o, lse = pca.oomb_paged_chunk_attn_fwd(pool, table, x["q"], t0, sel, count, w.scale)
    dq = pca.oomb_paged_chunk_attn_bwd(pool, table, gtable, x["q"], t0, sel, count, o, x["do"],
                                       lse, w.scale)
    torch.cuda.synchronize()
    return dict(pool=pool, sel=sel, count=count, qbar=qbar, score=score, o=o, lse=lse, dq=dq)


def _oracle_pool(w, x_cpu, spare=3):
    n = w.pool_pages + spare
    kp = torch.zeros(n, w.page, w.d, dtype=w.dtype)
    vp = torch.zeros(n, w.page, w.d, dtype=w.dtype)
    orc.append(kp, x_cpu["table"], x_cpu["k"], 0)
    orc.append(vp, x_cpu["table"], x_cpu["v"], 0)
    return kp, vp


def _check_selection(w, x_cpu, kp, r):
    summ = torch.zeros(kp.shape[0], 2, w.d, dtype=w.dtype)
    orc.summarize(kp, x_cpu["table"], summ, 0, w.pages_per_head, w.total)
    ref = orc.select_pages(x_cpu["q"], summ, x_cpu["table"], w.t0, w.page, w.group, w.top_k)
    gq, gs = r["qbar"].cpu(), r["score"].cpu()
    gsel, gcnt = r["sel"].cpu(), r["count"].cpu()
    out = []
    for g, (qb, sc, chosen) in enumerate(ref):
        assert torch.equal(bits(gq[g]), torch.from_numpy(qb).view(torch.int32)), f"qbar {g}"
        assert torch.equal(bits(gs[g]), torch.from_numpy(sc).view(torch.int32)), f"scores {g}"
        assert int(gcnt[g]) == len(chosen) and gsel[g, :len(chosen)].tolist() == chosen, f"sel {g}"
        out.append(chosen)
    recall = [len(set(c) & set(x_cpu["needles"].tolist())) for c in out]
    log(f"    selection bit-exact on {w.hkv} heads ({len(out[0])} pages each); "
        f"needle pages recalled per head: {recall}")
    # summaries are bit-identical too (all pages of every head)
    used = x_cpu["table"].reshape(-1).long()
    assert torch.equal(bits(r["pool"].summary.cpu()[used]), bits(summ[used]))
    return out


def _sampled_rows(w, x_cpu, kp, vp, osel, r, rows):
    """O, LSE, dQ of single query rows (all heads of a group), each by an oracle call on
    a one-query chunk whose selection includes the chunk pages before that query."""
    P, t0, G = w.page, w.t0, w.group
    go, glse, gdq = r["o"].cpu(), r["lse"].cpu(), r["dq"].cpu()
    got_o, ref_o, got_q, ref_q, lse_err = [], [], [], [], 0.0
    for (g, i) in rows:
        sel_g = list(range(t0 // P)) if osel is None else list(osel[g])
        sel_i = sorted(set(sel_g) | set(range(t0 // P, (t0 + i) // P)))
        hs = slice(g * G, (g + 1) * G)
        q1 = x_cpu["q"][hs, i:i + 1]
        O, L = orc.fwd(q1, kp, vp, x_cpu["table"][g:g + 1], t0 + i, [sel_i], w.scale)
        dQ, _ = orc.bwd(q1, kp, vp, x_cpu["table"][g:g + 1], t0 + i, [sel_i], w.scale,
                        x_cpu["do"][hs, i:i + 1])
        got_o.append(go[hs, i])
        ref_o.append(O[:, 0])
        got_q.append(gdq[hs, i])
        ref_q.append(dQ[:, 0])
        lse_err = max(lse_err, (glse[hs, i].double() - L[:, 0]).abs().max().item())
    compare("O(rows)", torch.stack(got_o), torch.stack(ref_o), w.dtype)
    compare("dQ(rows)", torch.stack(got_q), torch.stack(ref_q), w.dtype)
    log(f"    LSE(rows) max_abs={lse_err:.3e}")
    assert lse_err <= 1e-2


def _invariants(w, x_cpu, osel, r):
    """Per KV head, over its attended keys: sum dV = sum dO over the group's rows, and
    sum dK ~ 0 relative to ||dK||."""
    P, t0, C, G = w.page, w.t0, w.chunk, w.group
    dk, dv = r["pool"].dk.cpu(), r["pool"].dv.cpu()
    for g in range(w.hkv):
        pages = orc.attended_pages(t0, C, P, None if osel is None else osel[g])
        pos = orc.key_positions(pages, P, t0 + C)
        rows = x_cpu["gtable"][g].long()[pos // P] * P + pos % P
        dKg = dk.reshape(-1, w.d)[rows].double()
        dVg = dv.reshape(-1, w.d)[rows].double()
        sum_do = x_cpu["do"][g * G:(g + 1) * G].double().sum((0, 1))
        ev = ((dVg.sum(0) - sum_do).norm() / sum_do.norm()).item()
        ek = (dKg.sum(0).norm() / dKg.norm()).item()
        log(f"    head {g}: |sum dV - sum dO|/|sum dO| = {ev:.2e}, |sum dK|/||dK|| = {ek:.2e}")
        assert ev < 1e-2 and ek < 2e-2
        assert torch.isfinite(dKg).all() and torch.isfinite(dVg).all()


def _sentinels(w, r, x_cpu, spare=3):
    """Spare pool pages (never mapped) still hold their sentinel bytes."""
    mapped = torch.zeros(w.pool_pages + spare, dtype=torch.bool)
    mapped[x_cpu["table"].reshape(-1).long()] = True
    assert bool((bits(r["pool"].k.cpu()[~mapped]) == SENTINEL[w.dtype]).all())
    assert bool((bits(r["pool"].v.cpu()[~mapped]) == SENTINEL[w.dtype]).all())


def _to_cpu(x):
    return {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in x.items()}


def _row_sample(w, n_per_group=4):
    C = w.chunk
    cand = [0, 1, C // 3, C // 2 + 17, C - 129, C - 1]
    return [(g, cand[(g + j) % len(cand)]) for g in range(w.hkv) for j in range(n_per_group)]


def test_fullsize_sparse1m():
    """1M prior tokens, top-64: selection bit-exact on all heads; KV group 0 checked
    elementwise in full (O, LSE, dQ, dK, dV); invariants on all groups; determinism."""
    w = wl.WORKLOADS["sparse1m"]
    log(f"[case fullsize sparse1m] t0={w.t0} chunk={w.chunk}")
    x = wl.make_inputs(w, device=DEV)
    r = _gpu_step(w, x)
    log("    gpu step done")
    xc = _to_cpu(x)
    kp, vp = _oracle_pool(w, xc)
    osel = _check_selection(w, xc, kp, r)
    _sentinels(w, r, xc)
    # KV group 0 in full
    G = w.group
    O, L = orc.fwd(xc["q"][:G], kp, vp, xc["table"][:1], w.t0, osel[:1], w.scale)
    compare("O(g0)", r["o"][:G], O, w.dtype)
    assert (r["lse"][:G].cpu().double() - L).abs().max().item() <= 1e-2
    gk = torch.zeros(kp.shape, dtype=torch.float64)
    gv = torch.zeros(kp.shape, dtype=torch.float64)
    dQ, _ = orc.bwd(xc["q"][:G], kp, vp, xc["table"][:1], w.t0, osel[:1], w.scale, xc["do"][:G],
                    gk, gv, xc["gtable"][:1])
    compare("dQ(g0)", r["dq"][:G], dQ, w.dtype)
    pages = orc.attended_pages(w.t0, w.chunk, w.page, osel[0])
    pos = orc.key_positions(pages, w.page, w.t0 + w.chunk)
    rows = xc["gtable"][0].long()[pos // w.page] * w.page + pos % w.page
    compare("dK(g0)", r["pool"].dk.cpu().reshape(-1, w.d)[rows], gk.reshape(-1, w.d)[rows], w.dtype)
    compare("dV(g0)", r["pool"].dv.cpu().reshape(-1, w.d)[rows], gv.reshape(-1, w.d)[rows], w.dtype)
    _sampled_rows(w, xc, kp, vp, osel, r, _row_sample(w, 2))
    _invariants(w, xc, osel, r)
    # run-twice determinism of the backward at full size
    first = (r["dq"].clone(), r["pool"].dk.clone(), r["pool"].dv.clone())
    r["pool"].zero_grad()
    dq2 = pca.oomb_paged_chunk_attn_bwd(r["pool"], x["table"].to(DEV), x["gtable"].to(DEV),
                                        x["q"], w.t0, r["sel"], r["count"], r["o"], x["do"],
                                        r["lse"], w.scale)
    torch.cuda.synchronize()
    assert torch.equal(dq2, first[0])
    r["pool"].dk.zero_()
    r["pool"].dv.zero_()
    # (pool was re-zeroed above: rerun once more into zeros and compare with a fresh zero run)
    pca.oomb_paged_chunk_attn_bwd(r["pool"], x["table"].to(DEV), x["gtable"].to(DEV), x["q"],
                                  w.t0, r["sel"], r["count"], r["o"], x["do"], r["lse"], w.scale)
    dk_a, dv_a = r["pool"].dk.clone(), r["pool"].dv.clone()
    r["pool"].zero_grad()
    pca.oomb_paged_chunk_attn_bwd(r["pool"], x["table"].to(DEV), x["gtable"].to(DEV), x["q"],
                                  w.t0, r["sel"], r["count"], r["o"], x["do"], r["lse"], w.scale)
    torch.cuda.synchronize()
    assert torch.equal(dk_a, r["pool"].dk) and torch.equal(dv_a, r["pool"].dv)


def test_fullsize_sparse4m():
    """4M-token context, top-128, chunk 8192: selection bit-exact on all heads, sampled
    rows, invariants, sentinels."""
    w = wl.WORKLOADS["sparse4m"]
    log(f"[case fullsize sparse4m] t0={w.t0} chunk={w.chunk}")
    x = wl.make_inputs(w, device=DEV)
    r = _gpu_step(w, x)
    log("    gpu step done")
    xc = _to_cpu(x)
    del x
    kp, vp = _oracle_pool(w, xc)
    osel = _check_selection(w, xc, kp, r)
    _sentinels(w, r, xc)
    _sampled_rows(w, xc, kp, vp, osel, r, _row_sample(w, 2))
    _invariants(w, xc, osel, r)


def test_fullsize_dense128k():
    """128K context, all 992 prior pages: sampled rows and invariants."""
    w = wl.WORKLOADS["dense128k"]
    log(f"[case fullsize dense128k] t0={w.t0} chunk={w.chunk}")
    x = wl.make_inputs(w, device=DEV)
    r = _gpu_step(w, x)
    log("    gpu step done")
    xc = _to_cpu(x)
    kp, vp = _oracle_pool(w, xc)
    _sentinels(w, r, xc)
    _sampled_rows(w, xc, kp, vp, None, r, _row_sample(w, 3))
    _invariants(w, xc, None, r)


def _gpu_sweep(w, x):
    """Chunk-recurrent sweep through the library: forward c = 0..S-1 (append, summarize,
    select, fwd), then c = S-1..0 (fwd again, bwd)."""
    P, C = w.page, w.chunk
    pool = pca.PagedPool(w.pool_pages, P, w.d, w.hq, w.hkv, w.dtype, DEV)
    table, gtable = x["table"].to(DEV), x["gtable"].to(DEV)
    q_all, do_all = x["q"].to(DEV), x["do"].to(DEV)
    k_all, v_all = x["k"].to(DEV), x["v"].to(DEV)
    sels, outs = [], []
    for c in range(w.n_chunks):
        t0 = c * C
        pca.oomb_kv_append(pool, table, k_all[:, t0:t0 + C].contiguous(),
                           v_all[:, t0:t0 + C].contiguous(), t0)
        pca.oomb_page_summarize(pool, table, t0 // P, (t0 + C - 1) // P - t0 // P + 1, t0 + C)
        q = q_all[:, t0:t0 + C].contiguous()
        sc = (None, None)
        if w.top_k is not None:
            sc = pca.oomb_select_pages(pool, table, q, t0, w.top_k)
        sels.append(sc)
        outs.append(pca.oomb_paged_chunk_attn_fwd(pool, table, q, t0, sc[0], sc[1], w.scale)[0])
    dq = torch.zeros(w.hq, w.total, w.d, dtype=torch.float32, device=DEV)
    for c in reversed(range(w.n_chunks)):
        t0 = c * C
        q = q_all[:, t0:t0 + C].contiguous()
        s_, c_ = sels[c]
        o, lse = pca.oomb_paged_chunk_attn_fwd(pool, table, q, t0, s_, c_, w.scale)
        dq[:, t0:t0 + C] = pca.oomb_paged_chunk_attn_bwd(
            pool, table, gtable, q, t0, s_, c_, o, do_all[:, t0:t0 + C].contiguous(), lse, w.scale)
    torch.cuda.synchronize()
    return pool, torch.cat(outs, dim=1), dq, sels


@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),                                                          # the tiny workload itself
    ("sweep256k", dict(hq=28, hkv=4, chunk=512, total=4096)),              # sweep shape, reduced
    ("sweep256k_top64", dict(hq=28, hkv=4, chunk=512, total=4096, top_k=2)),
])
def test_sweep_parity(name, kw):
    """The GPU chunk-recurrent sweep equals the oracle's sweep: O of every chunk, dQ of
    the whole sequence, the gradient pools accumulated over all chunks, selections."""
    w = wl.custom(name, name=name + "_sweep", **kw) if kw else wl.WORKLOADS[name]
    log(f"[case sweep {w.name}] chunks={w.n_chunks} chunk={w.chunk} dtype={w.dtype} top_k={w.top_k}")
    x = wl.make_inputs(w)
    pool, O, dq, sels = _gpu_sweep(w, x)
    log("    gpu sweep done")
    ref = orc.sweep(x["q"], x["k"], x["v"], x["do"], x["table"], x["gtable"], w.pool_pages,
                    w.page, w.chunk, w.scale, top_k=w.top_k)
    if w.top_k is not None:
        for c, (s_, c_) in enumerate(sels):
            for g in range(w.hkv):
                n = int(c_[g])
                assert s_[g, :n].cpu().tolist() == ref["sels"][c][g], (c, g)
    compare("O", O, ref["O"], w.dtype)
    compare("dQ", dq, ref["dQ"], w.dtype)
    mapped = x["gtable"].reshape(-1).long()
    compare("dK", pool.dk.cpu()[mapped], ref["dk_pool"][mapped], w.dtype)
    compare("dV", pool.dv.cpu()[mapped], ref["dv_pool"][mapped], w.dtype)
