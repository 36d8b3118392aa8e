"""GPU parity at full workload sizes, in the launch configuration bench.py times,
and the chunk-recurrent sweep at its full shape (32 chunks of 8192, 28/4 heads).

Single chunks (1M, 4M, 128K): page selection bit for bit on every KV head; KV group 0
(7 query heads) in full against the oracle: O, LSE and dQ on every row, dK and dV on
every attended key; sampled rows of the other groups; and on every group the
identities that hold at any size:
  sum_t dV_t = sum_{h in group, i} dO_hi      (rows of P sum to one)
  sum_t dK_t = 0                              (sum_t dS_it = dO_i.O_i - Delta_i = 0)

Sweeps (the oracle cannot redo a whole 262,144-token sweep in the suite's time, so
the sample is bounded, never skipped):
  top-64: selections bit for bit for every chunk and KV head; KV group 0 in full
    over all 32 chunks (O, LSE, dQ of every row; dK/dV of every key after the whole
    reverse pass); sampled rows of the other groups in every chunk; the identities
    over the whole gradient pool.
  dense: the last 256 queries of KV group 0 in full, and dK/dV of the 256 keys that
    only those queries attend; sampled rows across the sequence; the identities.
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


def _sampled_rows(w, x_cpu, kp, vp, rows, go, glse, gdq, t0=None, sels=None, q_off=0):
    """O, LSE, dQ of single query rows (all heads of a group), each by an oracle call on
    a one-query chunk at that query's position, whose selection is the chunk's
    selection plus the chunk pages before the query (so it attends exactly the keys the
    query attends in the chunk).

    rows: (g, i) pairs, i the query's index in the chunk that starts at t0 (default
    w.t0); sels: per-group selected prior pages of that chunk (None = dense). go, glse,
    gdq: the GPU's outputs on CPU, indexed [head, q_off + i]."""
    P, G = w.page, w.group
    t0 = w.t0 if t0 is None else t0
    got_o, ref_o, got_q, ref_q, lse_err = [], [], [], [], 0.0
    for (g, i) in rows:
        sel_g = list(range(t0 // P)) if sels is None else list(sels[g])
        sel_i = sorted(set(sel_g) | set(range(t0 // P, (t0 + i) // P)))
        hs = slice(g * G, (g + 1) * G)
        q1 = x_cpu["q"][hs, q_off + i:q_off + i + 1]
        d1 = x_cpu["do"][hs, q_off + i:q_off + i + 1]
        dQ, _, O, L = orc.bwd(q1, kp, vp, x_cpu["table"][g:g + 1], t0 + i, [sel_i], w.scale, d1,
                              with_fwd=True)
        got_o.append(go[hs, q_off + i])
        ref_o.append(O[:, 0])
        got_q.append(gdq[hs, q_off + i])
        ref_q.append(dQ[:, 0])
        lse_err = max(lse_err, (glse[hs, q_off + i].double() - L[:, 0]).abs().max().item())
    compare("O(rows)", torch.stack(got_o), torch.stack(ref_o), w.dtype)
    compare("dQ(rows)", torch.stack(got_q), torch.stack(ref_q), w.dtype)
    log(f"    LSE(rows) max_abs={lse_err:.3e} over {len(rows)} rows")
    assert lse_err <= 1e-2


def _grad_rows(w, gtable_cpu, g, pos):
    """Flat row indices of the gradient pool for KV head g's key positions."""
    P = w.page
    return gtable_cpu[g].long()[pos // P] * P + pos % P


def _group_in_full(w, x_cpu, kp, vp, osel, r, g=0):
    """KV group g against the oracle in full: O, LSE, dQ on every row of its query heads,
    dK and dV on every key it attends (the pool was zero before this one backward)."""
    G, P, t0, C = w.group, w.page, w.t0, w.chunk
    hs = slice(g * G, (g + 1) * G)
    gk = torch.zeros(kp.shape, dtype=torch.float64)
    gv = torch.zeros(kp.shape, dtype=torch.float64)
    sel_g = None if osel is None else [osel[g]]
    log(f"    oracle: KV group {g} in full ...")
    dQ, _, O, L = orc.bwd(x_cpu["q"][hs], kp, vp, x_cpu["table"][g:g + 1], t0, sel_g, w.scale,
                          x_cpu["do"][hs], gk, gv, x_cpu["gtable"][g:g + 1], with_fwd=True)
    compare(f"O(g{g})", r["o"][hs], O, w.dtype)
    lse_err = (r["lse"][hs].cpu().double() - L).abs().max().item()
    log(f"    LSE(g{g}) max_abs={lse_err:.3e}")
    assert lse_err <= 1e-2
    compare(f"dQ(g{g})", r["dq"][hs], dQ, w.dtype)
    pages = orc.attended_pages(t0, C, P, None if osel is None else osel[g])
    pos = orc.key_positions(pages, P, t0 + C)
    rows = _grad_rows(w, x_cpu["gtable"], g, pos)
    compare(f"dK(g{g})", r["pool"].dk.cpu().reshape(-1, w.d)[rows], gk.reshape(-1, w.d)[rows],
            w.dtype)
    compare(f"dV(g{g})", r["pool"].dv.cpu().reshape(-1, w.d)[rows], gv.reshape(-1, w.d)[rows],
            w.dtype)


def _invariant_check(w, g, dKg, dVg, sum_do):
    ev = ((dVg.sum(0) - sum_do).norm() / sum_do.norm()).item()
    ek = (dKg.sum(0).norm() / dKg.norm()).item()
    log(f"    head {g}: |sum dV - sum dO|/|sum dO| = {ev:.2e}, |sum dK|/||dK|| = {ek:.2e}")
    assert ev < 1e-2 and ek < 2e-2
    assert torch.isfinite(dKg).all() and torch.isfinite(dVg).all()


def _invariants(w, x_cpu, osel, r):
    """Per KV head, over its attended keys: sum dV = sum dO over the group's rows, and
    sum dK ~ 0 relative to ||dK||."""
    P, t0, C, G = w.page, w.t0, w.chunk, w.group
    dk, dv = r["pool"].dk.cpu(), r["pool"].dv.cpu()
    for g in range(w.hkv):
        pages = orc.attended_pages(t0, C, P, None if osel is None else osel[g])
        pos = orc.key_positions(pages, P, t0 + C)
        rows = _grad_rows(w, x_cpu["gtable"], g, pos)
        _invariant_check(w, g, dk.reshape(-1, w.d)[rows].double(),
                         dv.reshape(-1, w.d)[rows].double(),
                         x_cpu["do"][g * G:(g + 1) * G].double().sum((0, 1)))


def _sentinels(w, r, x_cpu, spare=3):
    """Spare pool pages (never mapped) still hold their sentinel bytes."""
    mapped = torch.zeros(w.pool_pages + spare, dtype=torch.bool)
    mapped[x_cpu["table"].reshape(-1).long()] = True
    assert bool((bits(r["pool"].k.cpu()[~mapped]) == SENTINEL[w.dtype]).all())
    assert bool((bits(r["pool"].v.cpu()[~mapped]) == SENTINEL[w.dtype]).all())


def _to_cpu(x):
    return {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in x.items()}


def _row_sample(w, n_per_group=4, groups=None, C=None):
    C = w.chunk if C is None else C
    cand = [0, 1, C // 3, C // 2 + 17, C - 129, C - 1]
    groups = range(w.hkv) if groups is None else groups
    return [(g, cand[(g + j) % len(cand)]) for g in groups for j in range(n_per_group)]


def _single_chunk(name, check_determinism=False):
    w = wl.WORKLOADS[name]
    log(f"[case fullsize {name}] t0={w.t0} chunk={w.chunk} top_k={w.top_k}")
    x = wl.make_inputs(w, device=DEV)
    r = _gpu_step(w, x)
    log("    gpu step done")
    xc = _to_cpu(x)
    kp, vp = _oracle_pool(w, xc)
    osel = _check_selection(w, xc, kp, r) if w.top_k is not None else None
    _sentinels(w, r, xc)
    _group_in_full(w, xc, kp, vp, osel, r, g=0)
    _sampled_rows(w, xc, kp, vp, _row_sample(w, 2, groups=range(1, w.hkv)), r["o"].cpu(),
                  r["lse"].cpu(), r["dq"].cpu(), sels=osel)
    _invariants(w, xc, osel, r)
    return w, x, r


def test_fullsize_sparse1m():
    """1M prior tokens, top-64: selection bit-exact on all heads; KV group 0 in full;
    sampled rows of the other groups; invariants; run-twice determinism."""
    w, x, r = _single_chunk("sparse1m")
    # run-twice determinism of the backward at full size (the pool re-zeroed each time)
    table, gtable = x["table"].to(DEV), x["gtable"].to(DEV)
    res = []
    for _ in range(2):
        r["pool"].zero_grad()
        dq = pca.oomb_paged_chunk_attn_bwd(r["pool"], table, gtable, x["q"], w.t0, r["sel"],
                                           r["count"], r["o"], x["do"], r["lse"], w.scale)
        torch.cuda.synchronize()
        res.append((dq.clone(), r["pool"].dk.clone(), r["pool"].dv.clone()))
    for a, b in zip(*res):
        assert torch.equal(a, b)
    assert torch.equal(res[0][0], r["dq"])


def test_fullsize_sparse4m():
    """4M-token context, top-128, chunk 8192: selection bit-exact on all heads; KV group
    0 in full; sampled rows of the other groups; invariants; sentinels."""
    _single_chunk("sparse4m")


def test_fullsize_dense128k():
    """128K context, all 992 prior pages: KV group 0 in full; sampled rows of the other
    groups; invariants; sentinels."""
    _single_chunk("dense128k")


def _gpu_sweep(w, x):
    """Chunk-recurrent sweep through the library: forward c = 0..S-1 (append, summarize,
    select, fwd), then c = S-1..0 (fwd again, bwd). Returns the pool, O and LSE of the
    forward pass, dQ of the reverse pass (all chunks) and the selections."""
    P, C = w.page, w.chunk
    pool = pca.PagedPool(w.pool_pages, P, w.d, w.hq, w.hkv, w.dtype, DEV)
    table, gtable = x["table"].to(DEV), x["gtable"].to(DEV)
    q_all, do_all = x["q"].to(DEV), x["do"].to(DEV)
    k_all, v_all = x["k"].to(DEV), x["v"].to(DEV)
    sels, outs, lses = [], [], []
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
        o, lse = pca.oomb_paged_chunk_attn_fwd(pool, table, q, t0, sc[0], sc[1], w.scale)
        outs.append(o)
        lses.append(lse)
    dq = torch.zeros(w.hq, w.total, w.d, dtype=torch.float32, device=DEV)
    for c in reversed(range(w.n_chunks)):
        t0 = c * C
        q = q_all[:, t0:t0 + C].contiguous()
        s_, c_ = sels[c]
        o, lse = pca.oomb_paged_chunk_attn_fwd(pool, table, q, t0, s_, c_, w.scale)
        dq[:, t0:t0 + C] = pca.oomb_paged_chunk_attn_bwd(
            pool, table, gtable, q, t0, s_, c_, o, do_all[:, t0:t0 + C].contiguous(), lse, w.scale)
    torch.cuda.synchronize()
    return pool, torch.cat(outs, dim=1), torch.cat(lses, dim=1), dq, sels


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
    pool, O, _, dq, sels = _gpu_sweep(w, x)
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


def _sweep_invariants(w, x, pool):
    """Over the whole sweep, per KV head: sum of dV over all its keys = sum of dO over
    all its query rows of every chunk; sum of dK ~ 0."""
    G, P = w.group, w.page
    dk, dv = pool.dk.cpu().reshape(-1, w.d), pool.dv.cpu().reshape(-1, w.d)
    pos = torch.arange(w.total)
    for g in range(w.hkv):
        rows = _grad_rows(w, x["gtable"], g, pos)
        _invariant_check(w, g, dk[rows].double(), dv[rows].double(),
                         x["do"][g * G:(g + 1) * G].double().sum((0, 1)))


def _sweep_sampled_rows(w, x, kp, vp, chunks, sels, O, L, dq, n_per_group=1):
    """Sampled rows of the listed chunks, every group (sels[c]: the oracle's selections
    of chunk c per group, or None for dense)."""
    C = w.chunk
    go, glse, gdq = O.cpu(), L.cpu(), dq.cpu()
    for c in chunks:
        rows = [(g, i) for (g, i) in _row_sample(w, n_per_group)]
        rows = [(g, (i + 97 * c) % C) for (g, i) in rows]
        log(f"    chunk {c}:")
        _sampled_rows(w, x, kp, vp, rows, go, glse, gdq, t0=c * C,
                      sels=None if sels is None else sels[c], q_off=c * C)


_TOP64_PARTS = 4  # the oracle's reverse pass over KV group 0, a quarter of the chunks each


@pytest.fixture(scope="module")
def top64():
    """The 262,144-token top-64 sweep at full shape (28/4 heads, 32 chunks of 8192), run
    once on the GPU; the oracle's reverse pass over KV group 0 is added chunk by chunk
    by the tests below, in their file order, so that no single test runs for minutes."""
    w = wl.WORKLOADS["sweep256k_top64"]
    log(f"[case fullsize sweep {w.name}] chunks={w.n_chunks} chunk={w.chunk} top_k={w.top_k}")
    x = wl.make_inputs(w)
    pool, O, L, dq, gsels = _gpu_sweep(w, x)
    log("    gpu sweep done")
    kp, vp = _oracle_pool(w, x, spare=0)
    return dict(w=w, x=x, pool=pool, O=O, L=L, dq=dq, gsels=gsels, kp=kp, vp=vp, osels=None,
                gk=torch.zeros(kp.shape, dtype=torch.float64),
                gv=torch.zeros(kp.shape, dtype=torch.float64), parts_done=0)


def test_fullsize_sweep_top64_selections(top64):
    """Selections bit for bit for every chunk and KV head of the top-64 sweep."""
    w, x, gsels = top64["w"], top64["x"], top64["gsels"]
    C, P, G = w.chunk, w.page, w.group
    summ = torch.zeros(top64["kp"].shape[0], 2, w.d, dtype=w.dtype)
    # every page is complete by the time it is a candidate, so one summary of the
    # whole context gives the scores each chunk saw
    orc.summarize(top64["kp"], x["table"], summ, 0, w.pages_per_head, w.total)
    osels = []
    for c in range(w.n_chunks):
        t0 = c * C
        ref = orc.select_pages(x["q"][:, t0:t0 + C], summ, x["table"], t0, P, G, w.top_k)
        s_, c_ = gsels[c]
        s_, c_ = s_.cpu(), c_.cpu()
        for g, (_, _, chosen) in enumerate(ref):
            assert int(c_[g]) == len(chosen) and s_[g, :len(chosen)].tolist() == chosen, (c, g)
        osels.append([chosen for (_, _, chosen) in ref])
    top64["osels"] = osels
    log(f"    selections bit-exact: {w.n_chunks} chunks x {w.hkv} KV heads")


@pytest.mark.parametrize("part", range(_TOP64_PARTS))
def test_fullsize_sweep_top64_chunks(top64, part):
    """A quarter of the top-64 sweep's chunks, in the reverse pass's order (part 0 holds
    the last chunks): KV group 0 in full (O, LSE and dQ of every row, the oracle's dK/dV
    accumulated for the final check), sampled rows of the other groups."""
    if top64["osels"] is None or top64["parts_done"] != part:
        pytest.skip("needs the selections and the earlier parts of the same session")
    w, x, osels = top64["w"], top64["x"], top64["osels"]
    C, G = w.chunk, w.group
    hs = slice(0, G)
    per = w.n_chunks // _TOP64_PARTS
    chunks = list(reversed(range(w.n_chunks)))[part * per:(part + 1) * per]
    go, glse, gdq = top64["O"].cpu(), top64["L"].cpu(), top64["dq"].cpu()
    for c in chunks:
        t0 = c * C
        sl = slice(t0, t0 + C)
        dq_ref, _, o_ref, l_ref = orc.bwd(
            x["q"][hs, sl], top64["kp"], top64["vp"], x["table"][:1], t0, [osels[c][0]],
            w.scale, x["do"][hs, sl], top64["gk"], top64["gv"], x["gtable"][:1], with_fwd=True)
        compare(f"O(g0, chunk {c})", go[hs, sl], o_ref, w.dtype)
        lse_err = (glse[hs, sl].double() - l_ref).abs().max().item()
        assert lse_err <= 1e-2, (c, lse_err)
        compare(f"dQ(g0, chunk {c})", gdq[hs, sl], dq_ref, w.dtype)
        rows_c = [(g, (i + 97 * c) % C) for (g, i) in _row_sample(w, 1, groups=range(1, w.hkv))]
        _sampled_rows(w, x, top64["kp"], top64["vp"], rows_c, go, glse, gdq, t0=t0,
                      sels=osels[c], q_off=t0)
    top64["parts_done"] = part + 1
    log(f"    chunks {chunks[0]}..{chunks[-1]} done")


def test_fullsize_sweep_top64_grads(top64):
    """dK/dV of every key of KV group 0 after the whole reverse pass, and the identities
    over the whole gradient pool."""
    if top64["parts_done"] != _TOP64_PARTS:
        pytest.skip("needs every chunk part of the same session")
    w, x, pool = top64["w"], top64["x"], top64["pool"]
    rows = _grad_rows(w, x["gtable"], 0, torch.arange(w.total))
    compare("dK(g0)", pool.dk.cpu().reshape(-1, w.d)[rows], top64["gk"].reshape(-1, w.d)[rows],
            w.dtype)
    compare("dV(g0)", pool.dv.cpu().reshape(-1, w.d)[rows], top64["gv"].reshape(-1, w.d)[rows],
            w.dtype)
    _sweep_invariants(w, x, pool)


def test_fullsize_sweep_dense():
    """The 262,144-token dense sweep at full shape: the last 256 queries of KV group 0
    in full (O, LSE, dQ) and dK/dV of the 256 keys only they attend; sampled rows of
    chunks across the sequence; the identities over the whole gradient pool."""
    w = wl.WORKLOADS["sweep256k"]
    C, G, T = w.chunk, w.group, w.total
    log(f"[case fullsize sweep {w.name}] chunks={w.n_chunks} chunk={C}")
    x = wl.make_inputs(w)
    pool, O, L, dq, _ = _gpu_sweep(w, x)
    log("    gpu sweep done")
    kp, vp = _oracle_pool(w, x, spare=0)
    n_tail = 256
    t0 = T - n_tail
    hs = slice(0, G)
    gk = torch.zeros(kp.shape, dtype=torch.float64)
    gv = torch.zeros(kp.shape, dtype=torch.float64)
    log(f"    oracle: last {n_tail} queries of KV group 0 over all {T} keys ...")
    dQ, _, Ot, Lt = orc.bwd(x["q"][hs, t0:], kp, vp, x["table"][:1], t0, None, w.scale,
                            x["do"][hs, t0:], gk, gv, x["gtable"][:1], with_fwd=True)
    compare("O(tail)", O[hs, t0:], Ot, w.dtype)
    lse_err = (L[hs, t0:].cpu().double() - Lt).abs().max().item()
    log(f"    LSE(tail) max_abs={lse_err:.3e}")
    assert lse_err <= 1e-2
    compare("dQ(tail)", dq[hs, t0:], dQ, w.dtype)
    rows = _grad_rows(w, x["gtable"], 0, torch.arange(t0, T))
    compare("dK(tail)", pool.dk.cpu().reshape(-1, w.d)[rows], gk.reshape(-1, w.d)[rows], w.dtype)
    compare("dV(tail)", pool.dv.cpu().reshape(-1, w.d)[rows], gv.reshape(-1, w.d)[rows], w.dtype)
    n = w.n_chunks
    _sweep_sampled_rows(w, x, kp, vp, sorted({0, 1, n // 2 - 3, n - 2}), None, O, L, dq)
    _sweep_invariants(w, x, pool)
