"""GPU tests of the page movement between the device pools and pinned host memory
(the CPU offload of the KV cache and its gradients, gist.science explainer of OOMB,
2.C), through the C-ABI binding, against the oracle's page moves (bit-exact: the
moves are copies and one fp32 addition per element), and a whole offload cycle:
prior pages offloaded to the host and wiped on the device, the selected ones fetched
back into staging pages, then attention forward and backward over them, against the
oracle's attention over the resident cache.
"""
import pytest
import torch

import oracle as orc
import paged_chunk_attention_amd as pca
import workloads as wl
from tests.gpu_harness import DEV, SENTINEL, bits, compare, fill_sentinel, log, GpuLayer, oracle_layer

pytestmark = pytest.mark.gpu


def _pinned(shape, dtype):
    return torch.empty(shape, dtype=dtype, pin_memory=True)


def _rand(shape, seed, dtype):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g).to(dtype)


def _ids(x):
    return torch.tensor(x, dtype=torch.int32, device=DEV)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_copy_pages_device_host_round_trip(dtype):
    """Device -> pinned host -> device, with ids outside either array skipped, a
    device-side list length, and every page not named left bit-unchanged."""
    log(f"[case copy_pages {dtype}]")
    dev_cpu = _rand((64, 16, 128), 1, dtype)
    dev = dev_cpu.to(DEV)
    host = _pinned((80, 16, 128), dtype)
    fill_sentinel(host)
    want = host.clone()
    src, dst = [5, 63, 0, 17, -1, 64, 9], [79, 0, 40, 3, 5, 6, 80]
    pca.oomb_copy_pages(dev, host, _ids(src), _ids(dst))
    torch.cuda.synchronize()
    orc.copy_pages(dev_cpu, want, src, dst)
    assert torch.equal(bits(host), bits(want)), "device -> host pages differ"

    back = torch.zeros(64, 16, 128, dtype=dtype, device=DEV)
    want_back = torch.zeros(64, 16, 128, dtype=dtype)
    pca.oomb_copy_pages(host, back, _ids(dst), _ids(src))
    orc.copy_pages(want, want_back, dst, src)
    torch.cuda.synchronize()
    assert torch.equal(bits(back), bits(want_back)), "host -> device pages differ"
    assert torch.equal(bits(back[[5, 63, 0, 17]]), bits(dev_cpu[[5, 63, 0, 17]]))

    # the list length read on the device
    again = torch.zeros_like(back)
    pca.oomb_copy_pages(host, again, _ids(dst), _ids(src), n_dev=_ids([2]))
    torch.cuda.synchronize()
    want_again = torch.zeros(64, 16, 128, dtype=dtype)
    orc.copy_pages(want, want_again, dst, src, n=2)
    assert torch.equal(bits(again), bits(want_again))


def test_copy_pages_sdma_runs_and_skips():
    """The copy-engine path: host id lists with runs (coalesced into one transfer each),
    single pages and invalid ids, both directions, bitwise as the oracle."""
    log("[case copy_pages_sdma]")
    dev_cpu = _rand((64, 16, 128), 4, torch.bfloat16)
    dev = dev_cpu.to(DEV)
    host = _pinned((80, 16, 128), torch.bfloat16)
    fill_sentinel(host)
    want = host.clone()
    src = [10, 11, 12, 13, 40, 41, 7, -1, 5, 63, 70]
    dst = [20, 21, 22, 23, 50, 60, 0, 3, 79, 78, 1]
    pca.oomb_copy_pages_sdma(dev, host, src, dst)
    torch.cuda.synchronize()
    orc.copy_pages(dev_cpu, want, src, dst)
    assert torch.equal(bits(host), bits(want)), "device -> host (copy engine) differs"
    back = torch.zeros(64, 16, 128, dtype=torch.bfloat16, device=DEV)
    want_back = torch.zeros(64, 16, 128, dtype=torch.bfloat16)
    pca.oomb_copy_pages_sdma(host, back, dst, src)
    orc.copy_pages(want, want_back, dst, src)
    torch.cuda.synchronize()
    assert torch.equal(bits(back), bits(want_back)), "host -> device (copy engine) differs"


def test_add_pages_into_pinned_host():
    """Gradient pages added into a pinned fp32 pool (one rounding per element, as the
    oracle), the source pages cleared afterwards; pages not named unchanged."""
    log("[case add_pages_f32]")
    src_cpu = _rand((20, 16, 128), 2, torch.float32)
    src = src_cpu.to(DEV)
    host = _pinned((30, 16, 128), torch.float32)
    host.copy_(_rand((30, 16, 128), 3, torch.float32))
    want = host.clone()
    s_ids, d_ids = [0, 7, 19, 3, 25], [29, 0, 11, 12, -1]
    pca.oomb_add_pages_f32(src, host, _ids(s_ids), _ids(d_ids), zero_src=True)
    torch.cuda.synchronize()
    want_src = src_cpu.clone()
    orc.add_pages(want_src, want, s_ids, d_ids, zero_src=True)
    assert torch.equal(bits(host), bits(want)), "added pages differ"
    assert torch.equal(bits(src), bits(want_src)), "source pages not cleared as the oracle"


def test_pageable_memory_rejected():
    """Pageable host memory never reaches a kernel: the binding refuses it, and so does
    the library for a raw pointer."""
    dev = torch.zeros(4, 16, 128, device=DEV)
    pageable = torch.zeros(4, 16, 128)
    with pytest.raises(ValueError):
        pca.oomb_copy_pages(dev, pageable, _ids([0]), _ids([0]))
    import ctypes
    from paged_chunk_attention_amd import _lib as L
    lib = L.lib()
    ids = _ids([0])
    st = lib.oomb_copy_pages(ctypes.c_void_p(dev.data_ptr()), ctypes.c_void_p(pageable.data_ptr()),
                             16 * 128 * 4, 4, 4, ctypes.c_void_p(ids.data_ptr()),
                             ctypes.c_void_p(ids.data_ptr()), 1, None, None)
    assert st == L.OOMB_ERR_INVALID
    assert b"pinned" in lib.oomb_last_error()


@pytest.mark.parametrize("kw", [
    dict(name="offload_sparse_k5", chunk=333, total=2597 + 333, top_k=5, needles=3),
    dict(name="offload_gqa7_k3", hq=28, hkv=4, chunk=256, total=1024 + 256, top_k=3),
])
def test_offload_cycle_then_attention(kw):
    """Prior pages offloaded to pinned host memory and wiped on the device (NaN
    sentinels), the selected ones fetched back into staging pages with the table
    repointed on the device, then forward and backward over them: the same results as
    attention over the resident cache (the oracle), and only selected entries of the
    table changed."""
    base = dict(hq=8, hkv=2, d=128, page=128, dtype=torch.bfloat16)
    base.update(kw)
    w = wl.Workload(**base)
    x = wl.make_inputs(w)
    t0, C, P = w.t0, w.chunk, w.page
    n_cand = t0 // P
    k = min(w.top_k, n_cand)
    log(f"[case {w.name}] hq={w.hq} hkv={w.hkv} chunk={C} t0={t0} top_k={w.top_k}")
    L = GpuLayer(w, x, spare_pages=3 + w.hkv * k)
    L.append(x["k"][:, :t0 + C], x["v"][:, :t0 + C], 0)
    n_pages = -(-(t0 + C) // P)
    pca.oomb_page_summarize(L.pool, L.table, 0, n_pages, t0 + C)
    q, do = x["q"].to(DEV), x["do"].to(DEV)
    sel, count = pca.oomb_select_pages(L.pool, L.table, q, t0, w.top_k)

    # offload every prior page of every head to the host, then wipe the device copies
    host_k = _pinned((w.hkv * n_cand, P, w.d), w.dtype)
    host_v = _pinned((w.hkv * n_cand, P, w.d), w.dtype)
    host_table = torch.arange(w.hkv * n_cand, dtype=torch.int32, device=DEV).reshape(w.hkv, n_cand)
    prior_phys = L.table[:, :n_cand].contiguous().flatten()
    pca.oomb_copy_pages(L.pool.k, host_k, prior_phys, host_table.flatten())
    pca.oomb_copy_pages(L.pool.v, host_v, prior_phys, host_table.flatten())
    torch.cuda.synchronize()
    pp = prior_phys.long().cpu()
    iv = torch.int16
    L.pool.k.view(iv)[pp.to(DEV)] = SENTINEL[w.dtype]
    L.pool.v.view(iv)[pp.to(DEV)] = SENTINEL[w.dtype]

    # fetch the selection into staging pages past the pool's own
    stage = (w.pool_pages + 3 + torch.arange(w.hkv * k, dtype=torch.int32, device=DEV)).reshape(w.hkv, k)
    table = L.table.clone()
    pca.oomb_fetch_selected(L.pool, table, host_k, host_v, host_table, sel, count, stage,
                            n_logical=n_cand)
    o, lse = pca.oomb_paged_chunk_attn_fwd(L.pool, table, q, t0, sel, count, w.scale)
    dq = pca.oomb_paged_chunk_attn_bwd(L.pool, table, L.gtable, q, t0, sel, count, o, do, lse,
                                       w.scale)
    torch.cuda.synchronize()
    log("    gpu done")

    # only the selected entries of the table moved, onto their staging pages
    t_before, t_after = L.table.cpu(), table.cpu()
    osel = [sel[g, :int(count[g])].tolist() for g in range(w.hkv)]
    for g in range(w.hkv):
        for j, lp in enumerate(osel[g]):
            assert int(t_after[g, lp]) == int(stage[g, j]), (g, lp)
        moved = torch.zeros(t_before.shape[1], dtype=torch.bool)
        moved[osel[g]] = True
        assert torch.equal(t_after[g, ~moved], t_before[g, ~moved])

    kp, vp, _ = oracle_layer(w, x, t0 + C)
    O, LSE = orc.fwd(x["q"], kp, vp, x["table"], t0, osel, w.scale)
    compare("O", o, O, w.dtype)
    gpk = torch.zeros(kp.shape, dtype=torch.float64)
    gpv = torch.zeros(kp.shape, dtype=torch.float64)
    dQ, _ = orc.bwd(x["q"], kp, vp, x["table"], t0, osel, w.scale, x["do"], gpk, gpv, x["gtable"])
    compare("dQ", dq, dQ, w.dtype)
    touched = torch.zeros(kp.shape[0], P, dtype=torch.bool)
    for g in range(w.hkv):
        pos = orc.key_positions(orc.attended_pages(t0, C, P, osel[g]), P, t0 + C)
        touched[x["gtable"][g].long()[pos // P], pos % P] = True
    n = kp.shape[0]
    gdk = L.pool.dk.cpu()[:n].double() - L.grad_init[:n].double()
    gdv = L.pool.dv.cpu()[:n].double() - (L.grad_init[:n] * 0.5).double()
    compare("dK", gdk[touched], gpk[touched], w.dtype)
    compare("dV", gdv[touched], gpv[touched], w.dtype)


@pytest.mark.parametrize("top_k,grads_on_host", [(None, True), (3, True), (None, False)])
def test_offloaded_stack_matches_resident_and_oracle(top_k, grads_on_host):
    """Three attention layers with their caches in pinned host memory, one chunk step
    (forward through the layers, backward in reverse) with the transfers on a copy
    stream: O, LSE, dQ, the selections, every host gradient page and the chunk's pages
    written back to the host cache equal the all-resident run bit for bit; and each
    layer matches the oracle (selection bit-exact, attention at the bf16 bar)."""
    from paged_chunk_attention_amd.offload import OffloadedAttentionStack
    L, hq, hkv, d, P, prior, C = 3, 8, 2, 128, 64, 64 * 12, 192
    G = hq // hkv
    log(f"[case offloaded stack top_k={top_k} grads_on_host={grads_on_host}] layers={L} "
        f"prior={prior} chunk={C}")
    stk = OffloadedAttentionStack(L, hq, hkv, d, P, prior, C, top_k=top_k, device=DEV,
                                  grads_on_host=grads_on_host)
    gen = lambda shape, seed: _rand(shape, seed, torch.bfloat16)      # noqa: E731
    kp_in = [gen((hkv, prior, d), 100 + l) for l in range(L)]
    vp_in = [gen((hkv, prior, d), 200 + l) for l in range(L)]
    q = [gen((hq, C, d), 300 + l) for l in range(L)]
    kn = [gen((hkv, C, d), 400 + l) for l in range(L)]
    vn = [gen((hkv, C, d), 500 + l) for l in range(L)]
    do = [gen((hq, C, d), 600 + l) for l in range(L)]
    for l in range(L):
        stk.load_prior(l, kp_in[l], vp_in[l])
    stk.zero_grad()
    qd, knd, vnd, dod = ([t.to(DEV) for t in ts] for ts in (q, kn, vn, do))
    o = [torch.empty(hq, C, d, dtype=torch.bfloat16, device=DEV) for _ in range(L)]
    lse = [torch.empty(hq, C, dtype=torch.float32, device=DEV) for _ in range(L)]
    dq = [torch.empty(hq, C, d, dtype=torch.float32, device=DEV) for _ in range(L)]
    stk.step(qd, knd, vnd, dod, o, lse, dq)
    torch.cuda.synchronize()
    log("    offloaded step done")
    sels = None if top_k is None else [(s.clone(), c.clone()) for s, c in zip(stk.sel, stk.count)]
    pools = stk.resident_pools()
    o2 = [torch.empty_like(t) for t in o]
    lse2 = [torch.empty_like(t) for t in lse]
    dq2 = [torch.empty_like(t) for t in dq]
    stk.resident_step(pools, qd, knd, vnd, dod, o2, lse2, dq2)
    torch.cuda.synchronize()
    log("    resident step done")
    n_local = stk.n_local
    for l in range(L):
        assert torch.equal(bits(o[l]), bits(o2[l])), f"O layer {l}"
        assert torch.equal(lse[l].cpu(), lse2[l].cpu()), f"LSE layer {l}"
        assert torch.equal(dq[l].cpu(), dq2[l].cpu()), f"dQ layer {l}"
        assert torch.equal(stk.hdk[l].cpu(), pools[l].dk.cpu()), f"dK pool layer {l}"
        assert torch.equal(stk.hdv[l].cpu(), pools[l].dv.cpu()), f"dV pool layer {l}"
        if sels is not None:
            assert torch.equal(sels[l][0].cpu(), stk.sel[l].cpu()), f"selection layer {l}"
            assert torch.equal(sels[l][1].cpu(), stk.count[l].cpu())
        for g in range(hkv):   # the chunk's new pages reached the host cache
            pg = g * stk.npph + stk.first_local
            got_k = stk.hk[l][pg:pg + n_local].reshape(-1, d)[:C]
            got_v = stk.hv[l][pg:pg + n_local].reshape(-1, d)[:C]
            assert torch.equal(bits(got_k), bits(kn[l][g])) and torch.equal(bits(got_v), bits(vn[l][g]))
    log("    offloaded == resident, bit for bit")
    # the oracle, layer by layer, on its own pool (identity placement)
    table = torch.arange(hkv * stk.npph, dtype=torch.int32).reshape(hkv, stk.npph)
    for l in range(L):
        kpo = torch.zeros(hkv * stk.npph, P, d, dtype=torch.bfloat16)
        vpo = torch.zeros_like(kpo)
        orc.append(kpo, table, torch.cat([kp_in[l], kn[l]], dim=1), 0)
        orc.append(vpo, table, torch.cat([vp_in[l], vn[l]], dim=1), 0)
        osel = None
        if top_k is not None:
            summ = torch.zeros(hkv * stk.npph, 2, d, dtype=torch.bfloat16)
            orc.summarize(kpo, table, summ, 0, stk.npph, prior + C)
            osel = [ch for (_, _, ch) in orc.select_pages(q[l], summ, table, prior, P, G, top_k)]
            for g in range(hkv):
                n = int(sels[l][1][g])
                assert sels[l][0][g, :n].cpu().tolist() == osel[g], f"oracle selection layer {l}"
        gk = torch.zeros(kpo.shape, dtype=torch.float64)
        gv = torch.zeros(kpo.shape, dtype=torch.float64)
        dQ, _, O, Lse = orc.bwd(q[l], kpo, vpo, table, prior, osel, stk.scale, do[l], gk, gv,
                                table, with_fwd=True)
        compare(f"O(l{l})", o[l], O, torch.bfloat16)
        compare(f"dQ(l{l})", dq[l], dQ, torch.bfloat16)
        assert (lse[l].cpu().double() - Lse).abs().max().item() <= 1e-2
        compare(f"dK(l{l})", stk.hdk[l].cpu(), gk, torch.bfloat16)
        compare(f"dV(l{l})", stk.hdv[l].cpu(), gv, torch.bfloat16)
