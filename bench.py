#!/usr/bin/env python3
"""Benchmark of the paged chunk-attention hot path on one MI355X.

A step is one pass of the whole path over one chunk of synthetic Qwen2.5-7B-shaped
input (28 query heads, 4 KV heads, head_dim 128, bf16, 128-token pages):
append the chunk's K/V into the page pool, summarize its pages, select the top-k
prior pages (sparse workloads), forward, backward (dQ written, dK/dV added into the
fp32 gradient pool). The prior context is written into the pool before timing.

    python bench.py [--steps K] [--warmup W] [--workload sparse1m|dense128k|sparse4m]

Prints one JSON line (stdout). Progress goes to stderr.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
# Hardware queues per process (HIP's default is 4). The offload-schedule measurement
# runs a compute stream and two copy streams beside the default one; with four queues
# HIP can give a copy stream the compute stream's queue, where it waits behind the
# kernels (measured 5-80% slower schedules). Raised to 8 (when lower) before HIP
# initialises; the environment may already hold HIP's default of 4.
try:
    _hwq = int(os.environ.get("GPU_MAX_HW_QUEUES", "4"))
except ValueError:
    _hwq = 4
if _hwq < 8:
    os.environ["GPU_MAX_HW_QUEUES"] = "8"

METRIC = "fwd+bwd paged chunk-attn TFLOP/s @1M ctx; % MFMA/HBM peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_FP32_VECTOR_TFLOPS = 157.3  # MI355X fp32 vector peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# Algorithmic FLOP per attended (query, key) pair and head_dim unit, per kernel:
# forward = S and PV; the dK/dV pass = S, dP (recomputed), dV, dK; the dQ pass is
# credited with dQ only: dq_mfma recomputes S and dP, dqs_mfma reads the dS the dK/dV
# pass spilled.
FLOP_PER_PAIR_D = {"fwd_mfma": 4, "dkdv_mfma": 8, "dq_mfma": 2, "dqs_mfma": 2}
# what each pass executes on the matrix cores
HW_FLOP_PER_PAIR_D = {"fwd_mfma": 4, "dkdv_mfma": 8, "dq_mfma": 6, "dqs_mfma": 2}


def spill_read_bytes(w, counts):
    """Bytes of spilled dS the dQ-from-dS pass reads: for every query head and 64-query
    tile, the 64-key stages up to the one holding the tile's last query's key, 64 x 64
    bf16 each (the attended pairs plus the masked part of the diagonal stages)."""
    C, P, t0 = w.chunk, w.page, w.t0
    first_local = t0 // P
    n_local = (t0 + C - 1) // P - first_local + 1
    total = 0
    for g in range(w.hkv):
        n_sel = counts[g] if counts is not None else t0 // P
        n_keys = (n_sel + n_local) * P
        local0 = n_sel * P
        for qt in range((C + 63) // 64):
            qlast = t0 + min(C, 64 * qt + 64) - 1
            klim = min(qlast - first_local * P + local0, n_keys - 1)
            total += w.group * (klim // 64 + 1) * 64 * 64 * 2
    return total


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary
    (profiles/<workload>_step_traffic.txt, FETCH_SIZE/WRITE_SIZE scaled by a copy of
    known size), or None when there is none or the kernel source changed since."""
    from paged_chunk_attention_amd.build import mfma_source_hash
    path = os.path.join(ROOT, "profiles", f"{workload}_step_traffic.txt")
    if not os.path.exists(path):
        return None
    sha = mfma_source_hash()
    fields = {}
    for line in open(path):
        parts = line.split()
        if len(parts) >= 2 and parts[0] == "source_sha256_16":
            fields["sha"] = parts[1]
        elif len(parts) == 4 and parts[0] == "kernel":
            fields[parts[1]] = (int(parts[2]), int(parts[3]))
    if fields.get("sha") != sha:
        return None
    rec = fields.get(kernel + "_kernel") or fields.get(kernel)
    if rec is None:  # a template instance (the only one the profiled step ran)
        inst = [k for k in fields if k.startswith(kernel + "_kernel<")]
        rec = fields[inst[0]] if len(inst) == 1 else None
    return None if rec is None else {"read_bytes": rec[0], "write_bytes": rec[1],
                                     "bytes": rec[0] + rec[1]}


def attended_pairs(w, counts):
    """(query, key) pairs the chunk attends, summed over query heads."""
    C, P, t0 = w.chunk, w.page, w.t0
    if w.window > 0:  # local attention: min(window, p + 1) keys for the query at p
        return w.hq * sum(min(w.window, t0 + i + 1) for i in range(C))
    first_local = t0 // P
    # local keys visible to query i: positions first_local*P .. t0+i
    local = sum((t0 + i) - first_local * P + 1 for i in range(C))
    total = 0
    for g in range(w.hkv):
        prior = counts[g] if counts is not None else t0 // P
        total += w.group * (prior * P * C + local)
    return total


def _oracle_sample_head(w, x, sel_head, g: int, rows: int):
    """Oracle fwd+bwd for KV head g's query heads over the last `rows` chunk queries and
    exactly the keys they attend in the full chunk; returns (seconds, pairs)."""
    import torch
    import oracle as orc

    P, C, t0, G = w.page, w.chunk, w.t0, w.group
    t0s = t0 + C - rows
    shift = 0
    if w.window > 0:
        # local attention depends on positions only through p - t: renumber the pages
        # from the first one the sample's windows reach, so the oracle scans no others
        shift = max(0, t0s - w.window + 1) // P * P
    sel0 = list(sel_head) if sel_head is not None else list(range(shift // P, t0 // P))
    # the chunk's own pages before the sample are selected pages for the sample
    sel_s = sorted(set(sel0) | set(range(t0 // P, t0s // P)))
    pages = orc.attended_pages(t0s, rows, P, sel_s)
    # compact oracle pool holding only the attended pages of this head
    tab = torch.zeros(1, (t0 + C) // P + 1, dtype=torch.int32)
    for i, lp in enumerate(pages):
        tab[0, lp] = i
    kp = torch.zeros(len(pages), P, w.d, dtype=w.dtype)
    vp = torch.zeros_like(kp)
    kh, vh = x["k"][g:g + 1], x["v"][g:g + 1]
    for lp in pages:
        a, b = lp * P, min((lp + 1) * P, t0 + C)
        orc.append(kp, tab, kh[:, a:b].cpu(), a)
        orc.append(vp, tab, vh[:, a:b].cpu(), a)
    q = x["q"][g * G:(g + 1) * G, C - rows:].cpu()
    do = x["do"][g * G:(g + 1) * G, C - rows:].cpu()
    pairs = 0
    for i in range(rows):
        p = t0s + i
        lo = p - w.window + 1 if w.window > 0 else 0
        pairs += sum(max(0, min(P, p - lp * P + 1) - max(0, lo - lp * P)) for lp in pages
                     if lp * P <= p)
    pairs *= G
    t = time.perf_counter()
    if w.window > 0:
        # the same computation with every position moved down by `shift` (dense call)
        tab_w = torch.zeros_like(tab)
        for lp in pages:
            tab_w[0, lp - shift // P] = tab[0, lp]
        orc.fwd(q, kp, vp, tab_w, t0s - shift, None, w.scale, window=w.window)
        orc.bwd(q, kp, vp, tab_w, t0s - shift, None, w.scale, do, window=w.window)
    else:
        orc.fwd(q, kp, vp, tab, t0s, [sel_s], w.scale)
        orc.bwd(q, kp, vp, tab, t0s, [sel_s], w.scale, do)
    return time.perf_counter() - t, pairs


def cpu_baseline(w, x, sel_cpu, rows: int, max_pairs: float):
    """The oracle (fp64 CPU) on a bounded sample of the same step: the last `rows`
    queries of the chunk for as many KV heads (with their query heads) as fit in
    about `max_pairs` attended pairs, halving `rows` when one head alone exceeds it,
    each over exactly the keys those queries attend in the full chunk."""
    import torch

    P, C, t0, G = w.page, w.chunk, w.t0, w.group
    rows = min(rows, C)

    def est(g, r):  # upper bound on one head's pairs: every attended prior key plus the chunk
        n_prior = len(sel_cpu[g]) * P if sel_cpu is not None else t0
        if w.window > 0:
            n_prior = min(n_prior, w.window)
        return G * r * (n_prior + C)

    while rows > 64 and est(0, rows) > max_pairs:
        rows //= 2
    heads, total = 0, 0
    while heads < w.hkv and (heads == 0 or total + est(heads, rows) <= max_pairs):
        total += est(heads, rows)
        heads += 1
    threads = torch.get_num_threads()
    dt, pairs = 0.0, 0
    for g in range(heads):
        s, p = _oracle_sample_head(w, x, sel_cpu[g] if sel_cpu is not None else None, g, rows)
        dt += s
        pairs += p
    flop = 14 * w.d * pairs
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"KV heads 0..{heads - 1} of {w.hkv} ({heads * G} query heads), last {rows} "
                      f"of {C} chunk queries, each head over the keys its queries attend; oracle "
                      f"fwd+bwd in fp64; {pairs} pairs, {dt:.1f} s"}


PEAK_PCIE_GBS = 64.0  # PCIe 5.0 x16 host link, per direction


def offload_leg(pca, torch, w, pool, table, gtable, sel, count, reps=10):
    """The page moves of the CPU offload of one sparse layer-chunk (explainer 2.C), each
    timed alone with HIP events on a second stream: fetch of the selected pages from
    pinned host pages into another layer's device pool, offload of the chunk's new pages
    to the host, write-back of the attended gradient pages into a pinned fp32 host pool;
    and copy-engine transfers of 256 MiB as the link reference."""
    P, C, t0, D = w.page, w.chunk, w.t0, w.d
    esize = 2 if w.dtype == torch.bfloat16 else 4
    page_b = P * D * esize
    hkv = w.hkv
    n_cand = t0 // P
    first_local = n_cand
    n_local = (t0 + C - 1) // P - first_local + 1
    k = sel.shape[1]
    dev = "cuda"
    side = torch.cuda.Stream()
    # host copies of the layer's prior pages: contents do not matter for timing, so a
    # pool of 1024 pages stands in for the whole layer (logical pages map onto it)
    n_host = 1024
    host_k = torch.empty(n_host, P, D, dtype=w.dtype, pin_memory=True)
    host_v = torch.empty_like(host_k, pin_memory=True)
    host_table = ((torch.arange(hkv * n_cand, dtype=torch.int64) % n_host).to(torch.int32)
                  .reshape(hkv, n_cand).to(dev))
    # the next layer's device pool: its local pages plus one staging page per selection
    nxt = pca.PagedPool(hkv * (k + n_local), P, D, w.hq, hkv, w.dtype, dev, with_summary=False,
                        with_grad=False)
    nxt_table = torch.zeros(hkv, first_local + n_local, dtype=torch.int32, device=dev)
    stage = torch.arange(hkv * k, dtype=torch.int32, device=dev).reshape(hkv, k)
    # the chunk's new pages (K and V of every head) to host slots
    local_phys = table[:, first_local:first_local + n_local].contiguous().flatten()
    host_new_k = torch.empty(hkv * n_local, P, D, dtype=w.dtype, pin_memory=True)
    host_new_v = torch.empty_like(host_new_k, pin_memory=True)
    new_ids = torch.arange(hkv * n_local, dtype=torch.int32, device=dev)
    # the attended pages' gradients (selected + local) into a pinned fp32 host pool
    att = torch.cat([sel.to(torch.int64), torch.arange(first_local, first_local + n_local,
                                                        device=dev).expand(hkv, -1)], 1)
    g_ids = torch.gather(gtable.to(torch.int64), 1, att).to(torch.int32).flatten().contiguous()
    host_dk = torch.zeros(g_ids.numel(), P, D, dtype=torch.float32, pin_memory=True)
    host_dv = torch.zeros_like(host_dk, pin_memory=True)
    host_g_ids = torch.arange(g_ids.numel(), dtype=torch.int32, device=dev)

    moves = {
        "fetch_selected": (lambda st: pca.oomb_fetch_selected(nxt, nxt_table, host_k, host_v,
                                                              host_table, sel, count, stage,
                                                              n_logical=n_cand, stream=st),
                           hkv * k * 2 * page_b, "host -> device",
                           f"{hkv} x {k} selected pages, K and V"),
        "offload_new_pages": (lambda st: (pca.oomb_copy_pages(pool.k, host_new_k, local_phys, new_ids,
                                                              stream=st),
                                          pca.oomb_copy_pages(pool.v, host_new_v, local_phys, new_ids,
                                                              stream=st)),
                              hkv * n_local * 2 * page_b, "device -> host",
                              f"{hkv} x {n_local} chunk pages, K and V"),
        "grad_write_back": (lambda st: (pca.oomb_add_pages_f32(pool.dk, host_dk, g_ids, host_g_ids,
                                                               stream=st),
                                        pca.oomb_add_pages_f32(pool.dv, host_dv, g_ids, host_g_ids,
                                                               stream=st)),
                            2 * g_ids.numel() * P * D * 4, "device -> host (read + write host)",
                            f"{g_ids.numel()} attended gradient pages, dK and dV, added into the host pool"),
    }

    def timed(fn, stream):
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn(stream)
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        times.sort()
        return times[len(times) // 2]

    out = {"peak_GBps": PEAK_PCIE_GBS, "link": "PCIe 5.0 x16, per direction"}
    for name, (fn, nbytes, direction, what) in moves.items():
        fn(side)
        torch.cuda.synchronize()
        ms = timed(fn, side)
        gbs = nbytes / (ms * 1e-3) / 1e9
        out[name] = {"ms": ms, "bytes": nbytes, "GBps": gbs, "frac": gbs / PEAK_PCIE_GBS,
                     "direction": direction, "work": what}
    # copy-engine reference: 256 MiB pinned -> device and back
    hbuf = torch.empty(256 << 20, dtype=torch.uint8, pin_memory=True)
    dbuf = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    for name, fn in (("copy_engine_h2d", lambda st: dbuf.copy_(hbuf, non_blocking=True)),
                     ("copy_engine_d2h", lambda st: hbuf.copy_(dbuf, non_blocking=True))):
        def run(st, fn=fn):
            with torch.cuda.stream(st):
                fn(st)
        run(side)
        torch.cuda.synchronize()
        ms = timed(run, side)
        gbs = (256 << 20) / (ms * 1e-3) / 1e9
        out[name] = {"ms": ms, "bytes": 256 << 20, "GBps": gbs, "frac": gbs / PEAK_PCIE_GBS}
    return out


def offload_schedule_leg(pca, torch, name, n_layers, reps=3, steps=4, grads_on_host=True):
    """The offload schedule end to end (explainer 2.C): one chunk step (forward through
    `n_layers` attention layers, backward in reverse) of the named workload's geometry
    with every layer's K/V cache and gradient pool in pinned host memory and the page
    moves overlapped on a copy stream (paged_chunk_attention_amd.offload), against the
    same step on all-resident caches, each timed over `steps` consecutive chunk steps.
    Reports both times per step, the overhead and the bytes moved per step; the results
    of the two runs are equal bit for bit (GPU test)."""
    import workloads as wl
    from paged_chunk_attention_amd.offload import OffloadedAttentionStack
    w = wl.WORKLOADS[name]
    C, P, t0 = w.chunk, w.page, w.t0
    dev = "cuda"
    stk = OffloadedAttentionStack(n_layers, w.hq, w.hkv, w.d, P, t0, C, top_k=w.top_k,
                                  dtype=w.dtype, device=dev, grads_on_host=grads_on_host)
    gen = torch.Generator(device=dev).manual_seed(11)

    def rnd(*shape):
        return torch.randn(*shape, generator=gen, device=dev).to(w.dtype)

    for l in range(n_layers):
        stk.load_prior(l, rnd(w.hkv, t0, w.d), rnd(w.hkv, t0, w.d))
    q = [rnd(w.hq, C, w.d) for _ in range(n_layers)]
    kn = [rnd(w.hkv, C, w.d) for _ in range(n_layers)]
    vn = [rnd(w.hkv, C, w.d) for _ in range(n_layers)]
    do = [rnd(w.hq, C, w.d) for _ in range(n_layers)]
    o = [torch.empty(w.hq, C, w.d, dtype=w.dtype, device=dev) for _ in range(n_layers)]
    lse = [torch.empty(w.hq, C, dtype=torch.float32, device=dev) for _ in range(n_layers)]
    dq = [torch.empty(w.hq, C, w.d, dtype=torch.float32, device=dev) for _ in range(n_layers)]
    pools = stk.resident_pools()

    def resident():
        for _ in range(steps):
            for p_ in pools:
                p_.zero_grad()
            stk.resident_step(pools, q, kn, vn, do, o, lse, dq)

    def offloaded():
        for s_ in range(steps):   # consecutive chunk steps: one's tail overlaps the next's head
            stk.step(q, kn, vn, do, o, lse, dq, join=s_ == steps - 1)

    res = {}
    for label, fn in (("resident", resident), ("offloaded", offloaded), ("resident_again", resident),
                      ("offloaded_again", offloaded)):
        fn()
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            t = time.perf_counter()
            fn()
            torch.cuda.synchronize()
            times.append((time.perf_counter() - t) * 1e3 / steps)
        res[label] = times
    base = min(res["resident"] + res["resident_again"])
    off = min(res["offloaded"] + res["offloaded_again"])
    esize = 2 if w.dtype == torch.bfloat16 else 4
    page_b = P * w.d * esize
    grad_page_b = 2 * P * w.d * 4 if grads_on_host else 0   # dK and dV, fp32
    if w.top_k is None:
        # K/V: prior pages (forward) and every page (backward, but the last layer's);
        # gradients: every page in and out
        h2d = (n_layers * w.hkv * stk.n_prior + (n_layers - 1) * w.hkv * stk.npph) * 2 * page_b \
            + n_layers * w.hkv * stk.npph * grad_page_b
        d2h = n_layers * w.hkv * (stk.n_local * 2 * page_b + stk.npph * grad_page_b)
    else:
        # K/V: the selected pages twice, the local pages once; gradients: added into the
        # host pool (read and written there by the add kernel)
        h2d = (n_layers * w.hkv * 2 * stk.k_sel + (n_layers - 1) * w.hkv * stk.n_local) * 2 * page_b \
            + n_layers * w.hkv * (stk.k_sel + stk.n_local) * grad_page_b
        d2h = n_layers * w.hkv * (stk.n_local * 2 * page_b + (stk.k_sel + stk.n_local) * grad_page_b)
    out = {"layers": n_layers, "steps_timed": steps, "gradients_on_host": grads_on_host,
           "resident_ms": base, "offloaded_ms": off,
           "all_ms": {k_: [round(v_, 3) for v_ in t_] for k_, t_ in res.items()},
           "overhead": off / base - 1.0, "bytes_host_to_device": h2d,
           "bytes_device_to_host": d2h,
           "what": (f"one {C}-query chunk after {t0} tokens ({w.name} geometry, "
                    f"{'top-' + str(w.top_k) if w.top_k else 'dense'}), forward through "
                    f"{n_layers} layers then backward, caches and gradients in pinned host "
                    "memory with the next layer's pages fetched and the gradient pages written "
                    "back on a copy stream, against the same step on resident caches")}
    del stk, pools
    torch.cuda.empty_cache()
    return out


def mean_selector_leg(pca, torch, w, pool, table, q, sel, count, needles, reps=3):
    """The selector variant (mean-key page representatives): its whole-context summary
    timed with cold caches and its selection timed warm, both against HBM; then how far
    it agrees with the min/max selection of the step, and each one's recall of the
    needle pages."""
    P, C, t0, D = w.page, w.chunk, w.t0, w.d
    esize = 2 if w.dtype == torch.bfloat16 else 4
    n_pages = t0 // P
    n_cand = n_pages
    kmean = torch.zeros(pool.k.shape[0], D, dtype=torch.float32, device="cuda")
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(fn, cold):
        times = []
        for _ in range(reps):
            if cold:
                scratch.fill_(1)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        times.sort()
        return times[len(times) // 2]

    out = {}
    ms = timed(lambda: pca.oomb_page_summarize_mean(pool, table, 0, n_pages, t0, kmean), True)
    nbytes = w.hkv * t0 * D * esize + w.hkv * n_pages * D * 4
    out["page_summarize_mean"] = {"ms": ms, "algorithmic_bytes": nbytes,
                                  "achieved_GBps": nbytes / (ms * 1e-3) / 1e9,
                                  "frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                  "peak_GBps": PEAK_HBM_GBS, "cache": "cold",
                                  "work": f"{w.hkv} x {n_pages} pages of {P} tokens, fp32 means"}
    pca.oomb_page_summarize_mean(pool, table, 0, (t0 + C - 1) // P + 1, t0 + C, kmean)
    sel_m = torch.zeros_like(sel)
    cnt_m = torch.zeros_like(count)
    ws = torch.empty(pca.select_workspace_bytes(pool, C, t0), dtype=torch.uint8, device="cuda")
    ms = timed(lambda: pca.oomb_select_pages_mean(pool, table, q, t0, w.top_k, kmean, sel=sel_m,
                                                  count=cnt_m, workspace=ws), False)
    nbytes = w.hq * C * D * esize + w.hkv * n_cand * D * 4
    out["select_pages_mean"] = {"ms": ms, "algorithmic_bytes": nbytes,
                                "achieved_GBps": nbytes / (ms * 1e-3) / 1e9,
                                "frac": nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                "peak_GBps": PEAK_HBM_GBS, "cache": "warm",
                                "work": f"{w.hkv} x {n_cand} candidate pages, {w.hq} x {C} queries"}
    a = [set(sel[g, :int(count[g])].tolist()) for g in range(w.hkv)]
    b = [set(sel_m[g, :int(cnt_m[g])].tolist()) for g in range(w.hkv)]
    nd = set(int(j) for j in needles)
    k = max(1, sum(len(s_) for s_ in a))
    out["overlap"] = sum(len(a[g] & b[g]) for g in range(w.hkv)) / k
    out["needle_recall_minmax"] = (sum(len(a[g] & nd) for g in range(w.hkv)) /
                                   max(1, w.hkv * len(nd)))
    out["needle_recall_mean"] = (sum(len(b[g] & nd) for g in range(w.hkv)) /
                                 max(1, w.hkv * len(nd)))
    out["what"] = ("pages chosen by both selectors over pages chosen (overlap), and the share "
                   "of the needle pages each selection contains, summed over KV heads")
    del scratch
    return out


def tiled_selector_leg(pca, torch, w, pool, table, gtable, q, do, sel, count, needles, tile=1024,
                       reps=5):
    """The per-query-tile selection (explainer 2.D leaves the unit of selection open): each
    tile of `tile` queries selects its own top-k prior pages. Reports the tiled selection's
    time, how far each tile's pages agree with the per-chunk selection of the step and
    their needle recall, and the attention step (forward + backward, one call per tile)
    against the per-chunk step on the same pool."""
    C, t0 = w.chunk, w.t0
    n_tiles = -(-C // tile)
    stream = torch.cuda.current_stream()
    width = pca.tile_row_length(pool, C, t0, w.top_k, tile)
    sel_t = torch.full((n_tiles, w.hkv, width), -1, dtype=torch.int32, device="cuda")
    cnt_t = torch.zeros(n_tiles, w.hkv, dtype=torch.int32, device="cuda")
    ws = torch.empty(pca.select_tiled_workspace_bytes(pool, C, t0, tile), dtype=torch.uint8,
                     device="cuda")

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fn()
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        times.sort()
        return times[len(times) // 2]

    sel_ms = timed(lambda: pca.oomb_select_pages_tiled(pool, table, q, t0, w.top_k, tile,
                                                       sel=sel_t, count=cnt_t, workspace=ws))
    k = max(1, min(w.top_k, t0 // w.page))
    chunk_sets = [set(sel[g, :int(count[g])].tolist()) for g in range(w.hkv)]
    nd = set(int(j) for j in needles)
    sel_h, cnt_h = sel_t.cpu(), cnt_t.cpu()
    overlap, recall = [], []
    for j in range(n_tiles):
        for g in range(w.hkv):
            picked = set(sel_h[j, g, :k].tolist())      # the row's top-k part
            overlap.append(len(picked & chunk_sets[g]) / k)
            recall.append(len(picked & nd) / max(1, len(nd)))

    def chunk_attn():
        o, lse = pca.oomb_paged_chunk_attn_fwd(pool, table, q, t0, sel, count, w.scale)
        pca.oomb_paged_chunk_attn_bwd(pool, table, gtable, q, t0, sel, count, o, do, lse, w.scale)

    def tiled_attn():
        o, lses = pca.oomb_paged_chunk_attn_fwd_tiled(pool, table, q, t0, sel_t, cnt_t, tile,
                                                      w.scale)
        pca.oomb_paged_chunk_attn_bwd_tiled(pool, table, gtable, q, t0, sel_t, cnt_t, tile, o,
                                            do, lses, w.scale)

    t_chunk = timed(chunk_attn)
    t_tiled = timed(tiled_attn)
    return {"tile": tile, "tiles": n_tiles, "select_ms": sel_ms,
            "overlap_with_chunk_selection": sum(overlap) / len(overlap),
            "needle_recall_tiled": sum(recall) / len(recall),
            "attention_ms_per_chunk_selection": t_chunk, "attention_ms_tiled": t_tiled,
            "what": (f"{n_tiles} tiles of {tile} queries each select their own top-{w.top_k} "
                     "prior pages; overlap = share of a tile's pages that the chunk's selection "
                     "also holds, averaged over tiles and KV heads; attention = forward + "
                     "backward, one call per tile against one call per chunk")}


def layer_leg(pca, torch, tokens=65536, reps=2):
    """One chunk-recurrent attention layer (paged_chunk_attention_amd.layer) at the
    attention shape of the pages' model (hidden 3584, 28 query / 4 KV heads of 128,
    rotary theta 1e6), chunks of 4096, pages of 128: forward and backward over `tokens`
    tokens, dense and top-64. Reports the time of one layer step, tokens per second and
    the share of it spent in the library's kernels (the rest is the projection GEMMs and
    PyTorch glue)."""
    from paged_chunk_attention_amd.layer import ChunkRecurrentAttention
    hidden, hq, hkv, d, chunk, page = 3584, 28, 4, 128, 4096, 128
    out = {}
    for mode, top_k in (("dense", None), ("top64", 64)):
        layer = ChunkRecurrentAttention(hidden, hq, hkv, d, page, chunk, tokens, top_k=top_k,
                                        dtype=torch.bfloat16, device="cuda", seed=1)
        g = torch.Generator(device="cuda").manual_seed(2)
        x = torch.randn(tokens, hidden, generator=g, device="cuda").to(torch.bfloat16)
        x.requires_grad_()
        dy = torch.randn(tokens, hidden, generator=g, device="cuda").to(torch.bfloat16)

        def step():
            x.grad = None
            for p_ in layer.parameters():
                p_.grad = None
            layer(x).backward(dy)

        step()
        torch.cuda.synchronize()
        times, lib_ms = [], []
        for _ in range(reps):
            with pca.kernel_timer() as timer:
                torch.cuda.synchronize()
                t = time.perf_counter()
                step()
                torch.cuda.synchronize()
                times.append((time.perf_counter() - t) * 1e3)
            lib_ms.append(sum(ms for _, ms in timer.records))
        ms = min(times)
        out[mode] = {"ms_per_layer_step": ms, "tokens_per_s": tokens / (ms * 1e-3),
                     "library_kernel_ms": min(lib_ms), "library_share": min(lib_ms) / ms}
        del layer, x, dy
        torch.cuda.empty_cache()
    out["what"] = (f"forward + backward of one attention layer over {tokens} tokens in chunks of "
                   f"{chunk} (hidden {hidden}, {hq}/{hkv} heads of {d}, pages of {page}); "
                   "library kernels timed with HIP events, the rest is GEMMs and glue")
    return out


def other_workload(pca, torch, name, steps=5, warmup=2):
    """The same step (append, summarize, select when sparse, forward, backward) on another
    benchmark workload, briefly: ms per step, model TFLOP/s, and each matrix-core pass's
    time and hardware FLOP rate against the bf16 peak."""
    import workloads as wl
    w = wl.WORKLOADS[name]
    P, C, t0 = w.page, w.chunk, w.t0
    x = wl.make_inputs(w, device="cuda")
    table, gtable = x["table"].to("cuda"), x["gtable"].to("cuda")
    pool = pca.PagedPool(w.pool_pages, P, w.d, w.hq, w.hkv, w.dtype, "cuda")
    pca.oomb_kv_append(pool, table, x["k"][:, :t0], x["v"][:, :t0], 0)
    pca.oomb_page_summarize(pool, table, 0, t0 // P, t0)
    k_new = x["k"][:, t0:t0 + C].contiguous()
    v_new = x["v"][:, t0:t0 + C].contiguous()
    q, do = x["q"], x["do"]
    first_local = t0 // P
    n_local = (t0 + C - 1) // P - first_local + 1
    sparse = w.top_k is not None
    k = max(0, min(w.top_k, t0 // P)) if sparse else 0
    sel = torch.zeros(w.hkv, max(k, 1), dtype=torch.int32, device="cuda")
    count = torch.zeros(w.hkv, dtype=torch.int32, device="cuda")
    sstride = sel.stride(0) if sparse else -1
    ws_sel = torch.empty(pca.select_workspace_bytes(pool, C, t0), dtype=torch.uint8, device="cuda")
    ws_fwd = torch.empty(max(256, pca.fwd_workspace_bytes(pool, C, t0, sstride, w.window)),
                         dtype=torch.uint8, device="cuda")
    ws_bwd = torch.empty(pca.bwd_workspace_bytes(pool, C, t0, sstride, w.window),
                         dtype=torch.uint8, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(w.hq, C, dtype=torch.float32, device="cuda")
    dq = torch.empty(w.hq, C, w.d, dtype=torch.float32, device="cuda")

    def step():
        pca.oomb_kv_append(pool, table, k_new, v_new, t0)
        pca.oomb_page_summarize(pool, table, first_local, n_local, t0 + C)
        s_, c_ = (None, None)
        if sparse:
            s_, c_ = pca.oomb_select_pages(pool, table, q, t0, w.top_k, sel=sel, count=count,
                                           workspace=ws_sel)
        pca.oomb_paged_chunk_attn_fwd(pool, table, q, t0, s_, c_, w.scale, o=o, lse=lse,
                                      workspace=ws_fwd, window=w.window)
        pca.oomb_paged_chunk_attn_bwd(pool, table, gtable, q, t0, s_, c_, o, do, lse, w.scale,
                                      dq=dq, workspace=ws_bwd, window=w.window)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    with pca.kernel_timer() as timer:
        t_start = time.perf_counter()
        for _ in range(steps):
            step()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t_start
    ms = elapsed * 1e3 / steps
    pairs = attended_pairs(w, count.cpu().tolist() if sparse else None)
    value = 14 * w.d * pairs / (ms * 1e-3) / 1e12
    per = {}
    for kname, kms in timer.records:
        tot, n = per.get(kname, (0.0, 0))
        per[kname] = (tot + kms, n + 1)
    passes = {}
    for kname, hw in HW_FLOP_PER_PAIR_D.items():
        if kname in per:
            kms = per[kname][0] / per[kname][1]
            tf = hw * w.d * pairs / (kms * 1e-3) / 1e12
            passes[kname] = {"ms_per_launch": kms, "hardware_TFLOPs": tf,
                             "frac_of_bf16_peak": tf / PEAK_BF16_TFLOPS}
    if "dqs_mfma" in passes and w.window == 0:
        rd = spill_read_bytes(w, count.cpu().tolist() if sparse else None)
        gbs = rd / (passes["dqs_mfma"]["ms_per_launch"] * 1e-3) / 1e9
        passes["dqs_mfma"].update(spill_read_bytes=rd, spill_read_GBps=gbs,
                                  frac_of_hbm_peak=gbs / PEAK_HBM_GBS)
    del pool, x
    return {"ms_per_step": ms, "value": value, "unit": "TFLOP/s",
            "pct_mfma_peak": 100.0 * value / PEAK_BF16_TFLOPS, "steps": steps,
            "attended_pairs": pairs, "passes": passes}


def sweep_workload(pca, torch, name, reps=2, warmup=1):
    """The chunk-recurrent sweep of a whole sequence (explainer 2.A): forward over the
    chunks in order (append, summarize, select when sparse, forward), then in reverse
    order the forward again and the backward, dK/dV accumulating in the paged fp32 pool
    (zeroed first). Outputs and workspaces are allocated before timing. Returns ms per
    sweep, model TFLOP/s (14 D per attended pair, recomputation not counted) and each
    matrix-core pass's total time and hardware FLOP rate."""
    import types
    import workloads as wl
    w = wl.WORKLOADS[name]
    P, C, S, D = w.page, w.chunk, w.n_chunks, w.d
    x = wl.make_inputs(w, device="cuda")
    table, gtable = x["table"].to("cuda"), x["gtable"].to("cuda")
    pool = pca.PagedPool(w.pool_pages, P, D, w.hq, w.hkv, w.dtype, "cuda")
    sparse = w.top_k is not None
    q_all, do_all, k_all, v_all = x["q"], x["do"], x["k"], x["v"]
    o_all = torch.empty_like(q_all)
    lse_all = torch.empty(S, w.hq, C, dtype=torch.float32, device="cuda")
    dq_all = torch.empty(w.hq, w.total, D, dtype=torch.float32, device="cuda")
    k = max(1, w.top_k or 1)
    sel = torch.zeros(S, w.hkv, k, dtype=torch.int32, device="cuda")
    count = torch.zeros(S, w.hkv, dtype=torch.int32, device="cuda")
    sstride = k if sparse else -1
    nbytes = lambda f: max(256, max(f(c * C) for c in range(S)))
    ws_sel = torch.empty(nbytes(lambda t0: pca.select_workspace_bytes(pool, C, t0)),
                         dtype=torch.uint8, device="cuda")
    ws_fwd = torch.empty(nbytes(lambda t0: pca.fwd_workspace_bytes(pool, C, t0, sstride)),
                         dtype=torch.uint8, device="cuda")
    ws_bwd = torch.empty(nbytes(lambda t0: pca.bwd_workspace_bytes(pool, C, t0, sstride)),
                         dtype=torch.uint8, device="cuda")

    def sweep():
        pool.dk.zero_()
        pool.dv.zero_()
        for c in range(S):
            t0, sl = c * C, slice(c * C, (c + 1) * C)
            pca.oomb_kv_append(pool, table, k_all[:, sl], v_all[:, sl], t0)
            pca.oomb_page_summarize(pool, table, t0 // P, (t0 + C - 1) // P - t0 // P + 1, t0 + C)
            s_, c_ = (None, None)
            if sparse:
                s_, c_ = pca.oomb_select_pages(pool, table, q_all[:, sl], t0, w.top_k, sel=sel[c],
                                               count=count[c], workspace=ws_sel)
            pca.oomb_paged_chunk_attn_fwd(pool, table, q_all[:, sl], t0, s_, c_, w.scale,
                                          o=o_all[:, sl], lse=lse_all[c], workspace=ws_fwd)
        for c in reversed(range(S)):
            t0, sl = c * C, slice(c * C, (c + 1) * C)
            s_, c_ = (sel[c], count[c]) if sparse else (None, None)
            pca.oomb_paged_chunk_attn_fwd(pool, table, q_all[:, sl], t0, s_, c_, w.scale,
                                          o=o_all[:, sl], lse=lse_all[c], workspace=ws_fwd)
            pca.oomb_paged_chunk_attn_bwd(pool, table, gtable, q_all[:, sl], t0, s_, c_,
                                          o_all[:, sl], do_all[:, sl], lse_all[c], w.scale,
                                          dq=dq_all[:, sl], workspace=ws_bwd)

    for _ in range(warmup):
        sweep()
    torch.cuda.synchronize()
    with pca.kernel_timer() as timer:
        t_start = time.perf_counter()
        for _ in range(reps):
            sweep()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t_start
    ms = elapsed * 1e3 / reps
    counts = count.cpu().tolist()
    pairs = 0
    for c in range(S):
        wc = types.SimpleNamespace(chunk=C, page=P, t0=c * C, window=0, hq=w.hq, hkv=w.hkv,
                                   group=w.group)
        pairs += attended_pairs(wc, counts[c] if sparse else None)
    value = 14 * D * pairs / (ms * 1e-3) / 1e12
    # bf16 runs on the matrix cores; fp32 (the tiny workload) on the scalar kernels,
    # against the fp32 vector peak
    peak = PEAK_BF16_TFLOPS if w.dtype == torch.bfloat16 else PEAK_FP32_VECTOR_TFLOPS
    per = {}
    for kname, kms in timer.records:
        tot, n = per.get(kname, (0.0, 0))
        per[kname] = (tot + kms, n + 1)
    kernels = {kname: tot / reps for kname, (tot, n) in per.items()}
    passes = {}
    # per sweep: the forward runs twice per chunk (in order, then recomputed)
    launches = {"fwd_mfma": 2 * S, "dkdv_mfma": S, "dq_mfma": S, "dqs_mfma": S}
    for kname, hw in HW_FLOP_PER_PAIR_D.items():
        if kname in per:
            kms = per[kname][0] / reps
            passes[kname] = {"ms_per_sweep": kms, "launches_per_sweep": per[kname][1] / reps}
            if per[kname][1] == launches[kname] * reps:  # ran for every chunk
                tf = launches[kname] * hw * D * pairs / S / (kms * 1e-3) / 1e12
                passes[kname].update(hardware_TFLOPs=tf, frac_of_bf16_peak=tf / PEAK_BF16_TFLOPS)
    del pool, x, o_all, dq_all
    return {"ms_per_sweep": ms, "value": value, "unit": "TFLOP/s", "dtype": str(w.dtype)[6:],
            "peak_TFLOPs": peak, "pct_peak": 100.0 * value / peak, "sweeps": reps, "chunks": S,
            "chunk": C, "tokens": w.total, "top_k": w.top_k, "attended_pairs": pairs,
            "model_flop_per_sweep": 14 * D * pairs, "passes": passes,
            "kernel_ms_per_sweep": kernels}


def context_build(pca, torch, pool, table, x, w, reps):
    """Write the whole prior context into the pool (kv_append) and summarise its pages
    (page_summarize), each timed on its own stream with HIP events after evicting the
    caches (a 1 GiB scratch write between reps). Returns per-kernel median time, GB/s
    of algorithmic bytes and the fraction of HBM peak."""
    P, t0 = w.page, w.t0
    esize = 2 if w.dtype == torch.bfloat16 else 4
    n_pages = t0 // P
    scratch = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.Stream()
    kv_bytes = 2 * w.hkv * t0 * w.d * esize  # K and V
    # append: read K and V, write them into their pages; summarize: read K pages,
    # write a min and a max row per page
    algo = {"kv_append": 2 * kv_bytes,
            "page_summarize": kv_bytes // 2 + w.hkv * n_pages * 2 * w.d * esize}
    calls = {
        "kv_append": lambda: pca.oomb_kv_append(pool, table, x["k"][:, :t0], x["v"][:, :t0], 0,
                                                stream=stream),
        "page_summarize": lambda: pca.oomb_page_summarize(pool, table, 0, n_pages, t0,
                                                          stream=stream),
    }
    out = {}
    for name in ("kv_append", "page_summarize"):
        times = []
        for _ in range(max(1, reps)):
            scratch.fill_(1)  # evicts L2 and the 256 MB MALL
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            calls[name]()
            e1.record(stream)
            e1.synchronize()
            times.append(e0.elapsed_time(e1))
        ms = sorted(times)[len(times) // 2]
        gbs = algo[name] / (ms * 1e-3) / 1e9
        out[name] = {"ms": ms, "algorithmic_bytes": algo[name], "achieved_GBps": gbs,
                     "peak_GBps": PEAK_HBM_GBS, "frac": gbs / PEAK_HBM_GBS,
                     "cache": "cold", "reps": len(times),
                     "work": f"{w.hkv} kv heads x {t0} tokens" if name == "kv_append"
                             else f"{w.hkv} x {n_pages} pages of {P} tokens"}
        log(f"[bench] {name} (whole {t0}-token context, cold): {ms:.3f} ms, {gbs:.0f} GB/s "
            f"({100 * gbs / PEAK_HBM_GBS:.1f}% of HBM peak)")
    # secondary reference: the device's own streaming copy (torch copy_) of 1 GiB, cold,
    # i.e. what a plain read+write stream achieves on this GPU
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(3)
    dst = torch.empty_like(src)
    times = []
    for _ in range(max(1, reps)):
        scratch.fill_(1)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        with torch.cuda.stream(stream):
            dst.copy_(src)
        e1.record(stream)
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = sorted(times)[len(times) // 2]
    copy_gbs = 2 * src.numel() / (ms * 1e-3) / 1e9
    out["reference_copy"] = {"ms": ms, "bytes": 2 * src.numel(), "achieved_GBps": copy_gbs,
                             "frac": copy_gbs / PEAK_HBM_GBS, "cache": "cold",
                             "what": "torch copy_ of 1 GiB (read + write), achievable-peak reference"}
    for name in ("kv_append", "page_summarize"):
        out[name]["frac_of_reference_copy"] = out[name]["achieved_GBps"] / copy_gbs
    log(f"[bench] reference copy (1 GiB, cold): {copy_gbs:.0f} GB/s ({100 * copy_gbs / PEAK_HBM_GBS:.1f}% of peak)")
    del scratch, src, dst
    return out


def gemm_reference(torch, sizes=(4096, 8192, 16384), reps=10):
    """Secondary reference for the matrix-core roofline: the best rate a library bf16
    GEMM (torch.matmul, i.e. hipBLASLt) reaches on this GPU over n x n x n for the given
    sizes, fp32 accumulation."""
    best = None
    for n in sizes:
        a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
        b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
        c = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
        for _ in range(3):
            torch.matmul(a, b, out=c)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.matmul(a, b, out=c)
        e1.record()
        e1.synchronize()
        ms = e0.elapsed_time(e1) / reps
        tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
        del a, b, c
        if best is None or tf > best["TFLOPs"]:
            best = {"TFLOPs": tf, "ms": ms, "n": n}
    best.update({"frac_of_peak": best["TFLOPs"] / PEAK_BF16_TFLOPS,
                 "what": f"best bf16 GEMM n x n x n over n in {list(sizes)} through torch.matmul "
                         "(hipBLASLt), achievable-peak reference"})
    return best


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="sparse1m",
                    choices=["sparse1m", "dense128k", "sparse4m", "local1m"])
    ap.add_argument("--window", type=int, default=None,
                    help="local-attention window overriding the workload's (dense workloads)")
    ap.add_argument("--cpu-rows", type=int, default=4096,
                    help="chunk queries per KV head in the oracle's CPU-baseline sample")
    ap.add_argument("--cpu-pairs", type=float, default=1.5e9,
                    help="bound on the attended pairs of the CPU-baseline sample (~13 s on 16 threads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-layer", action="store_true",
                    help="skip timing one chunk-recurrent attention layer (65,536 tokens)")
    ap.add_argument("--no-selectors", action="store_true",
                    help="skip the selector-variant leg (mean-key and per-tile selection)")
    ap.add_argument("--no-offload", action="store_true",
                    help="skip the CPU-offload measurements (sparse workloads)")
    ap.add_argument("--offload-layers", type=int, default=4,
                    help="layers of the offload schedule measurement (dense 128K and sparse 1M)")
    ap.add_argument("--also", default="dense128k,sparse4m,local1m,sweep256k,sweep256k_top64,tiny",
                    help="comma-separated other workloads to time briefly ('none' for none)")
    ap.add_argument("--hbm-reps", type=int, default=3,
                    help="cold-cache repetitions of the whole-context append and summarize")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the hot path here is "
              "the single-GPU share; no multi-GPU configuration is built.", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_chunk_attention_amd as pca
    import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda"
    w = wl.WORKLOADS[args.workload]
    if args.window is not None:
        if w.top_k is not None:
            print("--window applies to dense workloads only", file=sys.stderr)
            sys.exit(2)
        w = dataclasses.replace(w, window=args.window, name=f"{w.name}_w{args.window}")
    P, C, t0 = w.page, w.chunk, w.t0
    log(f"[bench] workload={w.name} hq={w.hq} hkv={w.hkv} d={w.d} page={P} chunk={C} t0={t0} "
        f"top_k={w.top_k}")
    x = wl.make_inputs(w, device=dev)
    table = x["table"].to(dev)
    gtable = x["gtable"].to(dev)
    pool = pca.PagedPool(w.pool_pages, P, w.d, w.hq, w.hkv, w.dtype, dev)
    # prior context: written once here, and timed (cold cache) as the HBM-bound kernels
    # of the path: the whole-context append and page summaries
    hbm = context_build(pca, torch, pool, table, x, w, args.hbm_reps)
    k_new = x["k"][:, t0:t0 + C].contiguous()
    v_new = x["v"][:, t0:t0 + C].contiguous()
    q, do = x["q"], x["do"]
    first_local = t0 // P
    n_local = (t0 + C - 1) // P - first_local + 1
    k = max(0, min(w.top_k, t0 // P)) if w.top_k is not None else 0
    sel = torch.zeros(w.hkv, max(k, 1), dtype=torch.int32, device=dev)
    count = torch.zeros(w.hkv, dtype=torch.int32, device=dev)
    ws_sel = torch.empty(pca.select_workspace_bytes(pool, C, t0), dtype=torch.uint8, device=dev)
    sstride = sel.stride(0) if w.top_k is not None else -1
    ws_bwd = torch.empty(pca.bwd_workspace_bytes(pool, C, t0, sstride, w.window),
                         dtype=torch.uint8, device=dev)
    ws_fwd = torch.empty(max(256, pca.fwd_workspace_bytes(pool, C, t0, sstride, w.window)),
                         dtype=torch.uint8, device=dev)
    o = torch.empty_like(q)
    lse = torch.empty(w.hq, C, dtype=torch.float32, device=dev)
    dq = torch.empty(w.hq, C, w.d, dtype=torch.float32, device=dev)
    sparse = w.top_k is not None

    def step():
        pca.oomb_kv_append(pool, table, k_new, v_new, t0)
        pca.oomb_page_summarize(pool, table, first_local, n_local, t0 + C)
        s_, c_ = (None, None)
        if sparse:
            s_, c_ = pca.oomb_select_pages(pool, table, q, t0, w.top_k, sel=sel, count=count,
                                           workspace=ws_sel)
        pca.oomb_paged_chunk_attn_fwd(pool, table, q, t0, s_, c_, w.scale, o=o, lse=lse,
                                      workspace=ws_fwd, window=w.window)
        pca.oomb_paged_chunk_attn_bwd(pool, table, gtable, q, t0, s_, c_, o, do, lse, w.scale,
                                      dq=dq, workspace=ws_bwd, window=w.window)

    # One plain copy of known size, untimed: under rocprofv3 --pmc its FETCH_SIZE and
    # WRITE_SIZE calibrate the counters against 256 MiB read + 256 MiB written.
    calib_src = torch.empty(256 << 20, dtype=torch.uint8, device=dev).fill_(1)
    calib_dst = torch.empty_like(calib_src)
    calib_dst.copy_(calib_src)
    torch.cuda.synchronize()
    del calib_src, calib_dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")

    # timed region: every kernel is bracketed by HIP events on its own stream
    with pca.kernel_timer() as timer:
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for _ in range(args.steps):
            step()
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t_start
    ms_per_step = elapsed * 1e3 / args.steps
    per_kernel = {}
    for name, ms in timer.records:
        tot, n = per_kernel.get(name, (0.0, 0))
        per_kernel[name] = (tot + ms, n + 1)
    counts = count.cpu().tolist() if sparse else None
    pairs = attended_pairs(w, counts)
    flop = 14 * w.d * pairs
    value = flop / (ms_per_step * 1e-3) / 1e12
    log(f"[bench] {args.steps} steps: {ms_per_step:.3f} ms/step, {value:.1f} TFLOP/s, "
        f"pairs={pairs}")
    breakdown = {}
    for name, (tot, n) in sorted(per_kernel.items(), key=lambda kv: -kv[1][0]):
        breakdown[name] = {"ms_per_launch": tot / n, "launches_per_step": n / args.steps}
        log(f"    {name:16s} {tot / n:9.4f} ms x {n / args.steps:.0f}/step")

    # the selection scan (qbar, page scores, top-k) against HBM: it reads the chunk's
    # queries and the summaries of every candidate page once
    if sparse:
        names = ("qbar_partial", "qbar_final", "page_score", "topk")
        sel_ms = sum(per_kernel[n_][0] / args.steps for n_ in names if n_ in per_kernel)
        esize = 2 if w.dtype == torch.bfloat16 else 4
        sel_bytes = w.hq * C * w.d * esize + w.hkv * (t0 // P) * 2 * w.d * esize
        gbs = sel_bytes / (sel_ms * 1e-3) / 1e9
        hbm["select_pages"] = {"ms": sel_ms, "algorithmic_bytes": sel_bytes, "achieved_GBps": gbs,
                               "peak_GBps": PEAK_HBM_GBS, "frac": gbs / PEAK_HBM_GBS,
                               "cache": "warm (inside the timed step)",
                               "work": f"{w.hkv} x {t0 // P} candidate pages, {w.hq} x {C} queries"}

    # roofline of the dominant kernel (largest time per step)
    dom = max(per_kernel, key=lambda k_: per_kernel[k_][0])
    dom_ms = per_kernel[dom][0] / per_kernel[dom][1]
    if dom in FLOP_PER_PAIR_D:
        ach = FLOP_PER_PAIR_D[dom] * w.d * pairs / (dom_ms * 1e-3) / 1e12
        tr = measured_traffic(w.name, dom)
        gemm = gemm_reference(torch)
        log(f"[bench] bf16 GEMM reference: {gemm['TFLOPs']:.0f} TFLOP/s "
            f"({100 * gemm['frac_of_peak']:.1f}% of peak)")
        roof = {"kernel": dom, "bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS,
                "reference_gemm": gemm, "frac_of_reference_gemm": ach / gemm["TFLOPs"],
                "traffic": None if tr is None else tr["bytes"],
                "traffic_detail": tr,
                "algorithmic_flop_per_launch": FLOP_PER_PAIR_D[dom] * w.d * pairs,
                "ms_per_launch": dom_ms}
    else:
        roof = {"kernel": dom, "bound": "hbm", "achieved": None, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": None, "traffic": None, "ms_per_launch": dom_ms}

    selector = None
    if sparse and not args.no_selectors:
        selector = mean_selector_leg(pca, torch, w, pool, table, q, sel, count, x["needles"])
        hbm["page_summarize_mean"] = selector.pop("page_summarize_mean")
        hbm["select_pages_mean"] = selector.pop("select_pages_mean")
        selector["tiled"] = tiled_selector_leg(pca, torch, w, pool, table, gtable, q, do, sel,
                                               count, x["needles"])
        log(f"[bench] tiled selection ({selector['tiled']['tiles']} tiles): "
            f"{selector['tiled']['select_ms']:.3f} ms, overlap with the chunk's "
            f"{100 * selector['tiled']['overlap_with_chunk_selection']:.1f} %, attention "
            f"{selector['tiled']['attention_ms_tiled']:.3f} ms vs "
            f"{selector['tiled']['attention_ms_per_chunk_selection']:.3f} ms")
        log(f"[bench] selectors agree on {100 * selector['overlap']:.1f} % of pages; needle recall "
            f"min/max {selector['needle_recall_minmax']:.2f}, mean {selector['needle_recall_mean']:.2f}")

    offload = None
    if sparse and not args.no_offload:
        log("[bench] offload leg ...")
        offload = offload_leg(pca, torch, w, pool, table, gtable, sel, count)
        log(f"[bench] offload: fetch {offload['fetch_selected']['GBps']:.1f} GB/s")
        sched = {}
        for label, sname, on_host in (("dense128k", "dense128k", True),
                                      ("dense128k_grads_on_device", "dense128k", False),
                                      ("sparse1m", "sparse1m", True)):
            log(f"[bench] offload schedule {label}, {args.offload_layers} layers ...")
            sched[label] = offload_schedule_leg(pca, torch, sname, args.offload_layers,
                                                grads_on_host=on_host)
            log(f"[bench] offload schedule {label}: resident {sched[label]['resident_ms']:.2f} ms, "
                f"offloaded {sched[label]['offloaded_ms']:.2f} ms, overhead "
                f"{100 * sched[label]['overhead']:.1f} %")
        offload["schedule"] = sched

    layer = None
    if not args.no_layer:
        log("[bench] layer leg ...")
        layer = layer_leg(pca, torch)
        log(f"[bench] layer: dense {layer['dense']['tokens_per_s']:.0f} tok/s, top64 "
            f"{layer['top64']['tokens_per_s']:.0f} tok/s")

    others = {}
    for name in [n_ for n_ in args.also.split(",") if n_ not in ("", "none", w.name)]:
        if name not in wl.WORKLOADS:
            print(f"unknown workload {name!r} in --also", file=sys.stderr)
            sys.exit(2)
        if wl.WORKLOADS[name].sweep:
            log(f"[bench] {name} sweep ...")
            others[name] = sweep_workload(pca, torch, name)
            log(f"[bench] {name}: {others[name]['ms_per_sweep']:.1f} ms/sweep, "
                f"{others[name]['value']:.1f} TFLOP/s ({others[name]['pct_peak']:.1f}% of the "
                f"{others[name]['dtype']} peak)")
            continue
        log(f"[bench] {name} step ...")
        others[name] = other_workload(pca, torch, name)
        log(f"[bench] {name}: {others[name]['ms_per_step']:.3f} ms/step, "
            f"{others[name]['value']:.1f} TFLOP/s ({others[name]['pct_mfma_peak']:.1f}% of peak)")

    cpu = None
    if not args.no_cpu_baseline:
        x_cpu = {"k": x["k"], "v": x["v"], "q": x["q"], "do": x["do"]}
        sel_cpu = [sel[g, :counts[g]].tolist() for g in range(w.hkv)] if sparse else None
        log("[bench] timing the oracle on the CPU sample ...")
        cpu = cpu_baseline(w, x_cpu, sel_cpu, args.cpu_rows, args.cpu_pairs)
        log(f"[bench] cpu baseline: {cpu['value']:.4f} TFLOP/s on {cpu['cores']} threads")

    out = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "q_heads": w.hq, "kv_heads": w.hkv, "head_dim": w.d,
                   "page": P, "chunk": C, "prior_tokens": t0, "top_k": w.top_k,
                   "window": w.window,
                   "attended_pairs": pairs, "model_flop_per_step": flop,
                   "step": "kv_append+page_summarize+select_pages+fwd+bwd"},
        "pct_mfma_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "roofline": roof,
        "kernels": breakdown,
        "hbm_kernels": hbm,
        "offload": offload,
        "selector_variants": selector,
        "layer": layer,
        "other_workloads": others or None,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
