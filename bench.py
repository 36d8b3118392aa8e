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

METRIC = "fwd+bwd paged chunk-attn TFLOP/s @1M ctx; % MFMA/HBM peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# Algorithmic FLOP per attended (query, key) pair and head_dim unit, per kernel:
# forward = S and PV; the dK/dV pass = S, dP (recomputed), dV, dK; the dQ pass is
# credited with dQ only (its S and dP are recomputation).
FLOP_PER_PAIR_D = {"fwd_mfma": 4, "dkdv_mfma": 8, "dq_mfma": 2}


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


def cpu_baseline(w, x, table_cpu, sel_cpu, rows: int):
    """The oracle (fp64 CPU) on a bounded sample of the same step: KV head 0, its
    query heads, the last `rows` queries of the chunk, over exactly the keys those
    queries attend in the full chunk."""
    import torch
    import oracle as orc

    P, C, t0, G = w.page, w.chunk, w.t0, w.group
    rows = min(rows, C)
    t0s = t0 + C - rows
    shift = 0
    if w.window > 0:
        # local attention depends on positions only through p - t: renumber the pages
        # from the first one the sample's windows reach, so the oracle scans no others
        shift = max(0, t0s - w.window + 1) // P * P
    sel0 = list(sel_cpu[0]) if sel_cpu is not None else list(range(shift // P, t0 // P))
    # the chunk's own pages before the sample are selected pages for the sample
    sel_s = sorted(set(sel0) | set(range(t0 // P, t0s // P)))
    pages = orc.attended_pages(t0s, rows, P, sel_s)
    # compact oracle pool holding only the attended pages of head 0
    tab = torch.zeros(1, (t0 + C) // P + 1, dtype=torch.int32)
    for i, lp in enumerate(pages):
        tab[0, lp] = i
    kp = torch.zeros(len(pages), P, w.d, dtype=w.dtype)
    vp = torch.zeros_like(kp)
    kh, vh = x["k"][0:1], x["v"][0:1]
    for lp in pages:
        a, b = lp * P, min((lp + 1) * P, t0 + C)
        orc.append(kp, tab, kh[:, a:b].cpu(), a)
        orc.append(vp, tab, vh[:, a:b].cpu(), a)
    q = x["q"][0:G, C - rows:].cpu()
    do = x["do"][0:G, C - rows:].cpu()
    pairs = 0
    for i in range(rows):
        p = t0s + i
        lo = p - w.window + 1 if w.window > 0 else 0
        pairs += sum(max(0, min(P, p - lp * P + 1) - max(0, lo - lp * P)) for lp in pages
                     if lp * P <= p)
    pairs *= G
    threads = torch.get_num_threads()
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
    dt = time.perf_counter() - t
    flop = 14 * w.d * pairs
    return {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"KV head 0 of {w.hkv} ({G} query heads), last {rows} of {C} chunk queries "
                      f"over the same {len(pages)} attended pages; oracle fwd+bwd in fp64; "
                      f"{pairs} pairs, {dt:.1f} s"}


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="sparse1m",
                    choices=["sparse1m", "dense128k", "sparse4m", "local1m"])
    ap.add_argument("--window", type=int, default=None,
                    help="local-attention window overriding the workload's (dense workloads)")
    ap.add_argument("--cpu-rows", type=int, default=2048,
                    help="chunk queries in the oracle's CPU-baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
        roof = {"kernel": dom, "bound": "mfma", "achieved": ach, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS,
                "traffic": None if tr is None else tr["bytes"],
                "traffic_detail": tr,
                "algorithmic_flop_per_launch": FLOP_PER_PAIR_D[dom] * w.d * pairs,
                "ms_per_launch": dom_ms}
    else:
        roof = {"kernel": dom, "bound": "hbm", "achieved": None, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": None, "traffic": None, "ms_per_launch": dom_ms}

    cpu = None
    if not args.no_cpu_baseline:
        x_cpu = {"k": x["k"], "v": x["v"], "q": x["q"], "do": x["do"]}
        sel_cpu = [sel[g, :counts[g]].tolist() for g in range(w.hkv)] if sparse else None
        log("[bench] timing the oracle on the CPU sample ...")
        cpu = cpu_baseline(w, x_cpu, x["table"], sel_cpu, args.cpu_rows)
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
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
