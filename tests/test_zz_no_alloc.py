"""The allocation-free selection entry point (oomb_select_pages_noalloc, static device
scratch) against the entry point with a workspace (oomb_select_pages), through the
C ABI: two calls in a row, the second with a smaller input (the scratch then still
holds the first call's values), with and without the diagnostic outputs. Selection is
bit-exact, so selections, counts, query summaries and scores must be equal bit for
bit."""
import pytest
import torch

import paged_chunk_attention_amd as pca
import workloads as wl
from tests.gpu_harness import DEV, bits, log

pytestmark = pytest.mark.gpu


def _case(name, hq, hkv, page, chunk, total, top_k, needles):
    w = wl.Workload(name, hq, hkv, 128, page, chunk, total, torch.bfloat16, top_k,
                    needles=needles)
    x = wl.make_inputs(w, device=DEV, with_grad=False)
    table = x["table"].to(DEV)
    pool = pca.PagedPool(w.pool_pages, page, w.d, hq, hkv, w.dtype, DEV, with_grad=False)
    pca.oomb_kv_append(pool, table, x["k"], x["v"], 0)
    pca.oomb_page_summarize(pool, table, 0, w.pages_per_head, w.total)
    return w, pool, table, x["q"]


def _select(w, pool, table, q, noalloc, diagnostics):
    n_cand = w.t0 // w.page
    k = max(1, min(w.top_k, n_cand))
    sel = torch.full((w.hkv, k), -7, dtype=torch.int32, device=DEV)
    count = torch.full((w.hkv,), -7, dtype=torch.int32, device=DEV)
    qbar = score = None
    if diagnostics:
        qbar = torch.full((w.hkv, w.d), float("nan"), dtype=torch.float32, device=DEV)
        score = torch.full((w.hkv, n_cand), float("nan"), dtype=torch.float32, device=DEV)
    if noalloc:
        pca.oomb_select_pages_noalloc(pool, table, q, w.t0, w.top_k, sel, count, qbar, score)
    else:
        pca.oomb_select_pages(pool, table, q, w.t0, w.top_k, sel=sel, count=count,
                              qbar_out=qbar, score_out=score)
    torch.cuda.synchronize()
    return sel.cpu(), count.cpu(), None if qbar is None else qbar.cpu(), \
        None if score is None else score.cpu()


def test_select_noalloc_matches_workspace_call_twice():
    cases = [
        # 4 KV heads x 4000 candidate pages, 7 x 1024 query rows per head
        ("large", 28, 4, 128, 1024, 128 * 4000 + 1024, 64, 16),
        # then a smaller one: fewer heads, pages, queries and k; ragged t0
        ("small", 8, 2, 64, 300, 64 * 700 + 13 + 300, 9, 4),
    ]
    for diagnostics in (False, True):
        for (name, *shape) in cases:
            log(f"[case select_noalloc {name} diagnostics={diagnostics}] {shape}")
            w, pool, table, q = _case(name, *shape)
            ref = _select(w, pool, table, q, noalloc=False, diagnostics=diagnostics)
            got = _select(w, pool, table, q, noalloc=True, diagnostics=diagnostics)
            assert torch.equal(got[1], ref[1]), "count"
            for g in range(w.hkv):
                n = int(ref[1][g])
                assert n == min(w.top_k, w.t0 // w.page)
                assert torch.equal(got[0][g, :n], ref[0][g, :n]), f"selection head {g}"
            if diagnostics:
                assert torch.equal(bits(got[2]), bits(ref[2])), "qbar"
                assert torch.equal(bits(got[3]), bits(ref[3])), "scores"
            log(f"    equal: {w.hkv} heads x {int(ref[1][0])} pages")
            del pool
            torch.cuda.empty_cache()


def test_select_noalloc_rejects_oversized_call():
    """A call whose workspace would exceed the static scratch is refused before any
    launch, leaving the outputs untouched."""
    w, pool, table, q = _case("small", 8, 2, 64, 300, 64 * 700 + 300, 9, 0)
    sel = torch.full((2, 9), -7, dtype=torch.int32, device=DEV)
    count = torch.full((2,), -7, dtype=torch.int32, device=DEV)
    # a 1,048,576-row query view (G * n_q = 4 * 262144) needs 2 * 16384 * 128 * 4 bytes
    # of partial sums alone, more than the 8 MiB scratch: refused on the host
    big_q = torch.zeros(8, 262144, 128, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(pca.OombError, match="static scratch"):
        pca.oomb_select_pages_noalloc(pool, table, big_q, w.t0, 9, sel, count)
    torch.cuda.synchronize()
    assert bool((sel == -7).all()) and bool((count == -7).all())
