"""GPU parity: the HIP library (through its C-ABI binding) against the CPU oracle,
element by element on identical seeded inputs, at sizes the oracle finishes in
seconds that still span several tiles and ragged tails.

Bars: bit-exact for pages, summaries, query summaries, scores and selections;
max-abs 2e-2 and relative-L2 1e-2 for bf16 outputs (O, dQ, dK, dV), 1e-5 for fp32.
"""
import numpy as np
import pytest
import torch

import oracle as orc
import paged_chunk_attention_amd as pca
import workloads as wl
from tests.gpu_harness import DEV, bits, compare, log, run_chunk_parity

pytestmark = pytest.mark.gpu


def _w(**kw):
    base = dict(name="case", hq=8, hkv=2, d=128, page=128, chunk=300, total=1300,
                dtype=torch.bfloat16, top_k=None, needles=0)
    base.update(kw)
    return wl.Workload(**base)


# matrix-core path: bf16, head_dim 128
@pytest.mark.parametrize("kw", [
    dict(name="mfma_dense_ragged"),                                   # t0=1000 straddles a page
    dict(name="mfma_sparse_k5", chunk=333, total=2597 + 333, top_k=5, needles=3),
    dict(name="mfma_gqa7_sparse", hq=28, hkv=4, chunk=256, total=1024 + 256, top_k=3),
    dict(name="mfma_page16_sparse", hq=4, hkv=2, page=16, chunk=200, total=500, top_k=6),
    dict(name="mfma_page32_dense", hq=6, hkv=3, page=32, chunk=130, total=130 + 517),
    dict(name="mfma_first_chunk", hq=4, hkv=1, chunk=200, total=200),  # t0 = 0
    dict(name="mfma_single_query", hq=4, hkv=2, chunk=1, total=777),
    dict(name="mfma_k0_local_only", hq=4, hkv=2, chunk=128, total=1024, top_k=0),
    dict(name="mfma_k_exceeds", hq=4, hkv=2, chunk=64, total=640, top_k=50),
    # pages of 64 (a key block of 64 is one page) and 256 (a page spans four key blocks)
    dict(name="mfma_page64_dense", hq=4, hkv=2, page=64, chunk=160, total=160 + 900),
    dict(name="mfma_page256_sparse", hq=8, hkv=2, page=256, chunk=300, total=300 + 2600, top_k=4),
    dict(name="mfma_no_gqa", hq=4, hkv=4, chunk=200, total=200 + 900, top_k=3),  # G = 1
])
def test_chunk_parity_mfma(kw):
    run_chunk_parity(_w(**kw))


def test_chunk_parity_mfma_page_window_slides():
    """More attended pages than the kernels keep resident: 8,208 pages of 16 tokens per
    head, so the forward's page-id window (2,048 when a head attends over 8,192 pages)
    and the dQ pass's window slide several times within one workgroup."""
    run_chunk_parity(_w(name="mfma_window_slide", hq=4, hkv=1, page=16, chunk=256,
                        total=16 * 8192 + 256))


@pytest.mark.parametrize("n", [1, 2, 3])
@pytest.mark.parametrize("kw", [
    dict(name="mfma_sparse_k5", chunk=333, total=2597 + 333, top_k=5, needles=3),
    dict(name="mfma_window_slide", hq=4, hkv=1, page=16, chunk=256, total=16 * 8192 + 256),
])
def test_chunk_parity_mfma_fixed_splits(kw, n, monkeypatch):
    """The split counts fixed through the environment: 1 (forward and dQ tiles whole,
    dK/dV query stream unsplit), 2 and 3 (ranges of unequal length): every path of the
    forward, dQ and dK/dV passes and their merges, at sizes whose own choice differs."""
    for var in ("OOMB_FWD_SPLITS", "OOMB_DQ_SPLITS", "OOMB_DKDV_SPLITS"):
        monkeypatch.setenv(var, str(n))
    run_chunk_parity(_w(**dict(kw, name=f"{kw['name']}_splits{n}")))


@pytest.mark.parametrize("kw", [
    dict(name="mfma_nan_page0_dense"),
    dict(name="mfma_nan_page0_sparse", chunk=333, total=2597 + 333, top_k=5, needles=3),
    # pages of 16: every staging instruction reads its own page id (the per-instruction path)
    dict(name="mfma_nan_page0_p16", hq=4, hkv=2, page=16, chunk=200, total=900, top_k=6),
])
def test_padding_rows_come_from_zeros(kw):
    """Physical page 0 is never mapped and holds NaN: the rows staged for block tails,
    slots past the end of the sequence and invalid pages come from zeros, not from the
    pool, so nothing the attention does not attend reaches a result (a masked P of 0
    times a NaN row would be NaN)."""
    w = _w(**kw)
    x = wl.make_inputs(w)
    x["table"] = x["table"] + 1      # pages 1 .. N; page 0 keeps the NaN sentinel
    x["gtable"] = x["gtable"] + 1
    run_chunk_parity(w, x)


def test_padding_rows_come_from_zeros_recomputing_dq(monkeypatch):
    """The same NaN sentinel with the dS spill off, so the dQ pass recomputes S and dP and
    stages its own blocks of 128 keys (one page id per block with pages of 128; the block
    holding the sequence's end takes the per-row path): its padding rows come from zeros
    too."""
    monkeypatch.setenv("OOMB_DS_SPILL_MAX_MIB", "0")
    w = _w(name="mfma_nan_page0_recompute", chunk=333, total=2597 + 333, top_k=5, needles=3)
    x = wl.make_inputs(w)
    x["table"] = x["table"] + 1
    x["gtable"] = x["gtable"] + 1
    run_chunk_parity(w, x)


@pytest.mark.parametrize("n,whole", [(3, 5), (2, 13), (4, 14)])
@pytest.mark.parametrize("kw", [
    dict(name="mfma_gqa7_mixed_sparse", hq=28, hkv=4, chunk=333, total=2597 + 333, top_k=5, needles=3),
    dict(name="mfma_gqa7_mixed_window", hq=28, hkv=4, chunk=333, total=2597 + 333, window=300),
])
def test_chunk_parity_mfma_mixed_plans(kw, n, whole, monkeypatch):
    """Mixed split plans fixed through the environment: per KV head the first `whole`
    of its 14 query tiles (longest first) run whole and write O and dQ directly, the
    rest as n key ranges merged in order (whole = 14: every tile whole although the
    partials are laid out), so the merges must leave the whole tiles' rows alone. The
    dK/dV pass likewise: its first `whole` key blocks (of 8 with the selection, 23 with
    the window) add into the pool directly, the others' query streams in n parts."""
    for var, val in (("OOMB_FWD_SPLITS", n), ("OOMB_DQ_SPLITS", n), ("OOMB_DKDV_SPLITS", n),
                     ("OOMB_FWD_WHOLE", whole), ("OOMB_DQ_WHOLE", whole),
                     ("OOMB_DKDV_WHOLE", whole)):
        monkeypatch.setenv(var, str(val))
    run_chunk_parity(_w(**dict(kw, name=f"{kw['name']}_n{n}_w{whole}")))


# local attention (the sparse layers of sparse-native models): a window of W positions
@pytest.mark.parametrize("kw", [
    dict(name="mfma_window5", window=5),                              # inside one key block
    dict(name="mfma_window64", window=64),
    dict(name="mfma_window200_prior", window=200),                    # reaches the prior pages
    dict(name="mfma_window777_gqa7", hq=28, hkv=4, chunk=256, total=2000 + 256, window=777),
    dict(name="mfma_window_over_all", window=1 << 20),                # equals no window
    dict(name="mfma_window_first_chunk", hq=4, hkv=1, chunk=200, total=200, window=50),
    dict(name="mfma_window_page16", hq=4, hkv=2, page=16, chunk=200, total=900, window=130),
])
def test_chunk_parity_mfma_window(kw):
    run_chunk_parity(_w(**kw))


@pytest.mark.parametrize("n", [1, 3])
def test_chunk_parity_mfma_window_fixed_splits(n, monkeypatch):
    """Windows with the split counts fixed: key ranges that start past block 0."""
    for var in ("OOMB_FWD_SPLITS", "OOMB_DQ_SPLITS", "OOMB_DKDV_SPLITS"):
        monkeypatch.setenv(var, str(n))
    run_chunk_parity(_w(name=f"mfma_window300_splits{n}", chunk=333, total=2597 + 333, window=300))


# scalar path: fp32 (any head_dim) and bf16 head_dim 64
@pytest.mark.parametrize("kw", [
    dict(name="f32_d64_p16", hq=2, hkv=1, d=64, page=16, chunk=64, total=1024, dtype=torch.float32),
    dict(name="f32_d128_sparse", hq=4, hkv=2, d=128, page=32, chunk=70, total=70 + 300,
         dtype=torch.float32, top_k=4),
    dict(name="bf16_d64_dense", hq=4, hkv=1, d=64, page=64, chunk=100, total=300),
    dict(name="bf16_d64_sparse", hq=6, hkv=2, d=64, page=16, chunk=50, total=50 + 400, top_k=7),
    dict(name="f32_d64_window", hq=2, hkv=1, d=64, page=16, chunk=64, total=1024, window=40,
         dtype=torch.float32),
    dict(name="bf16_d64_window", hq=4, hkv=1, d=64, page=64, chunk=100, total=300, window=150),
    # the largest page size, a ragged chunk, rows whose keys take several rounds of the
    # workgroup's four waves (64 keys each)
    dict(name="f32_d128_p256_ragged", hq=2, hkv=1, d=128, page=256, chunk=77, total=77 + 1500,
         dtype=torch.float32),
    # a one-query chunk: one workgroup per head, two of its four waves without keys
    dict(name="f32_d64_one_query", hq=2, hkv=1, d=64, page=16, chunk=1, total=1 + 100,
         dtype=torch.float32),
    dict(name="bf16_d64_p256_sparse", hq=6, hkv=2, d=64, page=256, chunk=130, total=130 + 2600,
         top_k=3),
])
def test_chunk_parity_scalar(kw):
    run_chunk_parity(_w(**kw))


def test_selection_ties_break_to_lower_id():
    """Pages with identical keys score identically; the lower logical ids win."""
    w = _w(name="ties", hq=4, hkv=1, chunk=128, total=128 * 12 + 128, top_k=4)
    x = wl.make_inputs(w)
    k = x["k"].clone()
    for j in (2, 5, 6, 9, 10):
        k[:, j * 128:(j + 1) * 128] = k[:, 3 * 128:4 * 128]
    x["k"] = k
    run_chunk_parity(w, x)


def test_results_independent_of_page_placement():
    """Two different physical placements give bit-identical O, LSE, dQ and
    selections, and the same gradient rows after mapping pages back."""
    import paged_chunk_attention_amd as pca
    w = _w(name="placement", hq=8, hkv=2, chunk=256, total=256 + 1100, top_k=4)
    x = wl.make_inputs(w)
    outs = []
    for seed in (5, 50):
        perm = torch.randperm(w.pool_pages, generator=torch.Generator().manual_seed(seed))
        table = perm.to(torch.int32).reshape(w.hkv, -1).to(DEV)
        pool = pca.PagedPool(w.pool_pages, w.page, w.d, w.hq, w.hkv, w.dtype, DEV)
        log(f"[case placement seed={seed}]")
        pca.oomb_kv_append(pool, table, x["k"].to(DEV), x["v"].to(DEV), 0)
        pca.oomb_page_summarize(pool, table, 0, w.pages_per_head, w.total)
        q, do = x["q"].to(DEV), x["do"].to(DEV)
        sel, cnt = pca.oomb_select_pages(pool, table, q, w.t0, w.top_k)
        o, lse = pca.oomb_paged_chunk_attn_fwd(pool, table, q, w.t0, sel, cnt)
        dq = pca.oomb_paged_chunk_attn_bwd(pool, table, table, q, w.t0, sel, cnt, o, do, lse)
        torch.cuda.synchronize()
        idx = table.long()
        dk = pool.dk[idx].reshape(w.hkv, -1, w.d).cpu()
        outs.append((sel.cpu(), bits(o), lse.cpu(), dq.cpu(), dk))
    a, b = outs
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert torch.equal(a[2], b[2]) and torch.equal(a[3], b[3]) and torch.equal(a[4], b[4])


def test_backward_deterministic_run_twice():
    """dK/dV are written by exclusive owners (no atomics): two runs agree bitwise."""
    import paged_chunk_attention_amd as pca
    w = _w(name="determinism", hq=8, hkv=2, chunk=300, total=2000, top_k=6)
    x = wl.make_inputs(w)
    table = x["table"].to(DEV)
    pool = pca.PagedPool(w.pool_pages, w.page, w.d, w.hq, w.hkv, w.dtype, DEV)
    log("[case determinism]")
    pca.oomb_kv_append(pool, table, x["k"].to(DEV), x["v"].to(DEV), 0)
    pca.oomb_page_summarize(pool, table, 0, w.pages_per_head, w.total)
    q, do = x["q"].to(DEV), x["do"].to(DEV)
    sel, cnt = pca.oomb_select_pages(pool, table, q, w.t0, w.top_k)
    o, lse = pca.oomb_paged_chunk_attn_fwd(pool, table, q, w.t0, sel, cnt)
    res = []
    for _ in range(2):
        pool.zero_grad()
        dq = pca.oomb_paged_chunk_attn_bwd(pool, table, table, q, w.t0, sel, cnt, o, do, lse)
        torch.cuda.synchronize()
        res.append((dq.cpu(), pool.dk.cpu(), pool.dv.cpu()))
    for a, b in zip(*res):
        assert torch.equal(a, b)


@pytest.mark.parametrize("kw", [
    dict(name="mfma_dense_ragged"),
    dict(name="mfma_sparse_k5", chunk=333, total=2597 + 333, top_k=5, needles=3),
    dict(name="mfma_window_slide", hq=4, hkv=1, page=16, chunk=256, total=16 * 8192 + 256),
])
def test_chunk_parity_mfma_recomputed_dq(kw, monkeypatch):
    """With the dS spill turned off the dQ pass recomputes S and dP (the path of windowed
    calls and of workspaces beyond the spill's limit): the same bars."""
    monkeypatch.setenv("OOMB_DS_SPILL_MAX_MIB", "0")
    run_chunk_parity(_w(**dict(kw, name=f"{kw['name']}_recompute")))


@pytest.mark.parametrize("kw", [
    dict(name="spill_sparse", hq=8, hkv=2, chunk=300, total=2000, top_k=6),
    dict(name="spill_dense_gqa7", hq=28, hkv=4, chunk=333, total=1700),
])
def test_ds_spill_matches_recompute(kw, monkeypatch):
    """The backward with the dS spill and without: dK/dV bit for bit (the dK/dV pass does
    the same arithmetic, the spill only stores its dS), dQ within the bf16 bar of each
    other (the spilled dS is formed from the fp16 P the dK/dV pass exchanges, the
    recomputed one from an fp32 P)."""
    w = _w(**kw)
    x = wl.make_inputs(w)
    table = x["table"].to(DEV)
    pool = pca.PagedPool(w.pool_pages, w.page, w.d, w.hq, w.hkv, w.dtype, DEV)
    log(f"[case {w.name}] spill on / off")
    pca.oomb_kv_append(pool, table, x["k"].to(DEV), x["v"].to(DEV), 0)
    pca.oomb_page_summarize(pool, table, 0, w.pages_per_head, w.total)
    q, do = x["q"].to(DEV), x["do"].to(DEV)
    sel = cnt = None
    if w.top_k is not None:
        sel, cnt = pca.oomb_select_pages(pool, table, q, w.t0, w.top_k)
    o, lse = pca.oomb_paged_chunk_attn_fwd(pool, table, q, w.t0, sel, cnt)
    res = []
    for limit in (None, "0"):
        if limit is None:
            monkeypatch.delenv("OOMB_DS_SPILL_MAX_MIB", raising=False)
        else:
            monkeypatch.setenv("OOMB_DS_SPILL_MAX_MIB", limit)
        pool.zero_grad()
        dq = pca.oomb_paged_chunk_attn_bwd(pool, table, table, q, w.t0, sel, cnt, o, do, lse)
        torch.cuda.synchronize()
        res.append((dq.cpu(), pool.dk.cpu(), pool.dv.cpu()))
    assert torch.equal(res[0][1], res[1][1]) and torch.equal(res[0][2], res[1][2])
    compare("dQ spill vs recompute", res[0][0], res[1][0].double(), w.dtype)


def test_strided_views_match_contiguous():
    """[C, H, D] storage (token-major) gives the same results as [H, C, D]."""
    import paged_chunk_attention_amd as pca
    w = _w(name="strided", hq=8, hkv=2, chunk=192, total=192 + 640, top_k=2)
    x = wl.make_inputs(w)
    table = x["table"].to(DEV)
    pool = pca.PagedPool(w.pool_pages, w.page, w.d, w.hq, w.hkv, w.dtype, DEV)
    log("[case strided]")
    kt = x["k"].transpose(0, 1).contiguous().to(DEV).transpose(0, 1)
    vt = x["v"].transpose(0, 1).contiguous().to(DEV).transpose(0, 1)
    pca.oomb_kv_append(pool, table, kt, vt, 0)
    pca.oomb_page_summarize(pool, table, 0, w.pages_per_head, w.total)
    q = x["q"].to(DEV)
    do = x["do"].to(DEV)
    qt = x["q"].transpose(0, 1).contiguous().to(DEV).transpose(0, 1)
    dot = x["do"].transpose(0, 1).contiguous().to(DEV).transpose(0, 1)
    s1, c1 = pca.oomb_select_pages(pool, table, q, w.t0, w.top_k)
    s2, c2 = pca.oomb_select_pages(pool, table, qt, w.t0, w.top_k)
    o1, l1 = pca.oomb_paged_chunk_attn_fwd(pool, table, q, w.t0, s1, c1)
    o2 = torch.empty(w.chunk, w.hq, w.d, dtype=w.dtype, device=DEV).transpose(0, 1)
    o2, l2 = pca.oomb_paged_chunk_attn_fwd(pool, table, qt, w.t0, s2, c2, o=o2)
    d1 = pca.oomb_paged_chunk_attn_bwd(pool, table, table, q, w.t0, s1, c1, o1, do, l1)
    d2 = pca.oomb_paged_chunk_attn_bwd(pool, table, table, qt, w.t0, s2, c2, o2, dot, l2)
    torch.cuda.synchronize()
    assert torch.equal(s1, s2) and torch.equal(c1, c2)
    assert torch.equal(bits(o1), bits(o2.contiguous())) and torch.equal(l1, l2)
    assert torch.equal(d1, d2)


# selector variant: mean-key page representatives
@pytest.mark.parametrize("kw", [
    dict(name="mean_sel_k5", chunk=333, total=2597 + 333, top_k=5, needles=3),
    dict(name="mean_sel_page16", hq=4, hkv=2, page=16, chunk=200, total=900, top_k=6),
    dict(name="mean_sel_f32", hq=4, hkv=2, page=32, chunk=70, total=70 + 300, top_k=4,
         dtype=torch.float32),
    dict(name="mean_sel_d64", hq=6, hkv=2, d=64, page=16, chunk=50, total=50 + 400, top_k=7),
])
def test_mean_selector_bit_exact(kw):
    """Mean-key summaries bit-exact on every page written (NaN sentinels elsewhere
    untouched), then query summary, scores and selection bit-exact against the oracle,
    and the forward with that selection within the bar."""
    from tests.gpu_harness import GpuLayer, oracle_layer
    w = _w(**kw)
    x = wl.make_inputs(w)
    t0, C, P = w.t0, w.chunk, w.page
    log(f"[case {w.name}] mean-key selector hq={w.hq} hkv={w.hkv} d={w.d} page={P} t0={t0} "
        f"top_k={w.top_k} dtype={w.dtype}")
    L = GpuLayer(w, x)
    L.append(x["k"][:, :t0 + C], x["v"][:, :t0 + C], 0)
    n_pages = -(-(t0 + C) // P)
    N = L.pool.k.shape[0]
    kmean = torch.full((N, w.d), float("nan"), dtype=torch.float32, device=DEV)
    pca.oomb_page_summarize_mean(L.pool, L.table, 0, n_pages, t0 + C, kmean)
    q = x["q"].to(DEV)
    n_cand = t0 // P
    qbar = torch.empty(w.hkv, w.d, dtype=torch.float32, device=DEV)
    score = torch.empty(w.hkv, max(n_cand, 1), dtype=torch.float32, device=DEV)
    sel, count = pca.oomb_select_pages_mean(L.pool, L.table, q, t0, w.top_k, kmean, qbar_out=qbar,
                                            score_out=score)
    o, lse = pca.oomb_paged_chunk_attn_fwd(L.pool, L.table, q, t0, sel, count, w.scale)
    torch.cuda.synchronize()

    kp, vp, _ = oracle_layer(w, x, t0 + C)
    ref_mean = np.full((kp.shape[0], w.d), np.nan, np.float32)
    orc.summarize_mean(kp, x["table"], ref_mean, 0, n_pages, t0 + C)
    got_mean = kmean.cpu().numpy()[:kp.shape[0]]
    assert np.array_equal(got_mean.view(np.int32), ref_mean.view(np.int32)), "mean summaries differ"
    ref = orc.select_pages_mean(x["q"], ref_mean, x["table"], t0, P, w.group, w.top_k)
    osel = []
    for g, (qb, sc, chosen) in enumerate(ref):
        assert torch.equal(bits(qbar[g]), torch.from_numpy(qb).view(torch.int32)), f"qbar head {g}"
        assert torch.equal(bits(score[g, :n_cand]), torch.from_numpy(sc).view(torch.int32)), \
            f"scores head {g}"
        assert int(count[g]) == len(chosen) and sel[g, :len(chosen)].tolist() == chosen, f"head {g}"
        osel.append(chosen)
    log(f"    mean summaries + selection bit-exact ({[len(s) for s in osel]} pages per head)")
    O, _ = orc.fwd(x["q"], kp, vp, x["table"], t0, osel, w.scale)
    compare("O", o, O, w.dtype)


def _score_bits_equal(got: torch.Tensor, ref: np.ndarray) -> bool:
    """Bit equality of fp32 scores, NaN matching any NaN (its sign and payload are the
    arithmetic unit's choice, not part of the definition)."""
    g = got.cpu().numpy()
    nan_g, nan_r = np.isnan(g), np.isnan(ref)
    if not np.array_equal(nan_g, nan_r):
        return False
    return np.array_equal(g[~nan_g].view(np.int32), ref[~nan_r].view(np.int32))


def test_selection_signed_zero_inf_nan_scores():
    """Scores of exactly +0 and -0 (all-zero keys, and zero keys signed against qbar so
    that every product is -0) tie with each other and break to the lower logical id;
    +inf ranks first, -inf below every number, NaN (keys with infinities of both signs)
    below -inf with NaNs tied by id. qbar, every score and the selection against the
    oracle, for several k around those boundaries."""
    P, D = 128, 128
    w = _w(name="score_edges", hq=4, hkv=1, chunk=128, total=128 * 20 + 128)
    x = wl.make_inputs(w)
    qbar = orc.query_summary(x["q"], 0, w.group)
    sgn = torch.from_numpy(np.sign(qbar).astype(np.float32))
    assert bool((sgn != 0).all())
    k = x["k"].clone().float()
    pg = lambda j: slice(j * P, (j + 1) * P)          # noqa: E731
    for j, c in ((0, 0.01), (1, 0.02), (3, 0.03)):    # negative scores: -c * sum|qbar|
        k[0, pg(j)] = -c * sgn
    for j in (2, 7, 13):                               # all +0 keys: products +-0
        k[0, pg(j)] = 0.0
    for j in (4, 11):                                  # keys of sign -sgn: every product -0
        k[0, pg(j)] = torch.where(sgn > 0, torch.tensor(-0.0), torch.tensor(0.0))
    k[0, pg(8), 0] = float("inf") * sgn[0]             # +inf score
    k[0, pg(9), 0] = -float("inf") * sgn[0]            # -inf score
    for j in (5, 16):                                  # +inf in one dim, -inf in another: NaN
        k[0, pg(j), 0] = float("inf") * sgn[0]
        k[0, pg(j), 1] = -float("inf") * sgn[1]
    x["k"] = k.to(w.dtype)
    table = x["table"].to(DEV)
    pool = pca.PagedPool(w.pool_pages, P, D, w.hq, w.hkv, w.dtype, DEV)
    pca.oomb_kv_append(pool, table, x["k"].to(DEV), x["v"].to(DEV), 0)
    pca.oomb_page_summarize(pool, table, 0, w.pages_per_head, w.total)
    kp = torch.zeros(w.pool_pages, P, D, dtype=w.dtype)
    orc.append(kp, x["table"], x["k"], 0)
    summ = torch.zeros(w.pool_pages, 2, D, dtype=w.dtype)
    orc.summarize(kp, x["table"], summ, 0, w.pages_per_head, w.total)
    q = x["q"].to(DEV)
    for top_k in (1, 9, 10, 11, 12, 15, 17, 18, 19, 20):
        log(f"[case score_edges k={top_k}]")
        qb = torch.empty(1, D, dtype=torch.float32, device=DEV)
        sc = torch.empty(1, 20, dtype=torch.float32, device=DEV)
        sel, cnt = pca.oomb_select_pages(pool, table, q, w.t0, top_k, qbar_out=qb, score_out=sc)
        torch.cuda.synchronize()
        (rq, rs, chosen), = orc.select_pages(x["q"], summ, x["table"], w.t0, P, w.group, top_k)
        assert torch.equal(bits(qb[0]), torch.from_numpy(rq).view(torch.int32))
        assert _score_bits_equal(sc[0], rs)
        assert int(cnt[0]) == len(chosen) and sel[0, :len(chosen)].cpu().tolist() == chosen
        if top_k == 12:   # +inf, the 8 positive pages, then 3 of the 5 tied zero pages
            assert chosen == sorted([8, 6, 10, 12, 14, 15, 17, 18, 19, 2, 4, 7]), chosen
            assert np.signbit(rs[4]) and rs[4] == 0 and rs[2] == 0
        if top_k == 19:   # everything but the higher-id NaN page
            assert chosen == [j for j in range(20) if j != 16]


def test_side_stream_calls_match_default_stream():
    """Select, forward and backward issued on a second stream (outputs, workspaces and
    their fills made by the binding on that stream) give the default stream's results
    bit for bit."""
    w = _w(name="side_stream", hq=8, hkv=2, chunk=300, total=2000, top_k=6)
    x = wl.make_inputs(w)
    table = x["table"].to(DEV)
    q, do = x["q"].to(DEV), x["do"].to(DEV)
    outs = []
    for use_side in (False, True):
        log(f"[case side_stream {use_side}]")
        pool = pca.PagedPool(w.pool_pages, w.page, w.d, w.hq, w.hkv, w.dtype, DEV)
        pca.oomb_kv_append(pool, table, x["k"].to(DEV), x["v"].to(DEV), 0)
        pca.oomb_page_summarize(pool, table, 0, w.pages_per_head, w.total)
        st = torch.cuda.Stream() if use_side else None
        if st is not None:
            st.wait_stream(torch.cuda.current_stream())
        sel, cnt = pca.oomb_select_pages(pool, table, q, w.t0, w.top_k, stream=st)
        o, lse = pca.oomb_paged_chunk_attn_fwd(pool, table, q, w.t0, sel, cnt, stream=st)
        dq = pca.oomb_paged_chunk_attn_bwd(pool, table, table, q, w.t0, sel, cnt, o, do, lse,
                                           stream=st)
        torch.cuda.synchronize()
        outs.append((sel.cpu(), bits(o), lse.cpu(), dq.cpu(), pool.dk.cpu(), pool.dv.cpu()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def _tiled_case(name, hq, hkv, page, chunk, t0, top_k, needles=0):
    w = _w(name=name, hq=hq, hkv=hkv, page=page, chunk=chunk, total=t0 + chunk, top_k=top_k,
           needles=needles)
    x = wl.make_inputs(w)
    table = x["table"].to(DEV)
    pool = pca.PagedPool(w.pool_pages, page, w.d, hq, hkv, w.dtype, DEV)
    pca.oomb_kv_append(pool, table, x["k"].to(DEV), x["v"].to(DEV), 0)
    pca.oomb_page_summarize(pool, table, 0, w.pages_per_head, w.total)
    kp = torch.zeros(w.pool_pages, page, w.d, dtype=w.dtype)
    vp = torch.zeros_like(kp)
    orc.append(kp, x["table"], x["k"], 0)
    orc.append(vp, x["table"], x["v"], 0)
    summ = torch.zeros(w.pool_pages, 2, w.d, dtype=w.dtype)
    orc.summarize(kp, x["table"], summ, 0, w.pages_per_head, w.total)
    return w, x, pool, table, kp, vp, summ


@pytest.mark.parametrize("kw", [
    dict(name="tiles_aligned", hq=8, hkv=2, page=64, chunk=512, t0=64 * 30, top_k=4, tile=128),
    dict(name="tiles_ragged", hq=8, hkv=2, page=64, chunk=500, t0=64 * 30 + 17, top_k=5, tile=100),
    dict(name="tiles_gqa7", hq=28, hkv=4, page=128, chunk=1024, t0=128 * 40, top_k=6, tile=256,
         needles=5),
    dict(name="tiles_k_exceeds", hq=4, hkv=1, page=32, chunk=96, t0=32 * 5, top_k=9, tile=40),
])
def test_tiled_selection_bit_exact(kw):
    """Per-query-tile selection: every tile's qbar, scores and selection row (its top-k
    ids, then the chunk's pages before the tile) and count against the oracle, bit for
    bit; tiles not a multiple of the page size, a ragged last tile, k above the
    candidate count."""
    kw = dict(kw)
    tile = kw.pop("tile")
    w, x, pool, table, kp, vp, summ = _tiled_case(**kw)
    log(f"[case {w.name}] t0={w.t0} chunk={w.chunk} tile={tile} top_k={w.top_k}")
    n_tiles = -(-w.chunk // tile)
    n_cand = w.t0 // w.page
    qb = torch.empty(n_tiles, w.hkv, w.d, dtype=torch.float32, device=DEV)
    sc = torch.empty(n_tiles, w.hkv, max(1, n_cand), dtype=torch.float32, device=DEV)
    sel, cnt = pca.oomb_select_pages_tiled(pool, table, x["q"].to(DEV), w.t0, w.top_k, tile,
                                           qbar_out=qb, score_out=sc)
    torch.cuda.synchronize()
    ref = orc.select_pages_tiled(x["q"], summ, x["table"], w.t0, w.page, w.group, w.top_k, tile)
    sel, cnt, qb, sc = sel.cpu(), cnt.cpu(), qb.cpu(), sc.cpu()
    for g in range(w.hkv):
        for j in range(n_tiles):
            rq, rs, chosen = ref[g][j]
            assert torch.equal(bits(qb[j, g]), torch.from_numpy(rq).view(torch.int32)), (g, j)
            assert torch.equal(bits(sc[j, g, :n_cand]), torch.from_numpy(rs).view(torch.int32)), (g, j)
            row = orc.tile_selection_row(chosen, w.t0, w.page, tile, j)
            assert int(cnt[j, g]) == len(row) and sel[j, g, :len(row)].tolist() == row, (g, j)
    log(f"    {n_tiles} tiles x {w.hkv} heads bit-exact")


def test_tiled_selection_one_tile_is_select_pages():
    """A tile at least as long as the chunk gives oomb_select_pages' results bit for bit."""
    w, x, pool, table, kp, vp, summ = _tiled_case("one_tile", 8, 2, 64, 300, 64 * 20, 4)
    q = x["q"].to(DEV)
    a_sel, a_cnt = pca.oomb_select_pages(pool, table, q, w.t0, w.top_k)
    for tile in (300, 1000):
        b_sel, b_cnt = pca.oomb_select_pages_tiled(pool, table, q, w.t0, w.top_k, tile)
        torch.cuda.synchronize()
        assert b_sel.shape[0] == 1
        assert torch.equal(a_cnt.cpu(), b_cnt[0].cpu()) and torch.equal(a_sel.cpu(), b_sel[0].cpu())


@pytest.mark.parametrize("kw", [
    dict(name="tiled_attn", hq=8, hkv=2, page=64, chunk=500, t0=64 * 30 + 17, top_k=5, tile=128),
    dict(name="tiled_attn_gqa7", hq=28, hkv=4, page=128, chunk=768, t0=128 * 24, top_k=4, tile=256),
])
def test_tiled_attention_matches_oracle(kw):
    """Attention with per-tile selections (one forward / backward call per tile) against
    the oracle's tiled attention over its own tiled selection: O, LSE, dQ, and dK/dV
    accumulated over the tiles, at the bf16 bar."""
    kw = dict(kw)
    tile = kw.pop("tile")
    w, x, pool, table, kp, vp, summ = _tiled_case(**kw)
    log(f"[case {w.name}] t0={w.t0} chunk={w.chunk} tile={tile} top_k={w.top_k}")
    q, do = x["q"].to(DEV), x["do"].to(DEV)
    gtable = x["gtable"].to(DEV)
    sel, cnt = pca.oomb_select_pages_tiled(pool, table, q, w.t0, w.top_k, tile)
    o, lses = pca.oomb_paged_chunk_attn_fwd_tiled(pool, table, q, w.t0, sel, cnt, tile)
    dq = pca.oomb_paged_chunk_attn_bwd_tiled(pool, table, gtable, q, w.t0, sel, cnt, tile, o, do,
                                             lses)
    torch.cuda.synchronize()
    ref = orc.select_pages_tiled(x["q"], summ, x["table"], w.t0, w.page, w.group, w.top_k, tile)
    chosen = [[ch for (_, _, ch) in ref[g]] for g in range(w.hkv)]
    O, L = orc.fwd_tiled(x["q"], kp, vp, x["table"], w.t0, chosen, w.scale, tile)
    gk = torch.zeros(kp.shape, dtype=torch.float64)
    gv = torch.zeros(kp.shape, dtype=torch.float64)
    dQ = orc.bwd_tiled(x["q"], kp, vp, x["table"], w.t0, chosen, w.scale, tile, x["do"], gk, gv,
                       x["gtable"])
    compare("O", o, O, w.dtype)
    lse = torch.cat([t.cpu() for t in lses], dim=1)
    assert (lse.double() - L).abs().max().item() <= 1e-2
    compare("dQ", dq, dQ, w.dtype)
    mapped = x["gtable"].reshape(-1).long()
    compare("dK", pool.dk.cpu()[mapped], gk[mapped], w.dtype)
    compare("dV", pool.dv.cpu()[mapped], gv[mapped], w.dtype)
