"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test states the fact it checks: a library routine computing the same quantity
by another route (torch SDPA with autograd, torch.amin/amax), finite differences,
closed forms, hand-derived fp32 values (tests/golden/), brute-force order
statistics, and invariances the definition implies.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle as orc
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
F64 = torch.float64


# ----------------------------------------------------------------------------- helpers

def _rand(shape, seed, dtype=F64):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32).to(dtype)


def _build(k, v, P, table, n_pool):
    """Pool holding tokens [0, T) of k/v [hkv, T, D] at the given table."""
    hkv, T, D = k.shape
    kp = torch.full((n_pool, P, D), float("nan"), dtype=k.dtype)
    vp = torch.full((n_pool, P, D), float("nan"), dtype=v.dtype)
    orc.append(kp, table, k, 0)
    orc.append(vp, table, v, 0)
    return kp, vp


def _table(hkv, n_pages, seed):
    return torch.randperm(hkv * n_pages, generator=torch.Generator().manual_seed(seed)) \
        .to(torch.int32).reshape(hkv, n_pages)


def _sdpa(q, k, v, t0, pages_per_head, P, scale, window=0):
    """torch SDPA in fp64 with GQA and an explicit boolean mask: query i (position
    t0+i) of q head h sees key t iff page(t) is attended by head h // G and t <= t0+i
    (and, with a window W, t > t0+i-W). Returns O, and grads wrt q, k, v of
    sum(dO * O) via autograd (dO passed later)."""
    hq, C, D = q.shape
    hkv, T, _ = k.shape
    G = hq // hkv
    mask = torch.zeros(hq, C, T, dtype=torch.bool)
    qpos = t0 + torch.arange(C)
    kpos = torch.arange(T)
    for h in range(hq):
        allowed = torch.zeros(T, dtype=torch.bool)
        for j in pages_per_head[h // G]:
            allowed[j * P:(j + 1) * P] = True
        mask[h] = allowed[None, :] & (kpos[None, :] <= qpos[:, None])
        if window:
            mask[h] &= kpos[None, :] > qpos[:, None] - window
    return F.scaled_dot_product_attention(q[None], k[None], v[None], attn_mask=mask[None],
                                          scale=scale, enable_gqa=True)[0]


# ----------------------------------------------------------------------------- paging

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_append_gather_roundtrip_bitwise(dtype):
    """Appending in unaligned pieces then gathering returns the input bit for bit,
    and every slot outside the written tokens keeps its sentinel."""
    hkv, T, D, P = 2, 100, 8, 16
    n_pages = -(-T // P)
    table = _table(hkv, n_pages, 3)
    n_pool = hkv * n_pages + 5
    k = _rand((hkv, T, D), 1, dtype)
    pool = torch.full((n_pool, P, D), 7.25, dtype=dtype)
    for a, b in [(0, 13), (13, 16), (16, 70), (70, 100)]:
        orc.append(pool, table, k[:, a:b], a)
    for g in range(hkv):
        back = orc.gather(pool, table, g, range(n_pages))[:T]
        assert torch.equal(back.view(torch.int16 if dtype == torch.bfloat16 else torch.int32),
                           k[g].view(torch.int16 if dtype == torch.bfloat16 else torch.int32))
    written = torch.zeros(n_pool, P, dtype=torch.bool)
    for g in range(hkv):
        t = torch.arange(T)
        written[table[g].long()[t // P], t % P] = True
    assert bool((pool[~written] == 7.25).all())


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_summarize_equals_amin_amax(dtype):
    """Summary values equal torch.amin/amax over each page's valid tokens (a partial
    last page included); pages past seq_len are untouched."""
    hkv, T, D, P = 2, 75, 16, 16
    n_pages = 6
    table = _table(hkv, n_pages, 4)
    k = _rand((hkv, T, D), 2, dtype)
    pool = torch.zeros(hkv * n_pages, P, D, dtype=dtype)
    orc.append(pool, table, k, 0)
    summ = torch.full((hkv * n_pages, 2, D), 99.0, dtype=dtype)
    orc.summarize(pool, table, summ, 0, n_pages, T)
    for g in range(hkv):
        for j in range(n_pages):
            phys = int(table[g, j])
            tok = k[g, j * P:min(T, (j + 1) * P)]
            if len(tok) == 0:
                assert bool((summ[phys] == 99.0).all())
                continue
            assert torch.equal(summ[phys, 0], tok.amin(0))
            assert torch.equal(summ[phys, 1], tok.amax(0))


def test_summarize_signed_zero_rule():
    """min/max follow the total order with -0 < +0, independent of token order."""
    P, D = 4, 2
    for order in ([0.0, -0.0, 1.0, -1.0], [-0.0, 0.0, -1.0, 1.0]):
        page = torch.tensor(order, dtype=torch.float32)[:, None].repeat(1, D)
        page[:, 1] = torch.tensor([0.0, -0.0, 0.0, -0.0]) if order[0] == 0.0 else \
            torch.tensor([-0.0, 0.0, -0.0, 0.0])
        pool = page[None].clone()
        table = torch.zeros(1, 1, dtype=torch.int32)
        summ = torch.zeros(1, 2, D)
        orc.summarize(pool, table, summ, 0, 1, P)
        assert summ[0, 0, 0].item() == -1.0 and summ[0, 1, 0].item() == 1.0
        assert math.copysign(1.0, summ[0, 0, 1].item()) == -1.0   # min of {+0,-0} is -0
        assert math.copysign(1.0, summ[0, 1, 1].item()) == 1.0    # max is +0


# ----------------------------------------------------------------------------- selection

def _parse_golden(name):
    cases, cur = [], None
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        key, *vals = line.split()
        if key == "case":
            cur = {}
            cases.append(cur)
        else:
            cur[key] = vals
    return cases


def _sparse_col(spec, n):
    x = np.zeros(n, np.float32)
    for item in spec:
        idx, val = item.split(":")
        if "-" in idx:
            a, b = map(int, idx.split("-"))
            x[a:b + 1] = float(val)
        else:
            x[int(idx)] = float(val)
    return x


def test_query_summary_golden_order():
    """Hand-derived fp32 results that pin the blocked sequential order, the
    stride-halving tree over block sums, and head-major row order."""
    cases = _parse_golden("qbar_order.txt")
    a = cases[0]
    G, C, D = int(a["G"][0]), int(a["C"][0]), int(a["D"][0])
    q = torch.zeros(G, C, D)
    q[0, :, 0] = torch.from_numpy(_sparse_col(a["col0"], C))
    q[0, :, 1] = torch.from_numpy(_sparse_col(a["col1"], C))
    got = orc.query_summary(q, 0, G)
    assert got.tolist() == [float(x) for x in a["expect"]]
    b = cases[1]
    G, C, D = int(b["G"][0]), int(b["C"][0]), int(b["D"][0])
    q = torch.zeros(G, C, D)
    q[0, :, 0] = torch.from_numpy(_sparse_col(b["head0"], C))
    q[1, :, 0] = torch.from_numpy(_sparse_col(b["head1"], C))
    assert orc.query_summary(q, 0, G).tolist() == [float(x) for x in b["expect"]]


def test_query_summary_close_to_exact_mean():
    """qbar is the group mean: within the fp32 error bound of a blocked sum
    (<= (64 + log2 nb + 1) * eps * sum|x|) of the fp64 mean."""
    G, C, D = 7, 300, 16
    q = _rand((14, C, D), 5, torch.bfloat16)
    for g in range(2):
        x = q[g * G:(g + 1) * G].to(F64).reshape(-1, D)
        exact = x.mean(0).numpy()
        bound = (64 + 4 + 2) * 2.0 ** -24 * x.abs().sum(0).numpy() / (G * C) + 1e-30
        assert np.all(np.abs(orc.query_summary(q, g, G) - exact) <= bound)


def test_page_score_golden():
    """Hand-derived fp32 scores pin the stride-halving tree over d and the max rule."""
    for case in _parse_golden("score_order.txt"):
        qbar = np.array([float(x) for x in case["qbar"]], np.float32)
        kmin = torch.tensor([float(x) for x in case["kmin"]])
        kmax = torch.tensor([float(x) for x in case["kmax"]])
        summ = torch.stack([kmin, kmax])[None]
        table = torch.zeros(1, 1, dtype=torch.int32)
        assert orc.page_scores(qbar, summ, table, 0, 1).tolist() == [float(case["expect"][0])]


def test_page_score_constant_keys_closed_form():
    """Pages whose keys are c_j * e_0 score exactly qbar_0 * c_j."""
    D = 8
    qbar = np.zeros(D, np.float32)
    qbar[0] = np.float32(0.75)
    cs = [0.5, -2.0, 3.0, 1.25, -0.125]
    summ = torch.zeros(len(cs), 2, D)
    for j, c in enumerate(cs):
        summ[j, :, 0] = c
    table = torch.arange(len(cs), dtype=torch.int32)[None]
    got = orc.page_scores(qbar, summ, table, 0, len(cs))
    assert got.tolist() == [np.float32(0.75) * np.float32(c) for c in cs]


def test_page_score_upper_bounds_every_key():
    """Quest's property: sum_d max(q kmax, q kmin) >= q.k for every key of the page."""
    P, D = 16, 32
    k = _rand((1, 10 * P, D), 6, torch.bfloat16)
    table = torch.arange(10, dtype=torch.int32)[None]
    pool = k.reshape(10, P, D).clone()
    summ = torch.zeros(10, 2, D, dtype=torch.bfloat16)
    orc.summarize(pool, table, summ, 0, 10, 10 * P)
    qbar = _rand((D,), 7, torch.float32).numpy()
    sc = orc.page_scores(qbar, summ, table, 0, 10).astype(np.float64)
    dots = (pool.to(F64) @ torch.from_numpy(qbar).to(F64)).numpy()   # [10, P]
    assert np.all(sc + 1e-4 >= dots.max(axis=1))


def _brute_topk(scores, k):
    """Page j is chosen iff fewer than k pages beat it (higher score, or equal score
    and lower id). Independent of any sort."""
    n = len(scores)
    out = []
    for j in range(n):
        better = sum(1 for i in range(n)
                     if scores[i] > scores[j] or (scores[i] == scores[j] and i < j))
        if better < k:
            out.append(j)
    return out


def test_top_k_matches_brute_force_with_ties():
    rng = np.random.default_rng(0)
    for trial in range(30):
        n = int(rng.integers(0, 60))
        scores = rng.integers(-3, 4, size=n).astype(np.float32) * np.float32(0.5)
        if n and trial % 3 == 0:
            scores[rng.integers(0, n)] = -0.0
        for k in (0, 1, 5, n, n + 3):
            assert orc.top_k_pages(scores, k) == _brute_topk(list(scores), k)


def _brute_topk_nan(scores, k):
    """As _brute_topk, with NaN ranking below every number and NaNs tied (lower id
    first): page i beats page j iff both are numbers and (s_i > s_j, or s_i == s_j and
    i < j); or i is a number and j is NaN; or both are NaN and i < j."""
    n = len(scores)

    def beats(i, j):
        ni, nj = math.isnan(scores[i]), math.isnan(scores[j])
        if ni or nj:
            return (not ni and nj) or (ni and nj and i < j)
        return scores[i] > scores[j] or (scores[i] == scores[j] and i < j)

    return [j for j in range(n) if sum(1 for i in range(n) if i != j and beats(i, j)) < k]


def test_top_k_nan_ranks_lowest():
    """NaN scores (possible when keys hold infinities) rank below -inf; among NaNs the
    lower ids win; -0 and +0 still tie."""
    rng = np.random.default_rng(5)
    vals = np.array([np.nan, -np.inf, np.inf, -0.0, 0.0, 1.5, -1.5], np.float32)
    for trial in range(40):
        n = int(rng.integers(1, 40))
        scores = vals[rng.integers(0, len(vals), size=n)]
        for k in (0, 1, 3, n // 2, n, n + 2):
            assert orc.top_k_pages(scores, k) == _brute_topk_nan(list(scores), k)
    s = np.array([np.nan, -np.inf, np.nan, 2.0], np.float32)
    assert orc.top_k_pages(s, 2) == [1, 3]
    assert orc.top_k_pages(s, 3) == [0, 1, 3]


def test_top_k_special_cases():
    s = np.zeros(10, np.float32)
    assert orc.top_k_pages(s, 4) == [0, 1, 2, 3]            # all equal -> lowest ids
    assert orc.top_k_pages(s, 99) == list(range(10))        # k >= n -> all
    assert orc.top_k_pages(s, 0) == []
    s2 = np.array([0.0, -0.0, 0.0], np.float32)             # -0 == +0
    assert orc.top_k_pages(s2, 2) == [0, 1]


def test_selection_invariant_under_page_permutation():
    """The logical selection does not depend on where pages sit physically."""
    w = wl.custom("sparse1m", hq=4, hkv=2, d=64, page=16, chunk=64, total=64 + 40 * 16,
                  top_k=7, needles=3)
    x = wl.make_inputs(w, with_grad=False)
    res = []
    for seed in (11, 12):
        table = _table(w.hkv, w.pages_per_head, seed)
        pool = torch.zeros(w.pool_pages, w.page, w.d, dtype=w.dtype)
        orc.append(pool, table, x["k"], 0)
        summ = torch.zeros(w.pool_pages, 2, w.d, dtype=w.dtype)
        orc.summarize(pool, table, summ, 0, w.pages_per_head, w.total)
        res.append(orc.select_pages(x["q"], summ, table, w.t0, w.page, w.group, w.top_k))
    for (qa, sa, la), (qb, sb, lb) in zip(*res):
        assert np.array_equal(qa, qb) and np.array_equal(sa, sb) and la == lb


# ----------------------------------------------------------------------------- attention

def _case(hq=4, hkv=2, C=24, D=8, P=8, t0=37, seed=0, dtype=F64):
    T = t0 + C
    n_pages = -(-T // P)
    q = _rand((hq, C, D), seed + 1, dtype)
    k = _rand((hkv, T, D), seed + 2, dtype)
    v = _rand((hkv, T, D), seed + 3, dtype)
    do = _rand((hq, C, D), seed + 4, dtype)
    table = _table(hkv, n_pages, seed + 5)
    kp, vp = _build(k, v, P, table, hkv * n_pages)
    return dict(q=q, k=k, v=v, do=do, table=table, kp=kp, vp=vp, P=P, t0=t0, T=T,
                n_pages=n_pages)


@pytest.mark.parametrize("sparse", [False, True])
def test_fwd_bwd_match_sdpa_autograd(sparse):
    """One chunk call equals torch SDPA (fp64, GQA, explicit mask) and its autograd
    gradients, for dense and sparse page sets and an unaligned chunk start."""
    c = _case()
    P, t0 = c["P"], c["t0"]
    hkv = c["table"].shape[0]
    n_prior = t0 // P
    sel = None if not sparse else [[0, 2], [1, 3]]
    scale = 0.3
    O, L = orc.fwd(c["q"], c["kp"], c["vp"], c["table"], t0, sel, scale)
    pages = [orc.attended_pages(t0, c["q"].shape[1], P, None if sel is None else sel[g])
             for g in range(hkv)]
    q = c["q"].clone().requires_grad_()
    k = c["k"].clone().requires_grad_()
    v = c["v"].clone().requires_grad_()
    ref = _sdpa(q, k, v, t0, pages, P, scale)
    (ref * c["do"]).sum().backward()
    assert torch.allclose(O, ref.detach(), atol=1e-13, rtol=0)
    gpool_k = torch.zeros(c["kp"].shape, dtype=F64)
    gpool_v = torch.zeros(c["vp"].shape, dtype=F64)
    gtable = _table(hkv, c["n_pages"], 99)
    dQ, _, O2, L2 = orc.bwd(c["q"], c["kp"], c["vp"], c["table"], t0, sel, scale, c["do"],
                            gpool_k, gpool_v, gtable, with_fwd=True)
    assert torch.allclose(dQ, q.grad, atol=1e-12, rtol=0)
    # the forward recomputed inside the backward is the forward (SDPA and fwd itself)
    assert torch.allclose(O2, ref.detach(), atol=1e-13, rtol=0)
    assert torch.equal(O2, O) and torch.equal(L2, L)
    for g in range(hkv):
        dk = orc.gather(gpool_k, gtable, g, range(c["n_pages"]))[:c["T"]]
        dv = orc.gather(gpool_v, gtable, g, range(c["n_pages"]))[:c["T"]]
        assert torch.allclose(dk, k.grad[g], atol=1e-12, rtol=0)
        assert torch.allclose(dv, v.grad[g], atol=1e-12, rtol=0)
    assert n_prior > 2


@pytest.mark.parametrize("window", [3, 8, 17, 40])
def test_window_matches_banded_sdpa_autograd(window):
    """Local attention (explainer 2.D, sparse layers) equals torch SDPA under a banded
    causal mask, forward and autograd gradients: windows inside one page, across
    pages, reaching into the prior pages, and longer than the context at early
    queries."""
    c = _case()
    P, t0 = c["P"], c["t0"]
    hkv = c["table"].shape[0]
    scale = 0.3
    O, L = orc.fwd(c["q"], c["kp"], c["vp"], c["table"], t0, None, scale, window=window)
    pages = [orc.attended_pages(t0, c["q"].shape[1], P, None) for _ in range(hkv)]
    q = c["q"].clone().requires_grad_()
    k = c["k"].clone().requires_grad_()
    v = c["v"].clone().requires_grad_()
    ref = _sdpa(q, k, v, t0, pages, P, scale, window)
    (ref * c["do"]).sum().backward()
    assert torch.allclose(O, ref.detach(), atol=1e-13, rtol=0)
    gk = torch.zeros(c["kp"].shape, dtype=F64)
    gv = torch.zeros(c["vp"].shape, dtype=F64)
    dQ, _ = orc.bwd(c["q"], c["kp"], c["vp"], c["table"], t0, None, scale, c["do"], gk, gv,
                    c["table"], window=window)
    assert torch.allclose(dQ, q.grad, atol=1e-12, rtol=0)
    for g in range(hkv):
        dk = orc.gather(gk, c["table"], g, range(c["n_pages"]))[:c["T"]]
        dv = orc.gather(gv, c["table"], g, range(c["n_pages"]))[:c["T"]]
        assert torch.allclose(dk, k.grad[g], atol=1e-12, rtol=0)
        assert torch.allclose(dv, v.grad[g], atol=1e-12, rtol=0)


def test_window_one_and_window_covering_all():
    """Window 1: each query sees only its own key, so O = v_p, LSE = scale q.k_p, and
    the backward has dS = 0 (dQ = dK = 0) with dV_p = the sum of dO over the group's
    heads at p. A window reaching position 0 from every query equals no window,
    bitwise."""
    c = _case()
    P, t0, scale = c["P"], c["t0"], 0.3
    hq, C, D = c["q"].shape
    hkv = c["k"].shape[0]
    G = hq // hkv
    O, L = orc.fwd(c["q"], c["kp"], c["vp"], c["table"], t0, None, scale, window=1)
    gk = torch.zeros(c["kp"].shape, dtype=F64)
    gv = torch.zeros(c["vp"].shape, dtype=F64)
    dQ, per_head = orc.bwd(c["q"], c["kp"], c["vp"], c["table"], t0, None, scale, c["do"], gk,
                           gv, c["table"], window=1)
    for h in range(hq):
        g = h // G
        assert torch.equal(O[h], c["v"][g, t0:t0 + C])
        lse = scale * (c["q"][h] * c["k"][g, t0:t0 + C]).sum(-1)
        assert torch.allclose(L[h], lse, atol=1e-14, rtol=0)
    assert dQ.abs().max().item() < 1e-14
    for g, (pos, dk, dv) in enumerate(per_head):
        assert dk.abs().max().item() < 1e-14
        want = torch.zeros_like(dv)
        own = (pos >= t0).nonzero()[:, 0]
        want[own] = c["do"][g * G:(g + 1) * G, (pos[own] - t0)].sum(0)
        assert torch.allclose(dv, want, atol=1e-14, rtol=0)
    O0, L0 = orc.fwd(c["q"], c["kp"], c["vp"], c["table"], t0, None, scale)
    Ow, Lw = orc.fwd(c["q"], c["kp"], c["vp"], c["table"], t0, None, scale, window=t0 + C)
    assert torch.equal(O0, Ow) and torch.equal(L0, Lw)
    with pytest.raises(ValueError):
        orc.fwd(c["q"], c["kp"], c["vp"], c["table"], t0, [[0], [1]], scale, window=4)


def test_lse_matches_logsumexp():
    c = _case(seed=3)
    scale = 0.4
    O, L = orc.fwd(c["q"], c["kp"], c["vp"], c["table"], c["t0"], None, scale)
    hq, C, _ = c["q"].shape
    G = hq // c["k"].shape[0]
    for h in range(hq):
        for i in (0, 5, C - 1):
            s = scale * (c["k"][h // G, :c["t0"] + i + 1] @ c["q"][h, i])
            assert abs(L[h, i].item() - torch.logsumexp(s, 0).item()) < 1e-12


def test_finite_differences():
    """Central differences of L = sum(dO * O) agree with the analytic dQ, dK, dV."""
    c = _case(hq=2, hkv=1, C=6, D=4, P=4, t0=9, seed=7)
    P, t0, scale = c["P"], c["t0"], 0.7
    sel = [[0, 1]]
    table = c["table"]

    def loss(q, kp, vp):
        O, _ = orc.fwd(q, kp, vp, table, t0, sel, scale)
        return float((O * c["do"]).sum())

    gk = torch.zeros(c["kp"].shape, dtype=F64)
    gv = torch.zeros(c["vp"].shape, dtype=F64)
    dQ, _ = orc.bwd(c["q"], c["kp"], c["vp"], table, t0, sel, scale, c["do"], gk, gv, table)
    h = 1e-6
    rng = np.random.default_rng(1)
    for _ in range(12):
        idx = tuple(int(rng.integers(0, s)) for s in c["q"].shape)
        qp, qm = c["q"].clone(), c["q"].clone()
        qp[idx] += h
        qm[idx] -= h
        fd = (loss(qp, c["kp"], c["vp"]) - loss(qm, c["kp"], c["vp"])) / (2 * h)
        assert abs(fd - dQ[idx].item()) < 1e-7
    attended = orc.key_positions(orc.attended_pages(t0, 6, P, sel[0]), P, t0 + 6)
    for t in attended.tolist()[::2]:
        phys, slot = int(table[0, t // P]), t % P
        for d in range(4):
            for pool, grad in ((c["kp"], gk), (c["vp"], gv)):
                p_, m_ = pool.clone(), pool.clone()
                p_[phys, slot, d] += h
                m_[phys, slot, d] -= h
                if pool is c["kp"]:
                    fd = (loss(c["q"], p_, c["vp"]) - loss(c["q"], m_, c["vp"])) / (2 * h)
                else:
                    fd = (loss(c["q"], c["kp"], p_) - loss(c["q"], c["kp"], m_)) / (2 * h)
                assert abs(fd - grad[phys, slot, d].item()) < 1e-7


def test_closed_forms():
    """Single visible key: O = v0, LSE = s0, dQ = 0, dV += dO. All-zero keys: O is
    the prefix mean of V. Per KV head: sum_t dK_t = 0 and sum_t dV_t = sum dO."""
    hq, hkv, D, P = 2, 1, 4, 4
    q = _rand((hq, 3, D), 1)
    k = _rand((hkv, 3, D), 2)
    v = _rand((hkv, 3, D), 3)
    do = _rand((hq, 3, D), 4)
    table = torch.zeros(1, 1, dtype=torch.int32)
    kp, vp = _build(k, v, P, table, 1)
    O, L = orc.fwd(q, kp, vp, table, 0, None, 0.5)
    for h in range(hq):
        assert torch.allclose(O[h, 0], v[0, 0], atol=1e-15)
        assert abs(L[h, 0].item() - 0.5 * float(q[h, 0] @ k[0, 0])) < 1e-15
    gk = torch.zeros(1, P, D, dtype=F64)
    gv = torch.zeros(1, P, D, dtype=F64)
    dQ, _ = orc.bwd(q[:, :1], kp, vp, table, 0, None, 0.5, do[:, :1], gk, gv, table)
    assert torch.allclose(dQ, torch.zeros_like(dQ), atol=1e-15)
    assert torch.allclose(gv[0, 0], do[:, 0].sum(0), atol=1e-15)

    c = _case(seed=11)
    kz = torch.zeros_like(c["kp"])
    O, _ = orc.fwd(c["q"], kz, c["vp"], c["table"], c["t0"], None, 1.0)
    G = c["q"].shape[0] // c["k"].shape[0]
    for h in range(c["q"].shape[0]):
        for i in range(c["q"].shape[1]):
            m = c["v"][h // G, :c["t0"] + i + 1].mean(0)
            assert torch.allclose(O[h, i], m, atol=1e-13)

    c = _case(seed=12)
    _, per_head = orc.bwd(c["q"], c["kp"], c["vp"], c["table"], c["t0"], [[1, 3], [0]], 0.35,
                          c["do"])
    for g, (pos, dK, dV) in enumerate(per_head):
        assert torch.allclose(dK.sum(0), torch.zeros(dK.shape[1], dtype=F64), atol=1e-12)
        G = c["q"].shape[0] // c["k"].shape[0]
        assert torch.allclose(dV.sum(0), c["do"][g * G:(g + 1) * G].sum((0, 1)), atol=1e-12)


def test_page_permutation_invariance_bitwise():
    """O, LSE and dQ are bit-identical under two physical placements; gradient pools
    agree after mapping pages back."""
    c = _case(seed=21)
    res = []
    for seed in (1, 2):
        table = _table(2, c["n_pages"], seed)
        kp, vp = _build(c["k"], c["v"], c["P"], table, 2 * c["n_pages"])
        gk = torch.zeros(kp.shape, dtype=F64)
        gv = torch.zeros(kp.shape, dtype=F64)
        O, L = orc.fwd(c["q"], kp, vp, table, c["t0"], [[0, 3], [2]], 0.4)
        dQ, _ = orc.bwd(c["q"], kp, vp, table, c["t0"], [[0, 3], [2]], 0.4, c["do"], gk, gv,
                        table)
        dk = torch.stack([orc.gather(gk, table, g, range(c["n_pages"])) for g in range(2)])
        res.append((O, L, dQ, dk))
    for a, b in zip(*res):
        assert torch.equal(a, b)


def test_sparse_with_all_pages_equals_dense_bitwise():
    c = _case(seed=31)
    n_prior = c["t0"] // c["P"]
    everything = [list(range(n_prior))] * 2
    a = orc.fwd(c["q"], c["kp"], c["vp"], c["table"], c["t0"], None, 0.3)
    b = orc.fwd(c["q"], c["kp"], c["vp"], c["table"], c["t0"], everything, 0.3)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_sweep_equals_full_sequence_causal_attention():
    """Chunk-recurrent forward + reverse recompute/backward over the tiny workload
    (1024 fp32 tokens, 16 chunks of 64, shuffled pages) equals full-sequence causal
    SDPA and its autograd gradients (explainer 2.A: chunking with recomputation
    computes the same result as ordinary training)."""
    w = wl.WORKLOADS["tiny"]
    x = wl.make_inputs(w)
    r = orc.sweep(x["q"], x["k"], x["v"], x["do"], x["table"], x["gtable"], w.pool_pages,
                  w.page, w.chunk, w.scale)
    q = x["q"].to(F64).requires_grad_()
    k = x["k"].to(F64).requires_grad_()
    v = x["v"].to(F64).requires_grad_()
    ref = F.scaled_dot_product_attention(q[None], k[None], v[None], is_causal=True,
                                         scale=w.scale, enable_gqa=True)[0]
    (ref * x["do"].to(F64)).sum().backward()
    assert torch.allclose(r["O"], ref.detach(), atol=1e-12, rtol=0)
    assert torch.allclose(r["dQ"], q.grad, atol=1e-12, rtol=0)
    for g in range(w.hkv):
        dk = orc.gather(r["dk_pool"], x["gtable"], g, range(w.pages_per_head))
        dv = orc.gather(r["dv_pool"], x["gtable"], g, range(w.pages_per_head))
        assert torch.allclose(dk, k.grad[g], atol=1e-12, rtol=0)
        assert torch.allclose(dv, v.grad[g], atol=1e-12, rtol=0)


def test_sparse_sweep_selects_and_matches_masked_sdpa():
    """A top-k sweep: every chunk's O and the accumulated dK/dV equal SDPA with the
    page mask implied by the sweep's own selections."""
    w = wl.custom("sweep256k_top64", hq=4, hkv=2, d=16, page=8, chunk=32, total=160, top_k=3)
    x = wl.make_inputs(w)
    r = orc.sweep(x["q"], x["k"], x["v"], x["do"], x["table"], x["gtable"], w.pool_pages,
                  w.page, w.chunk, w.scale, top_k=w.top_k)
    q = x["q"].to(F64).requires_grad_()
    k = x["k"].to(F64).requires_grad_()
    v = x["v"].to(F64).requires_grad_()
    outs = []
    for c in range(w.n_chunks):
        t0 = c * w.chunk
        pages = [orc.attended_pages(t0, w.chunk, w.page, r["sels"][c][g]) for g in range(w.hkv)]
        for g in range(w.hkv):
            assert len(r["sels"][c][g]) == min(w.top_k, t0 // w.page)
        outs.append(_sdpa(q[:, t0:t0 + w.chunk], k, v, t0, pages, w.page, w.scale))
    ref = torch.cat(outs, dim=1)
    (ref * x["do"].to(F64)).sum().backward()
    assert torch.allclose(r["O"], ref.detach(), atol=1e-12, rtol=0)
    assert torch.allclose(r["dQ"], q.grad, atol=1e-12, rtol=0)
    for g in range(w.hkv):
        dk = orc.gather(r["dk_pool"], x["gtable"], g, range(w.pages_per_head))
        assert torch.allclose(dk, k.grad[g], atol=1e-12, rtol=0)


# ----------------------------------------------------------------------------- page movement

def test_copy_pages_round_trip_and_skips():
    """Copying pages out and back restores them bitwise; ids outside either array are
    skipped and every page not named keeps its value."""
    src = _rand((12, 4, 8), 21, torch.bfloat16)
    host = torch.full((20, 4, 8), 7.0, dtype=torch.bfloat16)
    src_ids = [3, 0, 11, -1, 5, 40]
    dst_ids = [19, 2, 7, 4, -3, 1]
    orc.copy_pages(src, host, src_ids, dst_ids)
    for s, d in ((3, 19), (0, 2), (11, 7)):
        assert torch.equal(host[d], src[s])
    untouched = [i for i in range(20) if i not in (19, 2, 7)]
    assert bool((host[untouched] == 7.0).all())
    back = torch.zeros_like(src)
    orc.copy_pages(host, back, [19, 2, 7], [3, 0, 11])
    assert torch.equal(back[[3, 0, 11]], src[[3, 0, 11]])
    orc.copy_pages(src, back, [1, 2], [1, 2], n=1)  # n limits the list
    assert torch.equal(back[1], src[1]) and bool((back[2] == 0).all())


def test_add_pages_identities():
    """Adding zero pages changes nothing bitwise; adding into zero pages copies; the sum
    is the correctly rounded one (integers below 2^24 add exactly); zero_src clears."""
    x = _rand((6, 4, 8), 22, torch.float32)
    acc = x.clone()
    zeros = torch.zeros_like(x)
    orc.add_pages(zeros, acc, range(6), range(6))
    assert torch.equal(acc, x)
    dst = torch.zeros_like(x)
    orc.add_pages(x, dst, [0, 1], [4, 5])
    assert torch.equal(dst[4], x[0]) and torch.equal(dst[5], x[1])
    a = torch.full((2, 4, 8), 3.0e6)
    b = torch.full((2, 4, 8), 1234567.0)
    orc.add_pages(b, a, [0, 1], [1, 0], zero_src=True)
    assert bool((a == 4234567.0).all()) and bool((b == 0).all())
    # one rounding: 1 + 2^-24 rounds to 1 in fp32 (ties to even), 1 + 3 * 2^-24 does not
    c = torch.ones(1, 1, 4)
    d = torch.tensor([[[2.0 ** -24, 3 * 2.0 ** -24, 0.0, -1.0]]])
    orc.add_pages(d, c, [0], [0])
    assert c.flatten().tolist() == [1.0, 1.0 + 2.0 ** -22, 1.0, 0.0]


def test_fetch_selected_then_gather_equals_host_pages():
    """After the fetch, gathering the selected logical pages through the updated table
    from the device pool gives the host's pages bitwise, for every KV head; unselected
    entries of the table are unchanged; out-of-range selections are skipped."""
    hkv, P, D, n_logical = 2, 4, 8, 10
    host_k = _rand((hkv * n_logical, P, D), 23, torch.bfloat16)
    host_v = _rand((hkv * n_logical, P, D), 24, torch.bfloat16)
    host_table = _table(hkv, n_logical, 25)
    k_pool = torch.zeros(16, P, D, dtype=torch.bfloat16)
    v_pool = torch.zeros_like(k_pool)
    table = torch.full((hkv, n_logical), -1, dtype=torch.int32)
    sel = torch.tensor([[1, 4, 8, 12], [0, 9, -2, 3]], dtype=torch.int32)
    count = torch.tensor([3, 4], dtype=torch.int32)
    stage = torch.tensor([[10, 11, 12, 13], [2, 3, 4, 5]], dtype=torch.int32)
    orc.fetch_selected(k_pool, v_pool, table, host_k, host_v, host_table, sel, count, stage,
                       n_logical)
    for g, chosen in ((0, [1, 4, 8]), (1, [0, 9, 3])):
        assert torch.equal(orc.gather(k_pool, table, g, chosen),
                           orc.gather(host_k, host_table, g, chosen))
        assert torch.equal(orc.gather(v_pool, table, g, chosen),
                           orc.gather(host_v, host_table, g, chosen))
        rest = [lp for lp in range(n_logical) if lp not in chosen]
        assert bool((table[g, rest] == -1).all())


# ----------------------------------------------------------------------------- mean-key selector

def test_summarize_mean_order_and_closed_forms():
    """The mean-key summary sums in token order: 1 + 2^-24 + 2^-24 stays 1 in fp32 (ties
    to even twice), so the mean of those three keys is fp32(1/3) exactly, where any
    other order would give more. Constant keys average to themselves; a partial page
    counts only tokens below seq_len; pages with none stay unchanged."""
    P, D = 4, 8
    k_pool = torch.zeros(3, P, D, dtype=torch.float32)
    k_pool[0, 0, 0], k_pool[0, 1, 0], k_pool[0, 2, 0] = 1.0, 2.0 ** -24, 2.0 ** -24
    k_pool[1] = 0.75
    k_pool[2] = 5.0
    table = torch.tensor([[0, 1, 2]], dtype=torch.int32)
    kmean = np.full((3, D), -7.0, np.float32)
    orc.summarize_mean(k_pool, table, kmean, 0, 1, seq_len=3)      # page 0: 3 valid tokens
    orc.summarize_mean(k_pool, table, kmean, 1, 2, seq_len=2 * P)  # page 1 full, page 2 none
    assert kmean[0, 0] == np.float32(1.0 / 3.0)
    assert kmean[0, 0] < np.float32(1.0 + 2.0 ** -23) * np.float32(1.0 / 3.0)
    assert bool((kmean[1] == np.float32(0.75)).all())  # 4 tokens of 0.75 (page 1 full)
    assert bool((kmean[2] == np.float32(-7.0)).all())  # page 2 starts at seq_len: unchanged


def test_page_scores_mean_equals_minmax_with_equal_bounds():
    """With kmin = kmax = kmean the min/max score takes the same products through the
    same tree, so the two score functions agree bitwise (pinning the mean score to the
    golden-pinned min/max one); constant means give qbar_0 * c exactly."""
    rng = np.random.default_rng(5)
    D, n = 64, 37
    qbar = rng.standard_normal(D).astype(np.float32)
    kmean = rng.standard_normal((n, D)).astype(np.float32)
    table = torch.arange(n, dtype=torch.int32)[None]
    summ = torch.from_numpy(np.stack([kmean, kmean], 1))
    assert np.array_equal(orc.page_scores_mean(qbar, kmean, table, 0, n),
                          orc.page_scores(qbar, summ, table, 0, n))
    cm = np.zeros((3, D), np.float32)
    cm[:, 0] = [0.5, -2.0, 3.0]
    got = orc.page_scores_mean(qbar, cm, torch.arange(3, dtype=torch.int32)[None], 0, 3)
    assert got.tolist() == [qbar[0] * np.float32(c) for c in (0.5, -2.0, 3.0)]


# ----------------------------------------------------------------------------- rotary embedding

def test_rope_closed_forms_and_invariants():
    """Position 0 is the identity; a hand-computed rotation (D = 4, theta = 100: angles
    p and p / 10); pair norms are kept; the inverse undoes the forward; dot products
    depend on positions only through their difference."""
    x = _rand((3, 5, 8), 31)
    assert torch.allclose(orc.rope(x[:, :1], 0), x[:, :1].double(), atol=0, rtol=0)
    v = torch.tensor([[[1.0, 2.0, 3.0, 4.0]]], dtype=F64)
    got = orc.rope(v, 2, theta=100.0)[0, 0]
    want = torch.tensor([1 * math.cos(2) - 3 * math.sin(2), 2 * math.cos(0.2) - 4 * math.sin(0.2),
                         3 * math.cos(2) + 1 * math.sin(2), 4 * math.cos(0.2) + 2 * math.sin(0.2)],
                        dtype=F64)
    assert torch.allclose(got, want, atol=1e-14, rtol=0)
    y = orc.rope(x, 12345)
    pair = lambda t: t[..., :4] ** 2 + t[..., 4:] ** 2
    assert torch.allclose(pair(y), pair(x.double()), atol=1e-12, rtol=0)
    assert torch.allclose(orc.rope(y, 12345, inverse=True), x.double(), atol=1e-12, rtol=0)
    q, k = _rand((1, 1, 8), 32), _rand((1, 1, 8), 33)
    d1 = (orc.rope(q, 40) * orc.rope(k, 17)).sum()
    d2 = (orc.rope(q, 1040) * orc.rope(k, 1017)).sum()
    assert abs(float(d1 - d2)) < 1e-11



def _layer_by_chunks(x, ws, hq, hkv, D, page, chunk, scale, theta, dy, top_k, window):
    """The same layer assembled chunk by chunk from the oracle's separately pinned
    pieces: float64 projections and rotary embedding, the paged chunk sweep (keys and
    values in fp32 pages, queries and dO in float64), then the chain rule through the
    projections and the rotation (its transpose is the inverse rotation) by hand."""
    X = x.double()
    Wq, Wk, Wv, Wo = (w.double() for w in ws)
    T = X.shape[0]
    q = orc.rope((X @ Wq).view(T, hq, D).transpose(0, 1), 0, theta)
    k = orc.rope((X @ Wk).view(T, hkv, D).transpose(0, 1), 0, theta)
    v = (X @ Wv).view(T, hkv, D).transpose(0, 1)
    dO = (dy.double() @ Wo.T).view(T, hq, D).transpose(0, 1)
    n_pages = T // page
    table = _table(hkv, n_pages, 3)
    gtable = _table(hkv, n_pages, 4)
    r = orc.sweep(q, k.float(), v.float(), dO, table, gtable, hkv * n_pages, page, chunk, scale,
                  top_k=top_k, window=window)
    O = r["O"].transpose(0, 1).reshape(T, hq * D)
    dk = torch.stack([orc.gather(r["dk_pool"], gtable, g, range(n_pages)) for g in range(hkv)])
    dv = torch.stack([orc.gather(r["dv_pool"], gtable, g, range(n_pages)) for g in range(hkv)])
    dq_lin = orc.rope(r["dQ"], 0, theta, inverse=True).transpose(0, 1).reshape(T, hq * D)
    dk_lin = orc.rope(dk, 0, theta, inverse=True).transpose(0, 1).reshape(T, hkv * D)
    dv_lin = dv.transpose(0, 1).reshape(T, hkv * D)
    y = O @ Wo
    dX = dq_lin @ Wq.T + dk_lin @ Wk.T + dv_lin @ Wv.T
    dW = [X.T @ dq_lin, X.T @ dk_lin, X.T @ dv_lin, O.T @ dy.double()]
    return y, dX, dW, r["sels"]


@pytest.mark.parametrize("top_k,window", [(None, 0), (None, 11), (2, 0)])
def test_layer_reference_equals_chunk_by_chunk(top_k, window):
    """The full-sequence layer reference (one masked softmax, autograd) equals the layer
    computed chunk by chunk over the paged sweep with a hand-written backward, for a
    dense, a local (window) and a top-k layer; the top-k layer's selections agree."""
    hidden, hq, hkv, D, page, chunk, T = 24, 4, 2, 8, 8, 32, 128
    g = torch.Generator().manual_seed(21)
    x = torch.randn(T, hidden, generator=g)
    ws = [torch.randn(a, b, generator=g) / math.sqrt(a)
          for a, b in ((hidden, hq * D), (hidden, hkv * D), (hidden, hkv * D), (hq * D, hidden))]
    dy = torch.randn(T, hidden, generator=g)
    scale, theta = D ** -0.5, 100.0
    y, dx, dw, sels = orc.layer_reference(x, *ws, hq, hkv, D, page, chunk, scale, theta, dy,
                                          top_k=top_k, window=window, sel_dtype=torch.float32)
    y2, dx2, dw2, sels2 = _layer_by_chunks(x, ws, hq, hkv, D, page, chunk, scale, theta, dy,
                                           top_k, window)
    if top_k is not None:
        assert sels == sels2
        assert any(len(s_[0]) == top_k for s_ in sels)          # selection really narrowed
    else:
        assert sels is None
    assert torch.allclose(y, y2, rtol=1e-5, atol=1e-5)
    assert torch.allclose(dx, dx2, rtol=1e-5, atol=1e-5)
    for a, b in zip(dw, dw2):
        assert torch.allclose(a, b, rtol=1e-5, atol=1e-5)
    # and the dense layer's attention is plain causal attention (SDPA, GQA, no mask)
    if top_k is None and window == 0:
        X = x.double()
        q = orc.rope((X @ ws[0].double()).view(T, hq, D).transpose(0, 1), 0, theta)
        k = orc.rope((X @ ws[1].double()).view(T, hkv, D).transpose(0, 1), 0, theta)
        v = (X @ ws[2].double()).view(T, hkv, D).transpose(0, 1)
        o = F.scaled_dot_product_attention(q, k, v, is_causal=True, scale=scale, enable_gqa=True)
        assert torch.allclose(y, o.transpose(0, 1).reshape(T, hq * D) @ ws[3].double(),
                              rtol=1e-10, atol=1e-10)


# ----------------------------------------------------------------- tiled selection

def _summ_case(hq=6, hkv=2, C=100, D=16, P=8, t0=203, seed=3, dtype=torch.float32):
    c = _case(hq=hq, hkv=hkv, C=C, D=D, P=P, t0=t0, seed=seed, dtype=dtype)
    summ = torch.zeros(c["kp"].shape[0], 2, D, dtype=dtype)
    orc.summarize(c["kp"], c["table"], summ, 0, c["n_pages"], c["T"])
    return c, summ


def test_tiled_selection_one_tile_is_the_chunk_rule():
    """A tile as long as the chunk reproduces the per-chunk selection bit for bit."""
    c, summ = _summ_case()
    G = c["q"].shape[0] // 2
    ref = orc.select_pages(c["q"], summ, c["table"], c["t0"], c["P"], G, 5)
    for tile in (100, 128, 1000):
        got = orc.select_pages_tiled(c["q"], summ, c["table"], c["t0"], c["P"], G, 5, tile)
        for g in range(2):
            assert len(got[g]) == 1
            qb, sc, ch = got[g][0]
            assert np.array_equal(qb.view(np.int32), ref[g][0].view(np.int32))
            assert np.array_equal(sc.view(np.int32), ref[g][1].view(np.int32))
            assert ch == ref[g][2]


def test_tiled_qbar_is_each_tiles_mean():
    """Each tile's query summary is the mean of that tile's rows over the head group,
    within the blocked-sum error bound; the last tile is the shorter one."""
    c, summ = _summ_case(C=150)
    G = 3
    out = orc.select_pages_tiled(c["q"], summ, c["table"], c["t0"], c["P"], G, 4, 64)
    assert [len(r) for r in out] == [3, 3]
    for g in range(2):
        for j, r in enumerate(orc.query_tiles(150, 64)):
            rows = c["q"][g * G:(g + 1) * G, r.start:r.stop].to(F64).reshape(-1, 16)
            exact = rows.mean(0).numpy()
            n = rows.shape[0]
            bound = (n + 10) * np.finfo(np.float32).eps * rows.abs().mean(0).numpy() + 1e-30
            assert np.all(np.abs(out[g][j][0] - exact) <= bound)
    assert orc.query_tiles(150, 64) == [range(0, 64), range(64, 128), range(128, 150)]


def test_tiled_selection_follows_each_tiles_queries():
    """Closed form: page 2 of each head holds keys along e0, page 5 along e1; the first
    tile's queries point along e0, the second's along e1, so with k = 1 the tiles pick
    pages 2 and 5, while the whole chunk (the mean of both) picks the larger one."""
    hq, hkv, D, P, C, t0 = 2, 1, 8, 4, 8, 32
    T = t0 + C
    k = torch.zeros(1, T, D)
    k[0, 2 * P:3 * P, 0] = 1.0
    k[0, 5 * P:6 * P, 1] = 1.0
    q = torch.zeros(hq, C, D)
    q[:, :4, 0] = 1.0
    q[:, 4:, 1] = 2.0
    table = torch.arange(T // P, dtype=torch.int32)[None]
    kp = torch.zeros(T // P, P, D)
    orc.append(kp, table, k, 0)
    summ = torch.zeros(T // P, 2, D)
    orc.summarize(kp, table, summ, 0, T // P, T)
    out = orc.select_pages_tiled(q, summ, table, t0, P, hq, 1, 4)
    assert [ch for (_, _, ch) in out[0]] == [[2], [5]]
    assert orc.select_pages(q, summ, table, t0, P, hq, 1)[0][2] == [5]
    # the rows a tile attends: its pick, then the chunk's pages before its first query
    assert orc.tile_selection_row([5], t0, P, 4, 1) == [5, 8]
    assert orc.tile_selection_row([2], t0, P, 4, 0) == [2]


@pytest.mark.parametrize("t0,C,tile", [(37, 24, 8), (40, 30, 16), (29, 17, 5)])
def test_tiled_attention_matches_masked_sdpa(t0, C, tile):
    """Tiled attention (each tile its own prior pages, the chunk's own pages for all)
    equals SDPA whose mask gives every query row its tile's pages, with autograd
    gradients, for unaligned chunk starts and tile edges and a short last tile."""
    c = _case(C=C, t0=t0)
    P, hkv, G = c["P"], 2, 2
    n_prior = t0 // P
    rng = np.random.default_rng(t0 + C)
    tiles = orc.query_tiles(C, tile)
    chosen = [[sorted(rng.choice(n_prior, size=int(rng.integers(0, n_prior + 1)),
                                 replace=False).tolist()) for _ in tiles] for _ in range(hkv)]
    scale = 0.3
    O, L = orc.fwd_tiled(c["q"], c["kp"], c["vp"], c["table"], t0, chosen, scale, tile)
    gk = torch.zeros(c["kp"].shape, dtype=F64)
    gv = torch.zeros(c["vp"].shape, dtype=F64)
    gtable = _table(hkv, c["n_pages"], 77)
    dQ = orc.bwd_tiled(c["q"], c["kp"], c["vp"], c["table"], t0, chosen, scale, tile, c["do"],
                       gk, gv, gtable)
    # the reference mask, row by row: prior pages of the row's tile, or the chunk's pages
    T = c["T"]
    kpos = torch.arange(T)
    mask = torch.zeros(4, C, T, dtype=torch.bool)
    for h in range(4):
        for j, r in enumerate(tiles):
            ok = (kpos // P) >= t0 // P
            for pg in chosen[h // G][j]:
                ok |= (kpos // P) == pg
            for i in r:
                mask[h, i] = ok & (kpos <= t0 + i)
    q = c["q"].clone().requires_grad_()
    k = c["k"].clone().requires_grad_()
    v = c["v"].clone().requires_grad_()
    ref = F.scaled_dot_product_attention(q[None], k[None], v[None], attn_mask=mask[None],
                                         scale=scale, enable_gqa=True)[0]
    (ref * c["do"]).sum().backward()
    assert torch.allclose(O, ref.detach(), atol=1e-12, rtol=0)
    assert torch.allclose(dQ, q.grad, atol=1e-12, rtol=0)
    for g in range(hkv):
        dk = orc.gather(gk, gtable, g, range(c["n_pages"]))[:T]
        dv = orc.gather(gv, gtable, g, range(c["n_pages"]))[:T]
        assert torch.allclose(dk, k.grad[g], atol=1e-12, rtol=0)
        assert torch.allclose(dv, v.grad[g], atol=1e-12, rtol=0)
    s = torch.logsumexp((scale * (c["q"] @ k.detach().repeat_interleave(2, 0).transpose(1, 2)))
                        .masked_fill(~mask, -math.inf), dim=-1)
    assert torch.allclose(L, s, atol=1e-12, rtol=0)
