"""The C-ABI library loads, exports every function include/oomb.h declares, and
rejects invalid arguments on the host with the documented status (no GPU needed:
every call here fails validation before any HIP call)."""
import ctypes
import os
import re

import pytest

from paged_chunk_attention_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "oomb.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(oomb_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from paged_chunk_attention_amd.build import build
        build()
    return L.lib()


def test_exports_every_declared_symbol(lib):
    names = _declared()
    assert len(names) == 24
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(L.SIGNATURES)


def test_status_strings(lib):
    assert lib.oomb_abi_version() == 11
    for code, text in [(0, b"ok"), (1, b"invalid argument"), (2, b"unsupported configuration"),
                       (3, b"HIP launch failure"), (4, b"workspace missing or too small")]:
        assert lib.oomb_status_string(code) == text


def _pool(**kw):
    base = dict(dtype=0, page_size=128, head_dim=128, num_q_heads=28, num_kv_heads=4, reserved=0,
                num_pages=64, num_grad_pages=64, k_pool=0x100000, v_pool=0x200000,
                k_summary=0x300000, dk_pool=0x400000, dv_pool=0x500000)
    base.update(kw)
    return L.OombPool(**base)


# Fake but well-aligned device addresses: never dereferenced, every call below is
# rejected by the host-side checks first.
T, Q, O, B = 0x600000, 0x700000, 0x800000, 0x900000


def _fwd(lib, pool, **kw):
    a = dict(table=T, tstride=64, q=Q, qhs=4096 * 128, qts=128, n_q=4096, t0=4096, sel=None,
             sstride=0, count=None, window=0, scale=0.088, o=O, ohs=4096 * 128, ots=128, lse=B,
             ws=0xA00000, wsb=1 << 30)
    a.update(kw)
    return lib.oomb_paged_chunk_attn_fwd(ctypes.byref(pool), a["table"], a["tstride"], a["q"],
                                         a["qhs"], a["qts"], a["n_q"], a["t0"], a["sel"],
                                         a["sstride"], a["count"], a["window"], a["scale"], a["o"],
                                         a["ohs"], a["ots"], a["lse"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(dtype=7), L.OOMB_ERR_UNSUPPORTED),
    (dict(head_dim=96), L.OOMB_ERR_UNSUPPORTED),
    (dict(page_size=100), L.OOMB_ERR_UNSUPPORTED),
    (dict(page_size=8), L.OOMB_ERR_UNSUPPORTED),
    (dict(num_q_heads=27), L.OOMB_ERR_INVALID),
    (dict(num_kv_heads=0), L.OOMB_ERR_INVALID),
    (dict(k_pool=None), L.OOMB_ERR_INVALID),
    (dict(v_pool=0x200008), L.OOMB_ERR_INVALID),
    (dict(reserved=1), L.OOMB_ERR_INVALID),
    (dict(num_pages=0), L.OOMB_ERR_INVALID),
])
def test_pool_descriptor_errors(lib, kw, code):
    assert _fwd(lib, _pool(**kw)) == code
    assert lib.oomb_last_error() != b""


@pytest.mark.parametrize("kw", [
    dict(table=None), dict(q=None), dict(q=Q + 2), dict(qts=100), dict(n_q=0), dict(n_q=-5),
    dict(t0=-1), dict(tstride=10), dict(o=None), dict(lse=None), dict(lse=B + 2),
    dict(scale=0.0), dict(scale=-1.0), dict(scale=float("nan")), dict(sel=T, count=None),
])
def test_fwd_argument_errors(lib, kw):
    assert _fwd(lib, _pool(), **kw) == L.OOMB_ERR_INVALID


def test_null_pool_and_append_errors(lib):
    assert lib.oomb_kv_append(None, T, 64, Q, O, 128, 128, 1, 0, None) == L.OOMB_ERR_INVALID
    p = _pool()
    # table too short for the last token's page
    assert lib.oomb_kv_append(ctypes.byref(p), T, 2, Q, O, 128, 128, 300, 0, None) == L.OOMB_ERR_INVALID
    assert lib.oomb_kv_append(ctypes.byref(p), T, 64, Q, O, 128, 128, -1, 0, None) == L.OOMB_ERR_INVALID
    assert lib.oomb_kv_append(ctypes.byref(p), T, 64, Q, O, 128, 127, 4, 0, None) == L.OOMB_ERR_INVALID
    assert lib.oomb_kv_append(ctypes.byref(p), T, 64, Q, O, 128, 128, 0, 0, None) == L.OOMB_OK


def test_summarize_and_select_errors(lib):
    p = _pool()
    nosum = _pool(k_summary=None)
    assert lib.oomb_page_summarize(ctypes.byref(nosum), T, 64, 0, 4, 512, None) == L.OOMB_ERR_INVALID
    assert lib.oomb_page_summarize(ctypes.byref(p), T, 3, 0, 4, 512, None) == L.OOMB_ERR_INVALID
    assert lib.oomb_page_summarize(ctypes.byref(p), T, 64, 0, 0, 512, None) == L.OOMB_OK
    ws = lib.oomb_select_workspace_bytes(ctypes.byref(p), 4096, 4096)
    assert ws > 0 and ws % 256 == 0

    def sel(**kw):
        a = dict(top_k=4, sel=B, sstride=4, count=B + 256, score=None, sstr=0, ws=0xA00000,
                 wsb=ws)
        a.update(kw)
        return lib.oomb_select_pages(ctypes.byref(p), T, 64, Q, 4096 * 128, 128, 4096, 4096,
                                     a["top_k"], a["sel"], a["sstride"], a["count"], None,
                                     a["score"], a["sstr"], a["ws"], a["wsb"], None)
    assert sel(top_k=-1) == L.OOMB_ERR_INVALID and b"top_k" in lib.oomb_last_error()
    assert sel(sstride=3) == L.OOMB_ERR_INVALID and b"sel rows must hold" in lib.oomb_last_error()
    assert sel(count=None) == L.OOMB_ERR_INVALID
    assert sel(score=B, sstr=10) == L.OOMB_ERR_INVALID and b"score_stride" in lib.oomb_last_error()
    assert sel(wsb=ws - 1) == L.OOMB_ERR_WORKSPACE
    assert sel(ws=0xA00010) == L.OOMB_ERR_WORKSPACE


def test_select_noalloc_host_checks(lib):
    """The allocation-free selection checks every argument as oomb_select_pages does,
    and rejects a call whose workspace would exceed its 8 MiB static scratch, all
    before any HIP call (none is possible here)."""
    p = _pool()

    def sel(t0=4096, tstride=64, **kw):
        a = dict(top_k=4, sel=B, sstride=4, count=B + 256, score=None, sstr=0)
        a.update(kw)
        return lib.oomb_select_pages_noalloc(ctypes.byref(p), T, tstride, Q, 4096 * 128, 128,
                                             4096, t0, a["top_k"], a["sel"], a["sstride"],
                                             a["count"], None, a["score"], a["sstr"], None)
    assert sel(top_k=-1) == L.OOMB_ERR_INVALID and b"top_k" in lib.oomb_last_error()
    assert sel(sstride=3) == L.OOMB_ERR_INVALID and b"sel rows must hold" in lib.oomb_last_error()
    assert sel(count=None) == L.OOMB_ERR_INVALID
    assert sel(tstride=10) == L.OOMB_ERR_INVALID
    # 4 KV heads x 600,000 candidate pages of scores = 9.6 MB > 8 MiB
    t0 = 128 * 600_000
    need = lib.oomb_select_workspace_bytes(ctypes.byref(p), 4096, t0)
    assert need > 8 * 2 ** 20
    assert sel(t0=t0, tstride=600_000 + 32) == L.OOMB_ERR_INVALID
    assert b"static scratch holds 8388608" in lib.oomb_last_error()
    # the 4M-token chunk of 8192 queries fits
    assert lib.oomb_select_workspace_bytes(ctypes.byref(p), 8192, 4_186_112) <= 8 * 2 ** 20


def test_fwd_workspace(lib):
    """The forward's workspace: sized by oomb_fwd_workspace_bytes (empty for a short
    prior context and for a first chunk, whose tiles are too short to cut; for a dense
    4096-query chunk after 126,976 tokens the query tiles are split into key ranges, so
    it is not), and a missing, short or misaligned one is rejected before any launch."""
    p = _pool()
    assert lib.oomb_fwd_workspace_bytes(ctypes.byref(p), 4096, 4096, -1, 0) == 0
    assert lib.oomb_fwd_workspace_bytes(ctypes.byref(p), 4096, 0, -1, 0) == 0
    assert lib.oomb_fwd_workspace_bytes(ctypes.byref(p), 0, 4096, -1, 0) == 0
    t0 = 126976
    need = lib.oomb_fwd_workspace_bytes(ctypes.byref(p), 4096, t0, -1, 0)
    assert need >= 2 * 28 * 4096 * 130 * 4 and need % 256 == 0
    kw = dict(t0=t0, tstride=1024)
    assert _fwd(lib, p, ws=None, wsb=0, **kw) == L.OOMB_ERR_WORKSPACE
    assert _fwd(lib, p, wsb=need - 1, **kw) == L.OOMB_ERR_WORKSPACE
    assert _fwd(lib, p, ws=0xA00010, wsb=need, **kw) == L.OOMB_ERR_WORKSPACE


@pytest.mark.parametrize("name,n_q,t0,sel_stride,splits", [
    ("sparse 1M", 4096, 1048576, 64, (1, 1, 4)),
    ("dense 128K", 4096, 126976, -1, (4, 4, 1)),
    ("sparse 4M", 8192, 4186112, 128, (2, 2, 2)),
])
def test_split_counts_at_the_workloads(lib, name, n_q, t0, sel_stride, splits):
    """The host's load-balance rule picks, at the three benchmark workloads, the split
    counts (forward key ranges, dQ key ranges, dK/dV query-stream splits) that measured
    fastest; they show in the workspace sizes, which are a function of them alone.
    (Where the forward and dQ cut tiles, dense 128K and sparse 4M, only the tiles
    beyond a whole number per CU are cut; the partials keep the uniform layout.)"""
    p = _pool()
    n_fwd, n_dq, n_kv = splits
    hq, hkv, d, page = 28, 4, 128, 128
    n_cand = t0 // page
    pages = (n_cand if sel_stride < 0 else min(sel_stride, n_cand)) + (-(-(t0 + n_q) // page) - n_cand)
    keys = pages * page
    a256 = lambda x: (x + 255) // 256 * 256
    fwd = 0 if n_fwd == 1 else n_fwd * hq * n_q * (d + 2) * 4
    bwd = (a256(hq * n_q * 4) + a256(0 if n_kv == 1 else n_kv * hkv * keys * 2 * d * 4)
           + a256(0 if n_dq == 1 else n_dq * hq * n_q * d * 4))
    # the bf16 dS spill: 2 bytes per pair of every (64-query tile, 128-key block)
    spill = hq * -(-keys // 128) * -(-n_q // 64) * 64 * 128 * 2
    assert lib.oomb_fwd_workspace_bytes(ctypes.byref(p), n_q, t0, sel_stride, 0) == fwd, name
    assert lib.oomb_bwd_workspace_bytes(ctypes.byref(p), n_q, t0, sel_stride, 0) == bwd + spill, name


def test_ds_spill_workspace(lib, monkeypatch):
    """The backward spills dS (and its workspace holds it) only without a window and
    within OOMB_DS_SPILL_MAX_MIB (default 32 GiB; 0 turns it off), read at every call."""
    p = _pool()
    size = lambda t0, w=0: lib.oomb_bwd_workspace_bytes(ctypes.byref(p), 4096, t0, -1, w)
    spill = 28 * 32 * 64 * 64 * 128 * 2  # 4096 local keys: 32 blocks x 64 tiles
    monkeypatch.setenv("OOMB_DS_SPILL_MAX_MIB", "0")
    base, base_w = size(0), size(0, w=1024)  # Delta and the split partials
    assert base < 2 ** 27 and base % 256 == 0
    monkeypatch.delenv("OOMB_DS_SPILL_MAX_MIB")
    assert size(0) == base + spill
    assert size(0, w=1024) == base_w  # no spill with a window
    monkeypatch.setenv("OOMB_DS_SPILL_MAX_MIB", str(spill >> 20))
    assert size(0) == base + spill
    monkeypatch.setenv("OOMB_DS_SPILL_MAX_MIB", str((spill >> 20) - 1))
    assert size(0) == base
    monkeypatch.delenv("OOMB_DS_SPILL_MAX_MIB")
    # dense 128K spills 27.4 GiB, within the default; the dense 262,144-token chunk not
    assert size(126976) > 27 * 2 ** 30
    assert size(262144 - 4096) < 2 ** 30


@pytest.mark.parametrize("name,n_q,t0,sel_stride,plan", [
    # forward (ranges, whole tiles), dQ (ranges, whole tiles), dK/dV (parts, whole blocks)
    ("sparse 1M", 4096, 1048576, 64, (1, 0, 1, 0, 4, 64)),
    ("dense 128K", 4096, 126976, -1, (4, 64, 4, 64, 1, 0)),
    ("sparse 4M", 8192, 4186112, 128, (2, 192, 2, 192, 2, 128)),
])
def test_split_plans_at_the_workloads(lib, name, n_q, t0, sel_stride, plan):
    """The whole load-balance plan at the three benchmark workloads (448, 448 and 896
    query tiles of 256 for the forward and dQ passes; 96, 1024 and 192 key blocks of 128
    per KV head for dK/dV). Sparse 1M: the forward and dQ tiles too short to cut; dK/dV
    keeps its 64 selected blocks per head whole (256, one per CU) and cuts the chunk's
    32 in four. Dense 128K: 256 of the 448 tiles whole (64 per head), the rest in four
    ranges; the 4,128 key blocks need no cut. Sparse 4M: 768 of 896 tiles whole, the
    rest in two ranges; the 128 selected blocks per head whole (two per CU), the chunk's
    64 in two parts."""
    p = _pool()
    out = (ctypes.c_int32 * 6)()
    assert lib.oomb_split_plan(ctypes.byref(p), n_q, t0, sel_stride, 0, out) == L.OOMB_OK, name
    assert tuple(out) == plan, name


def test_split_plan_overrides_and_errors(lib, monkeypatch):
    """The environment fixes a plan (whole clamped to the tiles or blocks per head; no
    whole count when a pass is not cut), and a bad geometry is rejected."""
    p = _pool()
    out = (ctypes.c_int32 * 6)()
    for var, val in (("OOMB_FWD_SPLITS", "3"), ("OOMB_FWD_WHOLE", "1000"), ("OOMB_DQ_SPLITS", "1"),
                     ("OOMB_DQ_WHOLE", "5"), ("OOMB_DKDV_SPLITS", "2"), ("OOMB_DKDV_WHOLE", "7")):
        monkeypatch.setenv(var, val)
    assert lib.oomb_split_plan(ctypes.byref(p), 4096, 1048576, 64, 0, out) == L.OOMB_OK
    assert tuple(out) == (3, 7 * 16, 1, 0, 2, 7)  # 16 tiles of 256 for each of 7 query heads
    assert lib.oomb_split_plan(ctypes.byref(p), 0, 4096, -1, 0, out) == L.OOMB_ERR_INVALID
    assert lib.oomb_split_plan(ctypes.byref(p), 4096, 4096, -1, 0, None) == L.OOMB_ERR_INVALID


def test_window_arguments(lib):
    """A window is local attention: negative windows and windows combined with a page
    selection are rejected before any launch; the workspace queries reject them too."""
    p = _pool()
    assert _fwd(lib, p, window=-1) == L.OOMB_ERR_INVALID
    assert b"window" in lib.oomb_last_error()
    assert _fwd(lib, p, window=128, sel=0xB00000, sstride=4, count=0xB10000) == L.OOMB_ERR_INVALID
    assert b"selection" in lib.oomb_last_error()
    assert lib.oomb_fwd_workspace_bytes(ctypes.byref(p), 4096, 4096, -1, -5) == 0
    assert lib.oomb_bwd_workspace_bytes(ctypes.byref(p), 4096, 4096, 8, 128) == 0
    assert lib.oomb_bwd_workspace_bytes(ctypes.byref(p), 4096, 4096, -1, 128) > 0


def test_bwd_errors(lib):
    p = _pool()
    nograd = _pool(dk_pool=None)
    need = lib.oomb_bwd_workspace_bytes(ctypes.byref(p), 4096, 4096, -1, 0)
    assert need >= 28 * 4096 * 4 and need % 256 == 0
    assert lib.oomb_bwd_workspace_bytes(ctypes.byref(p), 0, 4096, -1, 0) == 0

    def bwd(pool, **kw):
        a = dict(gtable=T, gts=64, dq=B, dqhs=4096 * 128, dqts=128, ws=0xA00000, wsb=need)
        a.update(kw)
        return lib.oomb_paged_chunk_attn_bwd(
            ctypes.byref(pool), T, 64, a["gtable"], a["gts"], Q, 4096 * 128, 128, 4096, 4096,
            None, 0, None, a.get("window", 0), 0.088, O, 4096 * 128, 128, O, 4096 * 128, 128, B,
            a["dq"], a["dqhs"], a["dqts"], a["ws"], a["wsb"], None)
    assert bwd(nograd) == L.OOMB_ERR_INVALID
    assert bwd(p, gtable=None) == L.OOMB_ERR_INVALID
    assert bwd(p, gts=5) == L.OOMB_ERR_INVALID
    assert bwd(p, dqts=130) == L.OOMB_ERR_INVALID
    assert bwd(p, wsb=need - 4) == L.OOMB_ERR_WORKSPACE


def test_copy_pages_sdma_refuses_scattered_lists(lib):
    """The copy-engine page list is for long runs of consecutive pages: a list of 64
    scattered pages (64 runs, more than max(16, 64 / 16)) is refused before any HIP call,
    pointing to the gather kernel."""
    n = 64
    scattered = (ctypes.c_int32 * n)(*[3 * i for i in range(n)])
    same = (ctypes.c_int32 * n)(*[3 * i for i in range(n)])
    st = lib.oomb_copy_pages_sdma(0x100000, 0x200000, 32768, 4096, 4096, scattered, same, n, None)
    assert st == L.OOMB_ERR_INVALID and b"oomb_copy_pages" in lib.oomb_last_error()
    # 16 runs of 4 pages are still accepted by the run count (the call then checks the
    # pointers, which here fails with a different message: no GPU, fake addresses)
    runs = (ctypes.c_int32 * n)(*[16 * (i // 4) + i % 4 for i in range(n)])
    st = lib.oomb_copy_pages_sdma(0x100000, 0x200000, 32768, 4096, 4096, runs, runs, n, None)
    assert b"runs" not in lib.oomb_last_error()
