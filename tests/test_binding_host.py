"""Host-side logic of the Python binding, on the CPU (no kernel runs: the library
call itself is replaced by a recorder).

- Every tensor the binding creates for a call (selection, counts, outputs, workspace)
  is created while the call's stream is current, so its fills are ordered before the
  library's kernels on that stream and the caching allocator hands the memory only to
  later work on that stream.
- The optional table checks (OOMB_CHECK_TABLES=1) reject a page table that maps two
  logical pages of a call onto one physical page, and selections that are not
  strictly ascending candidate ids.
"""
import contextlib

import pytest
import torch

import paged_chunk_attention_amd as pca
from paged_chunk_attention_amd import binding as B


class _FakeStream:
    cuda_stream = 0x1234


@pytest.fixture
def recorder(monkeypatch):
    """Replace torch.cuda.stream with a context that marks 'inside the call stream',
    _new with a wrapper that records whether it ran inside, and the library call with
    a recorder of the same."""
    state = {"inside": 0, "allocs": [], "calls": []}

    @contextlib.contextmanager
    def fake_stream(stream):
        assert isinstance(stream, _FakeStream)
        state["inside"] += 1
        try:
            yield
        finally:
            state["inside"] -= 1

    real_new = B._new

    def new(kind, shape, dtype, device, fill=None):
        state["allocs"].append(state["inside"] > 0)
        if dtype == torch.uint8:      # CPU memory is not 256-byte aligned: align a slice
            raw = real_new(kind, shape + 256, dtype, device, fill)
            off = (-raw.data_ptr()) % 256
            return raw[off:off + shape]
        return real_new(kind, shape, dtype, device, fill)

    def call(name, *args):
        state["calls"].append((name, state["inside"] > 0, args[-1].value))

    monkeypatch.setattr(torch.cuda, "stream", fake_stream)
    monkeypatch.setattr(B, "_new", new)
    monkeypatch.setattr(B, "call", call)
    return state


def _pool(hq=4, hkv=2, P=16, D=128, n=40):
    return pca.PagedPool(n, P, D, hq, hkv, torch.bfloat16, "cpu")


def _table(hkv, per_head):
    return torch.arange(hkv * per_head, dtype=torch.int32).reshape(hkv, per_head)


def test_allocations_happen_on_the_call_stream(recorder):
    pool = _pool()
    table = _table(2, 20)
    q = torch.zeros(4, 48, 128, dtype=torch.bfloat16)
    s = _FakeStream()
    sel, count = pca.oomb_select_pages(pool, table, q, 160, 3, stream=s)
    o, lse = pca.oomb_paged_chunk_attn_fwd(pool, table, q, 160, sel, count, stream=s)
    pca.oomb_paged_chunk_attn_bwd(pool, table, table, q, 160, sel, count, o, q, lse, stream=s)
    assert recorder["allocs"] and all(recorder["allocs"])
    assert [c[0] for c in recorder["calls"]] == [
        "oomb_select_pages", "oomb_paged_chunk_attn_fwd", "oomb_paged_chunk_attn_bwd"]
    assert all(inside and handle == s.cuda_stream for _, inside, handle in recorder["calls"])
    # the selection starts as -1 and the counts as 0 (filled on the call's stream)
    assert bool((sel == -1).all()) and bool((count == 0).all())


def test_check_page_tables_accepts_permutation_rejects_duplicates():
    perm = torch.randperm(60, generator=torch.Generator().manual_seed(0)).to(torch.int32)
    table = perm.reshape(3, 20)
    B.check_page_tables(table, 20, 60)
    B.check_page_tables(table, [[0, 5, 19], [1], []], 60)
    dup = table.clone()
    dup[2, 7] = dup[0, 3]                               # across KV heads
    with pytest.raises(ValueError, match="mapped 2 times"):
        B.check_page_tables(dup, 20, 60)
    # the duplicate is harmless when one of its logical pages is not touched
    B.check_page_tables(dup, [list(range(20)), list(range(20)), [0, 1]], 60)
    with pytest.raises(ValueError, match="mapped"):
        B.check_page_tables(dup, [[3], [], [7]], 60)
    bad = table.clone()
    bad[1, 1] = 60
    with pytest.raises(ValueError, match="outside"):
        B.check_page_tables(bad, 20, 60)
    with pytest.raises(ValueError, match="columns"):
        B.check_page_tables(table, 21, 60)


def test_check_selection():
    count = torch.tensor([3, 2], dtype=torch.int32)
    B.check_selection(torch.tensor([[1, 4, 9], [0, 2, -1]], dtype=torch.int32), count, 10)
    for sel in ([[1, 4, 4], [0, 2, -1]],      # repeated id
                [[4, 1, 9], [0, 2, -1]],      # not ascending
                [[1, 4, 10], [0, 2, -1]],     # not a candidate
                [[1, 4, 9], [-1, 2, 0]]):
        with pytest.raises(ValueError):
            B.check_selection(torch.tensor(sel, dtype=torch.int32), count, 10)
    # count is clamped to the candidates, as the kernels clamp it
    B.check_selection(torch.tensor([[0, 1, 7]], dtype=torch.int32),
                      torch.tensor([3], dtype=torch.int32), 2)


def test_attended_logical_pages():
    sel = torch.tensor([[5, 1, 3], [2, 0, 4]], dtype=torch.int32)
    count = torch.tensor([2, 3], dtype=torch.int32)
    # t0 = 100, P = 16: pages 0..5 are candidates, the chunk of 40 covers pages 6..8
    got = B.attended_logical_pages(2, 16, 100, 40, sel, count)
    assert got == [[1, 5, 6, 7, 8], [0, 2, 4, 6, 7, 8]]
    assert B.attended_logical_pages(1, 16, 100, 40) == [[0, 1, 2, 3, 4, 5, 6, 7, 8]]
    # window 30: the first query (position 100) reaches back to position 71, page 4
    assert B.attended_logical_pages(1, 16, 100, 40, window=30) == [[4, 5, 6, 7, 8]]


def test_debug_checks_run_before_the_call(recorder, monkeypatch):
    pool = _pool()
    table = _table(2, 20)
    q = torch.zeros(4, 48, 128, dtype=torch.bfloat16)
    s = _FakeStream()
    dup = table.clone()
    dup[1, 10] = dup[0, 11]         # both among the chunk's own pages (t0 = 160, P = 16)
    monkeypatch.setenv("OOMB_CHECK_TABLES", "1")
    with pytest.raises(ValueError, match="mapped"):
        pca.oomb_paged_chunk_attn_fwd(pool, dup, q, 160, stream=s)
    with pytest.raises(ValueError, match="mapped"):
        pca.oomb_kv_append(pool, dup, q[:2], q[:2], 160, stream=s)
    bad_sel = torch.tensor([[3, 3], [0, 1]], dtype=torch.int32)
    with pytest.raises(ValueError, match="ascending"):
        pca.oomb_paged_chunk_attn_fwd(pool, table, q, 160, bad_sel,
                                      torch.tensor([2, 2], dtype=torch.int32), stream=s)
    assert recorder["calls"] == []
    pca.oomb_paged_chunk_attn_fwd(pool, table, q, 160, stream=s)  # a good table passes
    assert [c[0] for c in recorder["calls"]] == ["oomb_paged_chunk_attn_fwd"]
    monkeypatch.setenv("OOMB_CHECK_TABLES", "0")
    pca.oomb_paged_chunk_attn_fwd(pool, dup, q, 160, stream=s)  # unchecked when off
