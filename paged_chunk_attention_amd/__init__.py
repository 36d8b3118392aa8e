"""Paged chunk attention for AMD MI355X (gfx950).

The hot path of OOMB-style chunk-recurrent long-context training as a small HIP
library (liboomb.so, C ABI in include/oomb.h) plus this thin torch binding:
KV append into fixed-size pages, per-page key summaries, top-k page selection,
chunk attention forward, and the recomputing backward that writes dQ and adds
dK/dV into a paged fp32 gradient pool.
"""
from .binding import (  # noqa: F401
    PagedPool,
    bwd_workspace_bytes,
    oomb_add_pages_f32,
    oomb_copy_pages,
    oomb_copy_pages_sdma,
    oomb_fetch_selected,
    fwd_workspace_bytes,
    kernel_timer,
    oomb_kv_append,
    oomb_page_summarize,
    oomb_page_summarize_mean,
    oomb_paged_chunk_attn_bwd,
    oomb_paged_chunk_attn_bwd_tiled,
    oomb_paged_chunk_attn_fwd,
    oomb_paged_chunk_attn_fwd_tiled,
    oomb_rope,
    oomb_select_pages,
    oomb_select_pages_mean,
    oomb_select_pages_noalloc,
    oomb_select_pages_tiled,
    select_tiled_workspace_bytes,
    tile_row_length,
    select_workspace_bytes,
    split_plan,
)
from ._lib import LIB_PATH, OombError, lib  # noqa: F401
