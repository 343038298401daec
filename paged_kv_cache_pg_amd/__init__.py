"""Paged KV-cache attention for AMD MI355X (gfx950).

The compute lives in libpagedattn.so (hand-written HIP kernels behind a C ABI,
declared in include/paged_attn.h); ``binding`` marshals arguments to it.
"""
from .binding import (  # noqa: F401
    PAGED_BF16,
    PAGED_EFULL,
    PAGED_OK,
    PAGED_F32,
    PAGED_FP8_E4M3,
    PagedError,
    make_kv,
    make_pg,
    paged_attn_decode,
    paged_attn_decode_workspace,
    paged_attn_decode_window,
    paged_attn_decode_window_workspace,
    paged_attn_prefill,
    paged_attn_prefill_workspace,
    paged_block_scores_topk,
    paged_kv_append,
    paged_pool_alloc,
    paged_pool_blocks,
    paged_pool_claim_run,
    paged_pool_free,
    paged_pool_free_count,
    paged_pool_init,
    paged_pool_release_run,
    paged_pool_state_bytes,
    paged_row_offsets,
    paged_rows_gather,
    paged_rows_store,
    paged_sparse_attn,
    paged_sparse_attn_workspace,
    paged_topk_workspace,
    strerror,
)
from .layout import ArenaLayout  # noqa: F401
