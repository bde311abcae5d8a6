"""pkv: paged K/V attention (decode, verify and prefill windows), greedy
speculative accept, the cache append / rollback around them, and the page
allocator, for AMD MI355X.

The compute lives in libpkv.so (hand-written HIP for gfx950, C ABI in
include/pkv.h). This package is its thin Python binding; importing it loads
the library and fails loudly when it has not been built.
"""

from ._lib import (  # noqa: F401
    PKV_PAGE_SIZE, PKV_MAX_Q_LEN, PKV_MAX_ROWS, PKV_OK, PKV_ERR_NULL, PKV_ERR_SHAPE,
    PKV_ERR_WORKSPACE, PKV_ERR_HIP, PKV_EFLAG_PAGE, PKV_EFLAG_QLEN, PKV_EFLAG_ROWS, PKV_EFLAG_SPACE,
    EXPORTS, LIB,
    LIB_PATH, PkvError, pkv_attn_shape, pkv_accept_shape, attn_shape, accept_shape,
    pkv_attn_workspace_bytes, pkv_attn_workspace_init, new_attn_workspace, pkv_attn_fwd,
    pkv_attn_check_errors, pkv_accept_workspace_bytes, new_accept_workspace, pkv_accept,
    pkv_window_next, pkv_status_string, pkv_version, pkv_kv_shape, kv_shape, pkv_kv_workspace_bytes,
    new_kv_workspace, pkv_kv_append, pkv_kv_rollback, pkv_kv_check_errors,
    PKV_ERR_SPACE, PKV_ERR_STATE, pkv_pool_create, pkv_pool_destroy, pkv_pool_stats, pkv_pool_admit,
    pkv_pool_alloc, pkv_pool_retain, pkv_pool_release, pkv_pool_defrag, pkv_pool_copy_pages, pkv_table_remap,
    pkv_attn_shared_workspace_bytes, new_attn_shared_workspace, pkv_attn_fwd_shared, pkv_attn_plan,
    pkv_shared_prefix_pages, pkv_q8_encode, pkv_attn_fwd_q8, pkv_q4_encode, pkv_attn_fwd_q4,
    pkv_kv_append_q8, pkv_kv_append_q4, pkv_pool_copy_page_bytes,
    PKV_ERR_SCRATCH, PKV_ACCEPT_SCRATCH_BYTES, pkv_accept_noalloc,
)
