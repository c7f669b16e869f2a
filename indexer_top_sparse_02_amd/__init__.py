"""MI355X-native sparse indexer + Top-K + sparse MLA attention.

The compute lives in libsia.so (hand-written HIP for gfx950, C ABI in
include/sia.h); this package is its thin torch binding.
"""
from ._lib import (  # noqa: F401
    DEVSTATUS_BAD_INDEX, DEVSTATUS_BAD_PAGE, DEVSTATUS_BAD_SEQ, DEVSTATUS_ROW_TOO_LONG, SCHED_AUTO,
    MLA_NOALLOC_MAX_BYTES, SCHED_HEAVY_FIRST, SCHED_NAIVE, SCHED_ZIGZAG, SiaError, lib, mla_workspace_size,
    indexer_prepare, indexer_workspace_size, new_workspace, read_device_status, sparse_indexer_scores,
    quantize_mxfp8, sparse_indexer_scores_mxfp8, sparse_indexer_topk, sparse_indexer_topk_mxfp8,
    sparse_indexer_topk_traced, sparse_mla_attention, sparse_mla_attention_noalloc, sparse_topk_from_scores,
    visible_max, version,
    zigzag_assign,
)
