"""MISA (Mixture of Indexer Sparse Attention) indexer for AMD Instinct MI355X.

The compute path is libmisa.so (hand-written HIP kernels for gfx950 behind a
C ABI, include/misa.h); this package is its Python binding plus the seeded
synthetic input generator.
"""
from ._lib import (  # noqa: F401
    EXPORTED, MAX_TOPK, MisaError, MisaShape, dsa_dense_logits, load, make_shape, misa_indexer,
    misa_indexer_workspace_bytes, misa_indexer_workspace_min_bytes, misa_pool_keys, misa_route_heads,
    misa_sparse_head_logits, misa_topk,
    misa_topk_workspace_bytes, misa_sparse_head_topk, misa_sparse_head_topk_workspace_bytes,
    misa_quantize_q, misa_sparse_head_logits_q8, misa_sparse_head_topk_q8, dsa_dense_logits_q8,
    PooledCache, misa_pool_keys_cached, misa_indexer_cached, misa_indexer_cached_workspace_bytes,
    misa_prefill_chunked, misa_prefill_workspace_bytes, misa_indexer_q8, misa_indexer_q8_workspace_bytes,
    misa_gather_keys_paged, status_str, misa_indexer_noalloc, NOALLOC_SCRATCH_BYTES, MISA_ERR_SCRATCH,
    misa_profile_stage, STAGES, misa_indexer_paged, misa_indexer_paged_workspace_bytes,
)
