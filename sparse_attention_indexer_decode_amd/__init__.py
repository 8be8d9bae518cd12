"""Sparse-attention lightning indexer for MI355X (gfx950).

Paged fp8 / MXFP4 index-cache scoring and top-k selection, as a C-ABI HIP
library (``libidx.so``, declared in ``include/idx.h``) with a thin ctypes
binding.  PyTorch supplies device memory and streams only.
"""

from .binding import (  # noqa: F401
    Cache,
    IdxError,
    Rows,
    EXPORTED,
    IDX_OP_CACHE_WRITE,
    IDX_OP_DECODE_TOPK,
    IDX_OP_LOGITS,
    IDX_OP_TOPK,
    IDX_OP_POOL_TOPK,
    IDX_OP_DECODE_POOL_TOPK,
    IdxPools,
    IDX_DEV_BAD_PAGE,
    IDX_DEV_BAD_SLOT,
    idx_cache_write,
    idx_decode_topk,
    idx_decode_topk_noalloc,
    idx_decode_pool_topk,
    idx_pool_topk,
    pools,
    idx_logits_paged,
    idx_prefill_chunks,
    idx_read_device_status,
    idx_topk,
    idx_version,
    idx_workspace_bytes,
    load,
    new_workspace,
)
