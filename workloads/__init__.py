"""Seeded synthetic inputs for the indexer scoring + top-k path.

This package only *makes inputs*: a paged, quantised index cache, block
tables, per-request lengths, bf16 queries and fp32 head weights, and the new
bf16 key tokens and int64 slots of a cache write.  It holds
none of the scoring or selection arithmetic, so both the CPU oracle (via the
tests) and the GPU path can be fed the very same bytes.
"""

from .gen import (  # noqa: F401
    Workload,
    build_decode,
    build_prefill,
    cache_write_inputs,
    CacheWriteInputs,
    config,
    CONFIG_NAMES,
    encode_fp8_rows,
    encode_mxfp4_rows,
    row_bytes_for,
)
