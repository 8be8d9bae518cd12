"""Reading keys out of the paged index cache (oracle side).

Key ``t`` of request ``b`` is slot ``t % page_size`` of physical page
``block_table[b, t // page_size]`` (the block-table addressing of the
DeepSeek-V3.2 indexer backend page: ``(num_blocks, block_size, head_size)``
cache, one int32 block table row per request).  Its row starts at byte
``page * page_bytes + slot * row_bytes`` of the cache (token-major rows; the
MXFP4 view of ``kv_cache_as_quant_view`` on the glm5next page has exactly this
token stride).

Dequantised value of element d:

* fp8:   e4m3(byte d) * f32(bytes D..D+3)
* mxfp4: e2m1(nibble d) * 2^(ue8m0(byte D/2 + d // 32) - 127), nibble d being
  the low nibble of byte d // 2 for even d and the high nibble for odd d.

Everything is exact in float64.  Pins: tests/test_oracle_score.py (hand
examples E1 and E3 written byte by byte; the MXFP4 nibble order).
"""

from __future__ import annotations

import numpy as np

from . import formats


def row_bytes(fmt: str, head_dim: int) -> int:
    return head_dim + 4 if fmt == "fp8" else head_dim // 2 + head_dim // 32


def key_rows(cache: np.ndarray, block_table: np.ndarray, b: int, L: int, *, fmt: str,
             head_dim: int, page_size: int, page_bytes: int) -> np.ndarray:
    """Raw bytes of keys 0..L-1 of request b, shape [L, row_bytes]."""
    rb = row_bytes(fmt, head_dim)
    flat = np.asarray(cache, dtype=np.uint8).reshape(-1)
    t = np.arange(L, dtype=np.int64)
    page = np.asarray(block_table, dtype=np.int64)[b, t // page_size]
    start = page * page_bytes + (t % page_size) * rb
    return flat[start[:, None] + np.arange(rb, dtype=np.int64)[None, :]]


def dequantize(rows: np.ndarray, *, fmt: str, head_dim: int) -> np.ndarray:
    """Token rows [n, row_bytes] -> exact float64 keys [n, head_dim]."""
    D = head_dim
    if fmt == "fp8":
        vals = formats.e4m3(rows[:, :D])
        scale = formats.f32le(rows[:, D : D + 4])
        return vals * scale[:, None]
    if fmt == "mxfp4":
        packed = rows[:, : D // 2]
        nib = np.empty((rows.shape[0], D), dtype=np.uint8)
        nib[:, 0::2] = packed & 0x0F
        nib[:, 1::2] = packed >> 4
        vals = formats.e2m1(nib)
        scales = formats.ue8m0(rows[:, D // 2 : D // 2 + D // 32])
        return vals * np.repeat(scales, 32, axis=1)
    raise ValueError(fmt)


def keys(wl, b: int, L: int) -> np.ndarray:
    """Exact float64 keys 0..L-1 of request b of a workload-like object."""
    rows = key_rows(wl.cache, wl.block_table, b, L, fmt=wl.fmt, head_dim=wl.head_dim,
                    page_size=wl.page_size, page_bytes=wl.page_bytes)
    return dequantize(rows, fmt=wl.fmt, head_dim=wl.head_dim)
