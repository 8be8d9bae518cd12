"""Writing new keys into the paged index cache (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Before the indexer can score a token's key, the key is quantised and stored
in the paged cache at the token's slot: on the DeepSeek-V3.2 indexer backend
page the metadata carries an int64 ``slot_mapping`` per token (and its
compressed variant), and the MiniMax-M3 mono runner page documents the same
int64 page slots for its K/V and index caches.  Slot ``s`` is row
``s % page_size`` of physical page ``s // page_size``; a negative slot marks a
token that is not stored (padding).  The row layouts are those the cache
readers use (``oracle.cache``): fp8 = ``D`` e4m3fn codes + fp32 per-token scale,
MXFP4 = ``D/2`` packed e2m1 (even element in the low nibble) + ``D/32`` ue8m0
block scales (``_gather_workspace_shapes`` on the glm5next page).

The pages do not print the quantiser; the reading taken here is the one the
workload definition names -- "per-token absmax fp32 scale" for fp8 and OCP MX
block scaling for MXFP4:

* fp8, per token: ``amax = max_d |k_d|`` (the bf16 key read exactly as fp32);
  ``scale = amax / 448`` rounded to fp32 (``1`` when the row is all zeros);
  ``x_d = k_d / scale`` rounded to fp32, clipped to [-448, 448], then rounded
  to the nearest e4m3fn value, ties to the even code; the sign bit is the
  key's (so -0.0 stays -0.0).  Both roundings are fp32 because the decision
  of each code is taken in the same precision the kernel takes it.
* MXFP4, per 32-element block: ``e = floor(log2 amax) - 2`` (2 being the
  largest e2m1 exponent), at least -127 (an all-zero block gets -127),
  stored as the ue8m0 byte ``e + 127``; elements ``x_d = k_d * 2^-e``
  (exact), magnitudes clipped to 6 and rounded to the nearest e2m1 value,
  ties to the even code, sign bit from the key.

Pins (tests/test_oracle_cache_write.py): the e4m3 encoder against torch's
float -> float8_e4m3fn cast on every midpoint between codes and its
neighbours; the e2m1 encoder against a hand-derived tie table; row
quantisers against closed forms (all-zero rows, the absmax element mapping
to +-448, block exponents of chosen amax values) and against the quantisation
error bounds after decoding with ``oracle.cache``; the fp8 rows against the
workload generator's independent torch-cast encoding; slots against a
block-table read-back, negative and out-of-range slots skipped.
"""

from __future__ import annotations

import numpy as np

from . import formats

FP8_MAX = 448.0
E2M1_MAX = 6.0

# Non-negative finite code values in code order (ascending for both formats).
_E4M3_VALUES = formats.e4m3(np.arange(0x7F, dtype=np.uint8))   # codes 0x00..0x7E
_E2M1_VALUES = formats.e2m1(np.arange(8, dtype=np.uint8))        # codes 0..7


def _nearest_code(mag: np.ndarray, values: np.ndarray) -> np.ndarray:
    """Index of the nearest entry of ascending `values` to each magnitude
    (within [0, values[-1]]), ties to the even index."""
    hi = np.clip(np.searchsorted(values, mag, side="left"), 0, len(values) - 1)
    lo = np.clip(hi - 1, 0, len(values) - 1)
    d_lo = mag - values[lo]
    d_hi = values[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    return np.where(pick_hi, hi, lo)


def e4m3_encode(x) -> np.ndarray:
    """Finite values with |x| <= 448 -> e4m3fn codes (round to nearest,
    ties to even; sign bit from x)."""
    x = np.asarray(x, dtype=np.float64)
    code = _nearest_code(np.abs(x), _E4M3_VALUES).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def e2m1_encode(x) -> np.ndarray:
    """Finite values with |x| <= 6 -> 4-bit e2m1 codes (nearest, ties to
    even; sign bit from x)."""
    x = np.asarray(x, dtype=np.float64)
    code = _nearest_code(np.abs(x), _E2M1_VALUES).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x8, code).astype(np.uint8)


def fp8_rows(k_bits: np.ndarray) -> np.ndarray:
    """bf16 keys [n, D] (uint16 bit patterns) -> fp8 cache rows [n, D + 4]."""
    k = formats.bf16(k_bits).astype(np.float32)             # exact
    n, D = k.shape
    amax = np.abs(k).max(axis=1) if D else np.zeros(n, np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        scale = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
        x = (k / scale[:, None]).astype(np.float32)            # fp32 division, RNE
    x = np.clip(x.astype(np.float64), -FP8_MAX, FP8_MAX)
    out = np.empty((n, D + 4), dtype=np.uint8)
    out[:, :D] = e4m3_encode(x)
    out[:, D:] = scale.astype("<f4").view(np.uint8).reshape(n, 4)
    return out


def mx_block_exponent(amax) -> np.ndarray:
    """Shared exponent e of a block: floor(log2 amax) - 2, at least -127
    (-127 for amax = 0)."""
    a = np.asarray(amax, dtype=np.float64)
    m, ex = np.frexp(a)                  # a = m 2^ex, m in [0.5, 1): floor(log2 a) = ex - 1
    e = np.where(a > 0, ex.astype(np.int64) - 1 - 2, -127)
    return np.maximum(e, -127)


def mxfp4_rows(k_bits: np.ndarray) -> np.ndarray:
    """bf16 keys [n, D] (uint16 bit patterns) -> MXFP4 cache rows
    [n, D/2 + D/32]."""
    k = formats.bf16(k_bits)                                   # float64, exact
    n, D = k.shape
    assert D % 32 == 0
    blocks = k.reshape(n, D // 32, 32)
    e = mx_block_exponent(np.abs(blocks).max(axis=2))          # [n, D/32]
    x = blocks * np.exp2(-e.astype(np.float64))[:, :, None]    # exact
    x = np.clip(x, -E2M1_MAX, E2M1_MAX)
    nib = e2m1_encode(x).reshape(n, D)
    out = np.empty((n, D // 2 + D // 32), dtype=np.uint8)
    out[:, : D // 2] = nib[:, 0::2] | (nib[:, 1::2] << 4)
    out[:, D // 2 :] = (e + 127).astype(np.uint8)
    return out


def quantize_rows(k_bits: np.ndarray, fmt: str) -> np.ndarray:
    if fmt == "fp8":
        return fp8_rows(k_bits)
    if fmt == "mxfp4":
        return mxfp4_rows(k_bits)
    raise ValueError(fmt)


def write(cache: np.ndarray, k_bits: np.ndarray, slots: np.ndarray, *, fmt: str, page_size: int,
          page_bytes: int) -> tuple[np.ndarray, bool]:
    """Copy of the flat cache bytes with token t's quantised row stored at
    slot slots[t].  Negative slots are skipped; slots at or past the pool's
    num_pages * page_size are skipped and reported (second result True).
    Slots are assumed distinct."""
    flat = np.array(cache, dtype=np.uint8).reshape(-1)
    num_pages = flat.size // page_bytes
    rows = quantize_rows(np.asarray(k_bits, dtype=np.uint16), fmt)
    rb = rows.shape[1]
    bad = False
    for t, s in enumerate(np.asarray(slots, dtype=np.int64)):
        if s < 0:
            continue
        if s >= num_pages * page_size:
            bad = True
            continue
        start = (s // page_size) * page_bytes + (s % page_size) * rb
        flat[start : start + rb] = rows[t]
    return flat, bad
