"""The indexer score (oracle side).

For one query row with bf16 queries q[h, :] (h < H) and fp32 head weights
w[h], and keys k_t dequantised exactly:

    logit[t] = sum_h w[h] * max(q[h, :] . k_t, 0)          for t < L

With an fp8 key k_t = scale_t * code_t and scale_t >= 0 this is
``scale_t * sum_h w_h * relu(q_h . code_t)``; the oracle evaluates the
left-hand form on the dequantised keys, which is the same number for every
non-negative scale (per-token absmax scales always are) and is also the MXFP4
definition, where the block scales sit inside the dot product.

Precision: q, w and the keys are exact in float64; each product q*k has at
most 8 + 4 (or 8 + 2 + scale) significant bits and the float64 sums add an
error of order 1e-15 relative -- far below the 2e-3 / 1e-4 tolerance used
against the GPU.  The dot products are one numpy matmul (a library
primitive); relu, weighting and the head sum follow the formula literally.

Pins (tests/test_oracle_score.py): brute force with Python ``Fraction``
(exact rationals) on tiny inputs; H=1, w=1, positive dots reduce to a plain
matrix-vector product; hand-worked 2-head examples E1 (fp8) and E3 (MXFP4).
"""

from __future__ import annotations

import numpy as np

from . import formats


def logits(q_bits: np.ndarray, w: np.ndarray, keys: np.ndarray) -> np.ndarray:
    """q_bits uint16 [H, D] (bf16), w float32 [H], keys float64 [L, D]
    -> float64 [L]."""
    q = formats.bf16(q_bits)                       # [H, D]
    wh = np.asarray(w, dtype=np.float32).astype(np.float64)
    dots = keys @ q.T                              # [L, H]
    return (np.maximum(dots, 0.0) * wh[None, :]).sum(axis=1)
