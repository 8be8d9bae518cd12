"""Top-k selection for one row (oracle side).

Given a row of ``L`` scores and ``k``:

* ``L == 0`` (padded row)  -> k entries of -1  (empty output; the glm5next
  page's "pad rows ... empty tail");
* ``L <= k``               -> 0, 1, ..., L-1, then -1 padding: every key is
  selected, which is the exact causal fill of
  ``_fill_short_decode_causal_indices`` on the glm5next page, applied per row;
* ``L > k``                -> the k indices of the largest scores, ties
  between equal scores going to the lower index.

Output rows hold indices in ascending order, -1 padded.  Equality is float
equality, so -0.0 and +0.0 are the same score.

The selection is a full stable sort (numpy ``lexsort`` on (index, -score)),
i.e. the definition itself.  Pins (tests/test_oracle_topk.py): a brute-force
pairwise-rank selection on random tiny rows with many ties, the +-0 example
E2, the invariants (indices < L, no duplicates, full causal rows, padded rows
empty) and the hand example E1.
"""

from __future__ import annotations

import numpy as np


def topk_row(scores, L: int, k: int) -> np.ndarray:
    out = np.full(k, -1, dtype=np.int32)
    if L <= 0:
        return out
    if L <= k:
        out[:L] = np.arange(L, dtype=np.int32)
        return out
    s = np.asarray(scores, dtype=np.float64)[:L] + 0.0   # -0.0 -> +0.0
    order = np.lexsort((np.arange(L), -s))           # by -score, then index
    chosen = np.sort(order[:k])
    out[:] = chosen.astype(np.int32)
    return out
