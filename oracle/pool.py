"""Pool-level (block-level) top-k selection for one row (oracle side).

The pages name this variant without defining its arithmetic: the glm5next
``sparse_indexer`` page runs ``pool_topk`` on the logits of the padded
decode grid (one row per token, token-granular length pos + 1, padded rows
0 = empty tail), then ``expand_pools_and_append_tail`` turns the chosen
pools back into token positions and appends the row's tail tokens; the
MiniMax-M3 mono runner page configures its indexer with ``topk_blocks``,
``init_blocks`` and ``local_blocks``.  Reading taken here (the plainest one
those names support):

* a pool is ``pool_size`` consecutive key positions: pool p holds keys
  [p B, p B + B);  a row of L keys has n = L // B complete pools and a tail
  of the last L - n B keys (fewer than B, possibly none);
* a pool's score is the largest logit of its keys;
* the first ``init_pools`` and the last ``local_pools`` complete pools are
  always kept, and count toward ``topk_pools``; the remaining
  ``topk_pools - kept`` places go to the highest-scoring other complete
  pools, ties going to the lower pool index (the token top-k's rule);
* when n <= topk_pools every complete pool is kept (the pool form of the
  exact causal fill);
* the output lists the kept pools' key positions in ascending order, then
  the tail keys, -1 padded to (topk_pools + 1) * pool_size entries; the kept
  pool indices go to a second list, ascending, -1 padded to topk_pools;
  a padded row (L = 0) is all -1.

Pins (tests/test_oracle_pool.py): a hand-worked row (tests/golden/pool_topk.json);
pool size 1 with no kept pools is the token top-k; brute force by pairwise
rank on random tiny rows with ties; the invariants (ascending, unique,
< L, the kept pools present, the tail present, padded rows empty).
"""

from __future__ import annotations

import numpy as np


def forced_pools(n_full: int, init_pools: int, local_pools: int):
    """(first candidate pool, end of candidates): the kept prefix is pools
    [0, a), the kept suffix [e, n_full); candidates [a, e)."""
    a = min(init_pools, n_full)
    z = min(local_pools, n_full - a)
    return a, n_full - z


def pool_topk_row(scores, L: int, pool_size: int, topk_pools: int, init_pools: int, local_pools: int):
    """-> (tokens int32 [(topk_pools + 1) * pool_size], pools int32 [topk_pools])."""
    B = pool_size
    assert B >= 1 and init_pools >= 0 and local_pools >= 0 and init_pools + local_pools <= topk_pools
    tokens = np.full((topk_pools + 1) * B, -1, dtype=np.int32)
    pools_out = np.full(topk_pools, -1, dtype=np.int32)
    if L <= 0:
        return tokens, pools_out
    n_full = L // B
    if n_full <= topk_pools:
        kept = list(range(n_full))
    else:
        a, e = forced_pools(n_full, init_pools, local_pools)
        forced = list(range(a)) + list(range(e, n_full))
        cand = np.arange(a, e)
        s = np.asarray(scores, dtype=np.float64)[: n_full * B].reshape(n_full, B)
        pool_max = s.max(axis=1) + 0.0                    # -0.0 -> +0.0
        order = np.lexsort((cand, -pool_max[cand]))       # by -score, then pool index
        chosen = cand[order[: topk_pools - len(forced)]]
        kept = sorted(forced + chosen.tolist())
    toks = [t for p in kept for t in range(p * B, p * B + B)] + list(range(n_full * B, L))
    tokens[: len(toks)] = toks
    pools_out[: len(kept)] = kept
    return tokens, pools_out
