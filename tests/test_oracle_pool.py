"""Pins for the oracle's pool-level selection (oracle/pool.py), CPU only."""

import numpy as np

from oracle import pool, topk
from tests.conftest import load_golden


def test_hand_worked_cases():
    g = load_golden("pool_topk.json")
    for c in g["cases"]:
        row = np.asarray(g["rows"][c["row"]], dtype=np.float64)
        toks, pools = pool.pool_topk_row(row, c["L"], c["B"], c["topk"], c["init"], c["local"])
        assert toks.tolist() == c["tokens"], c["name"]
        assert pools.tolist() == c["pools"], c["name"]


def test_pool_size_one_is_token_topk():
    """Pools of one key and nothing kept by position: the token top-k (the
    tie rule and the causal fill included)."""
    rng = np.random.default_rng(4)
    for _ in range(200):
        L = int(rng.integers(0, 40))
        k = int(rng.integers(1, 12))
        s = (rng.integers(-3, 4, size=L) * 0.5).astype(np.float64)
        s[rng.random(L) < 0.2] = -0.0
        toks, pools = pool.pool_topk_row(s, L, 1, k, 0, 0)
        exp = topk.topk_row(s, L, k)
        n = min(L, k)
        assert toks[:n].tolist() == exp[:n].tolist()
        assert (toks[n:] == -1).all() and pools[:n].tolist() == exp[:n].tolist()


def _brute(scores, L, B, k, init, local):
    """Kept pools by the definition: kept by position, else selected iff
    fewer than the free places' worth of candidates beat it (a higher
    score, or the same score at a lower index)."""
    n = L // B
    if n <= k:
        return list(range(n))
    a = min(init, n)
    z = min(local, n - a)
    forced = set(range(a)) | set(range(n - z, n))
    free = k - len(forced)
    m = {p: max(float(x) for x in scores[p * B:(p + 1) * B]) + 0.0 for p in range(n)}
    cand = [p for p in range(n) if p not in forced]
    chosen = [p for p in cand
              if sum(1 for q in cand if m[q] > m[p] or (m[q] == m[p] and q < p)) < free]
    return sorted(forced | set(chosen))


def test_brute_force_random_rows():
    rng = np.random.default_rng(8)
    for _ in range(400):
        B = int(rng.choice([1, 2, 3, 4, 8]))
        L = int(rng.integers(0, 60))
        k = int(rng.integers(1, 8))
        init = int(rng.integers(0, k + 1))
        local = int(rng.integers(0, k - init + 1))
        s = (rng.integers(-4, 5, size=L) * 0.25).astype(np.float64)
        s[rng.random(L) < 0.15] = -0.0
        toks, pools = pool.pool_topk_row(s, L, B, k, init, local)
        kept = _brute(s, L, B, k, init, local)
        assert pools[: len(kept)].tolist() == kept and (pools[len(kept):] == -1).all()
        exp = [t for p in kept for t in range(p * B, p * B + B)] + list(range((L // B) * B, L))
        assert toks[: len(exp)].tolist() == exp and (toks[len(exp):] == -1).all()


def test_invariants():
    rng = np.random.default_rng(12)
    for _ in range(200):
        B = int(rng.choice([4, 16, 64]))
        L = int(rng.integers(0, 3000))
        k = int(rng.integers(1, 20))
        init, local = int(rng.integers(0, 3)), int(rng.integers(0, 3))
        if init + local > k:
            continue
        s = rng.standard_normal(L)
        toks, pools = pool.pool_topk_row(s, L, B, k, init, local)
        v = toks[toks >= 0]
        assert (toks[len(v):] == -1).all()
        assert (np.diff(v) > 0).all() and (v < max(L, 1)).all()
        n = L // B
        kept = pools[pools >= 0]
        assert len(kept) == min(n, k)
        assert len(v) == len(kept) * B + (L - n * B)
        assert set(range(n * B, L)) <= set(v.tolist())                   # the tail
        if n > k:
            assert set(range(min(init, n))) <= set(kept.tolist())         # kept first pools
            assert set(range(n - min(local, n - min(init, n)), n)) <= set(kept.tolist())
        else:
            assert v.tolist() == list(range(L))                          # every key
