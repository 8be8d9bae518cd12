"""Pins for the oracle's top-k selection (CPU only)."""

import numpy as np

from oracle import topk
from tests.conftest import load_golden


def _pairwise_rank_select(s, k):
    """Brute force: i is selected iff fewer than k elements beat it, where j
    beats i when s_j > s_i or (s_j == s_i and j < i)."""
    L = len(s)
    sel = []
    for i in range(L):
        beaten = sum(1 for j in range(L) if s[j] > s[i] or (s[j] == s[i] and j < i))
        if beaten < k:
            sel.append(i)
    return sel


def test_bruteforce_random_rows_with_ties():
    rng = np.random.default_rng(7)
    for _ in range(400):
        L = int(rng.integers(1, 40))
        k = int(rng.integers(1, 45))
        # few distinct values -> many ties; include signed zeros
        s = rng.choice(np.array([-2.0, -0.0, 0.0, 0.5, 1.0, 3.0]), size=L)
        got = topk.topk_row(s, L, k)
        if L <= k:
            exp = list(range(L)) + [-1] * (k - L)
        else:
            exp = _pairwise_rank_select(s, k)
        assert got.tolist() == exp


def test_signed_zero_tie_e2():
    g = load_golden("e2_signed_zero_tie.json")
    s = np.array(g["scores"])
    got = topk.topk_row(s, len(s), g["k"])
    assert got.tolist() == g["topk"]
    assert got.tolist() != g["wrong_if_minus_zero_lower"]


def test_e1_selection():
    g = load_golden("e1_fp8_two_heads.json")
    s = np.array(g["logits"])
    for k, exp in g["topk"].items():
        k = int(k)
        got = topk.topk_row(s, 4, k)
        assert got.tolist() == (exp + [-1] * (k - len(exp)))[:k]


def test_invariants():
    rng = np.random.default_rng(8)
    k = 16
    for L in (0, 1, k - 1, k, k + 1, 63, 64, 65, 300):
        s = rng.standard_normal(max(L, 1))
        got = topk.topk_row(s, L, k)
        valid = got[got >= 0]
        assert len(valid) == min(L, k)
        assert (valid < L).all()
        assert len(set(valid.tolist())) == len(valid)
        assert (np.diff(valid) > 0).all()                 # ascending
        assert (got[len(valid):] == -1).all()
        if L <= k:
            assert valid.tolist() == list(range(L))        # exact causal row
        else:
            # every selected score >= every unselected score
            mask = np.zeros(L, bool)
            mask[valid] = True
            assert s[:L][mask].min() >= s[:L][~mask].max()
