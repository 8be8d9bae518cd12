"""Pins for the oracle's row expansion (CPU only)."""

import numpy as np

from oracle import rows
from tests.conftest import load_golden


def test_pages_worked_example_flattened():
    g = load_golden("decode_expansion_worked_example.json")
    got = rows.flattened_token_lengths(g["seq_lens"], g["decode_lens"])
    assert got.tolist() == g["flattened_token_lengths"]
    # context lengths = seq_len - decode_len, as the comment states
    assert (np.array(g["seq_lens"]) - np.array(g["decode_lens"])).tolist() == g["context_lens"]


def test_grid_rows_e4():
    g = load_golden("e4_grid_rows.json")
    L = rows.decode_lengths(g["seq_lens"], g["decode_lens"], g["next_n"])
    assert L.tolist() == g["grid_lengths"]
    q = rows.decode_query_rows(g["decode_lens"], g["next_n"], len(g["seq_lens"]), packed=True)
    assert q.tolist() == g["packed_query_rows"]
    # the grid keeps every real token's flattened length, in order
    flat = rows.flattened_token_lengths(g["seq_lens"], g["decode_lens"])
    assert L[L > 0].tolist() == flat.tolist()


def test_uniform_grid_is_token_rows():
    """Full requests (decode_len == next_n): the grid lengths are the mono
    runner page's token_rows and the DeepSeek-V3.2 page's native 2-D
    lengths, written out by hand here (seq 5 and 100 at next_n 1, 2, 3)."""
    seq = [5, 100]
    hand = {1: [5, 100], 2: [4, 5, 99, 100], 3: [3, 4, 5, 98, 99, 100]}
    for q, exp in hand.items():
        assert rows.decode_lengths(seq, None, q).tolist() == exp
        assert rows.token_rows(seq, q).tolist() == exp


def test_packed_mapping_brute_force():
    rng = np.random.default_rng(3)
    for _ in range(50):
        B = int(rng.integers(1, 9))
        nn = int(rng.integers(1, 5))
        dl = rng.integers(0, nn + 1, size=B)
        q = rows.decode_query_rows(dl, nn, B, packed=True)
        # enumerate the packed tokens as (request id, intra index) pairs
        pairs = [(b, i) for b in range(B) for i in range(int(dl[b]))]
        for t, (b, i) in enumerate(pairs):
            assert q[b * nn + i] == t
        assert (q >= 0).sum() == len(pairs)
        qg = rows.decode_query_rows(dl, nn, B, packed=False)
        for b in range(B):
            for i in range(nn):
                assert qg[b * nn + i] == (b * nn + i if i < dl[b] else -1)


def test_prefill_rows_windows():
    seq = [6, 4]
    ql = [3, 2]
    req, j, L, ks = rows.prefill_rows(seq, ql, 0, 2, 0, 5)
    assert req.tolist() == [0, 0, 0, 1, 1]
    assert j.tolist() == [0, 1, 2, 0, 1]
    assert L.tolist() == [4, 5, 6, 3, 4]       # last query token sees every key
    assert ks.tolist() == [0, 0, 0, 6, 6]
    req, j, L, ks = rows.prefill_rows(seq, ql, 0, 2, 2, 4)
    assert req.tolist() == [0, 1] and L.tolist() == [6, 3] and ks.tolist() == [0, 6]


def test_compressed_lengths_hand_example():
    """The compressed index cache's lengths: the pages' division rules
    applied by hand (tests/golden/compressed_lengths.json)."""
    g = load_golden("compressed_lengths.json")
    r = g["compress_ratio"]
    d = g["decode"]
    L = rows.decode_lengths(d["seq_lens"], d["decode_lens"], d["next_n"], r)
    assert list(L) == d["grid_lengths"]
    p = g["prefill"]
    req, j, L, ks = rows.prefill_rows(p["seq_lens"], p["query_lens"], 0, 2, 0, 8, r)
    assert list(L) == p["lengths"] and list(ks) == p["ks"]
    # ratio 1 is the uncompressed rule
    assert list(rows.decode_lengths(d["seq_lens"], d["decode_lens"], d["next_n"], 1)) == \
        list(rows.decode_lengths(d["seq_lens"], d["decode_lens"], d["next_n"]))


def test_compressed_lengths_brute_force():
    """Every compressed length equals the count of stored keys at or before
    the token: key c stands for tokens [c r, c r + r), so it is visible to a
    token at position p once c r + r <= p + 1."""
    rng = np.random.default_rng(2)
    for r in (2, 4, 128):
        seq = rng.integers(0, 700, 20)
        dl = np.minimum(rng.integers(0, 4, 20), seq)
        L = rows.decode_lengths(seq, dl, 3, r)
        for b in range(20):
            for i in range(3):
                if i >= dl[b]:
                    assert L[b * 3 + i] == 0
                    continue
                pos = int(seq[b] - dl[b] + i)
                assert L[b * 3 + i] == sum(1 for c in range(int(seq[b]) // r) if c * r + r <= pos + 1)
