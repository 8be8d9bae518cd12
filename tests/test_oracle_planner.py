"""Pins for the oracle's prefill chunk planner (CPU only)."""

import numpy as np

from oracle import planner
from tests.conftest import load_golden


def test_hand_cases():
    g = load_golden("planner_cases.json")
    fields = g["record_fields"]
    for c in g["cases"]:
        ch = planner.split_chunks(c["seq"], c["q"], c["workspace"], c["budget_bytes"])
        assert [list(x) for x in ch] == c["chunks"], c
        recs = planner.chunk_records(c["seq"], c["q"], c["workspace"], c["budget_bytes"])
        assert [[r[f] for f in fields] for r in recs] == c["records"], c


def test_c5_split_sixteen_chunks():
    # 2 requests, query 16384 of 65536 keys each; 65,536-token workspace,
    # 512 MiB of fp32 logits -> each request alone, 8 slices of 2048 rows
    recs = planner.chunk_records([65536, 65536], [16384, 16384], 65536, 512 << 20)
    assert len(recs) == 16
    for i, r in enumerate(recs):
        b = i // 8
        assert (r["req_begin"], r["req_end"]) == (b, b + 1)
        assert (r["q_begin"], r["q_end"]) == ((i % 8) * 2048, (i % 8 + 1) * 2048)
        assert r["total_seq_lens"] == 65536
        assert (r["q_end"] - r["q_begin"]) * r["total_seq_lens"] * 4 == 512 << 20
        assert r["skip_kv_gather"] == int(i % 8 != 0)
        assert r["token_begin"] == b * 16384 + (i % 8) * 2048


def test_request_offset_shifts_indices_only():
    a = planner.split_chunks([5, 9, 3], [2, 2, 2], 16, 400)
    b = planner.split_chunks([5, 9, 3], [2, 2, 2], 16, 400, request_offset=7)
    assert [(x[0] + 7, x[1] + 7, x[2], x[3]) for x in a] == b


def test_coverage_and_budget_random():
    rng = np.random.default_rng(9)
    for _ in range(300):
        n = int(rng.integers(1, 8))
        seq = rng.integers(0, 200, size=n)
        ql = np.minimum(rng.integers(0, 50, size=n), seq)
        ws = int(rng.integers(1, 400))
        budget = int(rng.integers(1, 20000))
        chunks = planner.split_chunks(seq, ql, ws, budget)
        # every (request, query token) covered exactly once, in order
        seen = []
        for rb, re, q0, q1 in chunks:
            toks = [(b, j) for b in range(rb, re) for j in range(int(ql[b]))]
            seen.extend(toks[q0:q1])
        assert seen == [(b, j) for b in range(n) for j in range(int(ql[b]))]
        # budgets hold unless a lone request is taken anyway
        for rb, re, q0, q1 in chunks:
            N = int(seq[rb:re].sum())
            if re - rb > 1:
                assert N <= ws
            if q1 - q0 > 1 or re - rb > 1:
                assert (q1 - q0) * N * 4 <= budget or N == 0


def test_chunk_end_is_largest_fitting_brute_force():
    """Rule 1 by enumeration: every chunk [s, e) of several requests fits
    both budgets and adding request e would break one; a one-request chunk
    either fits or no chunk starting there fits.  Slices cover the chunk's
    query tokens in pieces of max(1, budget/4 // N)."""
    rng = np.random.default_rng(21)
    for _ in range(400):
        n = int(rng.integers(1, 9))
        seq = rng.integers(0, 120, size=n)
        ql = np.minimum(rng.integers(0, 40, size=n), seq)
        ws = int(rng.integers(1, 300))
        budget = int(rng.integers(4, 40000))
        elems = budget // 4

        def fits(s, e):
            N = sum(int(x) for x in seq[s:e])
            M = sum(int(x) for x in ql[s:e])
            return N <= ws and M * N <= elems

        chunks = planner.split_chunks(seq, ql, ws, budget)
        # expected boundaries: from each start, the largest end that fits
        # (enumerating every end), else the lone request; chunks without
        # query tokens produce no slice
        expect = []
        s = 0
        while s < n:
            ends = [e for e in range(s + 1, n + 1) if fits(s, e)]
            e = max(ends) if ends else s + 1
            if sum(int(x) for x in ql[s:e]) > 0:
                expect.append((s, e))
            s = e
        got = []
        for rb, re, q0, q1 in chunks:
            if not got or got[-1] != (rb, re):
                got.append((rb, re))
        assert got == expect
        for rb, re, q0, q1 in chunks:
            N = sum(int(x) for x in seq[rb:re])
            M = sum(int(x) for x in ql[rb:re])
            width = max(1, elems // N) if N else M
            assert q0 % width == 0 and q1 == min(q0 + width, M)
