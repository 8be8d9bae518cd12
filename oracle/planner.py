"""Prefill chunk planner (oracle side).

The rules of ``split_indexer_prefill_chunks`` and
``build_prefill_chunk_metadata`` on the DeepSeek-V3.2 indexer page, stated
as properties of prefix sums rather than as a walk over the requests:

1. A chunk starting at request s ends at the largest e > s for which the
   requests [s, e) keep both N = sum(seq_lens[s:e]) <= workspace_size and
   M * N <= max_logits_bytes // 4 (M = sum(query_lens[s:e]); 4 bytes per
   fp32 logit).  Both sums only grow with e, so the requests that fit form a
   prefix of the remaining ones and e is found by bisection on the prefix
   sums.  (The page grows the chunk one request at a time and stops at the
   first one that does not fit: the same e.)
2. When not even request s alone fits, the chunk is that request alone.
3. The chunk's M query tokens are cut into slices of
   max(1, (max_logits_bytes // 4) // N) tokens, or one slice of all M when
   N == 0; no slice when M == 0.  A lone request whose N exceeds the element
   budget thus gets 1-token slices whose M * N breaks the budget -- kept, as
   the page does.
4. Per slice: total_seq_lens = N of the chunk (a chunk with N == 0 gives no
   record), token range = the chunk's first query token + the slice, and
   ``skip_kv_gather`` when the slice does not start at 0 (the keys were
   gathered for the chunk's first slice).

Token positions are relative to the first request passed in;
``request_offset`` only shifts the reported request indices.

Pins (tests/test_oracle_planner.py): hand-derived chunkings (the C5 split
into 16 chunks; 3-request, over-budget and zero-length cases); coverage
invariant: every (request, query token) appears exactly once, in order; a
brute-force check of rule 1 (the chosen end is the largest that fits).
"""

from __future__ import annotations

import numpy as np


def _fits(S, Q, s, e, workspace_size, elems):
    """Requests [s, e) within both budgets (prefix sums S, Q)."""
    n = S[e] - S[s]
    return n <= workspace_size and (Q[e] - Q[s]) * n <= elems


def _chunk_end(S, Q, s, n_req, workspace_size, elems):
    """Largest e in (s, n_req] with [s, e) within budget, or s + 1 when
    none is (rule 2)."""
    if not _fits(S, Q, s, s + 1, workspace_size, elems):
        return s + 1
    lo, hi = s + 1, n_req          # fits(lo) holds; find the last e that fits
    while lo < hi:
        mid = (lo + hi + 1) // 2
        if _fits(S, Q, s, mid, workspace_size, elems):
            lo = mid
        else:
            hi = mid - 1
    return lo


def split_chunks(seq_lens, query_lens, workspace_size: int, max_logits_bytes: int,
                 request_offset: int = 0):
    """List of (req_begin, req_end, q_begin, q_end) in planning order."""
    seq = np.asarray(seq_lens, dtype=np.int64).reshape(-1)
    ql = np.asarray(query_lens, dtype=np.int64).reshape(-1)
    S = [0] + np.cumsum(seq).tolist()
    Q = [0] + np.cumsum(ql).tolist()
    elems = max_logits_bytes // 4
    out = []
    s = 0
    while s < len(seq):
        e = _chunk_end(S, Q, s, len(seq), workspace_size, elems)
        N, M = S[e] - S[s], Q[e] - Q[s]
        width = max(1, elems // N) if N > 0 else M
        for a in range(0, M, max(width, 1)):
            out.append((s + request_offset, e + request_offset, a, min(a + width, M)))
        s = e
    return out


def chunk_records(seq_lens, query_lens, workspace_size: int, max_logits_bytes: int,
                  request_offset: int = 0):
    """Chunk records as dicts with the fields the library reports."""
    seq = np.asarray(seq_lens, dtype=np.int64).reshape(-1)
    ql = np.asarray(query_lens, dtype=np.int64).reshape(-1)
    qstart = np.concatenate([[0], np.cumsum(ql)])
    recs = []
    for rb, re, q0, q1 in split_chunks(seq, ql, workspace_size, max_logits_bytes, request_offset):
        b0, b1 = rb - request_offset, re - request_offset
        total = int(seq[b0:b1].sum())
        if total == 0:
            continue
        tok0 = int(qstart[b0])
        recs.append(dict(req_begin=rb, req_end=re, q_begin=q0, q_end=q1,
                         total_seq_lens=total, token_begin=tok0 + q0, token_end=tok0 + q1,
                         skip_kv_gather=int(q0 > 0)))
    return recs
