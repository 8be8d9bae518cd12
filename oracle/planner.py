"""Prefill chunk planner (oracle side).

Restates, in the order the DeepSeek-V3.2 indexer page gives them, the rules
of ``split_indexer_prefill_chunks`` and ``build_prefill_chunk_metadata``:

1. Walk the requests in order, greedily growing a chunk while both
   N = sum(seq_lens) <= workspace_size and M * N <= max_logits_bytes // 4
   (M = sum(query_lens)); the 4 is the fp32 logit size.
2. If not even the first request fits, take that one request alone anyway.
3. Split the chunk's M query tokens into slices of
   max_q = max(1, (max_logits_bytes // 4) // N) tokens (one slice of all M
   when N == 0).  A single request whose N exceeds the element budget thus
   still gets 1-token slices whose M * N is over budget -- reproduced as is.
4. Per slice: total_seq_lens = N of the chunk (a chunk with N == 0 produces
   no record), token range = the chunk's first query token + the slice, and
   ``skip_kv_gather`` when the slice does not start at 0 (the keys were
   already gathered for the chunk's first slice).

Token positions are relative to the first request passed in;
``request_offset`` only shifts the reported request indices.

Pins (tests/test_oracle_planner.py): hand-derived chunkings (the C5 split
into 16 chunks; 3-request, over-budget and zero-length cases); coverage
invariant: every (request, query token) appears exactly once, in order.
"""

from __future__ import annotations

import numpy as np


def split_chunks(seq_lens, query_lens, workspace_size: int, max_logits_bytes: int,
                 request_offset: int = 0):
    """List of (req_begin, req_end, q_begin, q_end) in planning order."""
    seq = [int(x) for x in np.asarray(seq_lens).reshape(-1)]
    ql = [int(x) for x in np.asarray(query_lens).reshape(-1)]
    n = len(seq)
    elems = max_logits_bytes // 4
    chunks = []
    end = 0
    while end < n:
        start, m, nn = end, 0, 0
        while end < n:
            new_m, new_n = m + ql[end], nn + seq[end]
            if new_n <= workspace_size and new_m * new_n <= elems:
                m, nn = new_m, new_n
                end += 1
            else:
                break
        if end == start:
            m, nn = ql[end], seq[end]
            end += 1
        max_q = max(1, elems // nn) if nn > 0 else m
        q0 = 0
        while q0 < m:
            sub = min(max_q, m - q0)
            chunks.append((start + request_offset, end + request_offset, q0, q0 + sub))
            q0 += sub
    return chunks


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
