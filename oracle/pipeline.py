"""Whole-batch oracle: per-row logits and top-k for decode grids and prefill
chunks, composed from the row, cache, score and top-k definitions.

Keys are read once per request; each row scores keys [0, L_row) of its
request.  Row order is the padded decode grid (decode) or the chunk's query
slice (prefill).
"""

from __future__ import annotations

import numpy as np

from . import cache, pool, rows, score, topk


def decode_row_info(wl):
    """(L per grid row, q/w row per grid row or -1)."""
    L = rows.decode_lengths(wl.seq_lens, wl.decode_lens, wl.next_n, getattr(wl, "compress_ratio", 1))
    qrow = rows.decode_query_rows(wl.decode_lens, wl.next_n, wl.num_req, wl.q_packed)
    return L, qrow


def decode_logits(wl, requests=None):
    """Dict grid_row -> float64 logits [L_row] for the requested requests
    (all by default).  Padded rows map to empty arrays."""
    L, qrow = decode_row_info(wl)
    out = {}
    reqs = range(wl.num_req) if requests is None else requests
    for b in reqs:
        r0 = b * wl.next_n
        Lmax = int(L[r0 : r0 + wl.next_n].max(initial=0))
        kb = cache.keys(wl, b, Lmax) if Lmax > 0 else None
        for i in range(wl.next_n):
            r = r0 + i
            if L[r] == 0:
                out[r] = np.zeros(0)
                continue
            out[r] = score.logits(wl.q[qrow[r]], wl.w[qrow[r]], kb[: L[r]])
    return out


def decode_topk(wl, logits_by_row=None, requests=None):
    """int32 [grid_rows, k] top-k of every grid row (or the requested
    requests' rows; other rows stay -1)."""
    L, _ = decode_row_info(wl)
    if logits_by_row is None:
        logits_by_row = decode_logits(wl, requests)
    out = np.full((wl.num_req * wl.next_n, wl.topk), -1, dtype=np.int32)
    for r, lg in logits_by_row.items():
        out[r] = topk.topk_row(lg, int(L[r]), wl.topk)
    return out


def decode_pool_topk(wl, pool_size, topk_pools, init_pools, local_pools, logits_by_row=None, requests=None):
    """Pool-level selection of every grid row (or the requested requests'
    rows; other rows stay -1): (tokens int32 [grid_rows, (topk_pools + 1)
    * pool_size], pools int32 [grid_rows, topk_pools])."""
    L, _ = decode_row_info(wl)
    if logits_by_row is None:
        logits_by_row = decode_logits(wl, requests)
    R = wl.num_req * wl.next_n
    toks = np.full((R, (topk_pools + 1) * pool_size), -1, dtype=np.int32)
    pools = np.full((R, topk_pools), -1, dtype=np.int32)
    for r, lg in logits_by_row.items():
        toks[r], pools[r] = pool.pool_topk_row(lg, int(L[r]), pool_size, topk_pools, init_pools, local_pools)
    return toks, pools


def prefill_chunk_row_info(wl, rec):
    """Rows of one chunk record: (request, j, L, ks, q/w row)."""
    req, j, L, ks = rows.prefill_rows(wl.seq_lens, wl.query_lens, rec["req_begin"],
                                      rec["req_end"], rec["q_begin"], rec["q_end"],
                                      getattr(wl, "compress_ratio", 1))
    qstart = np.concatenate([[0], np.cumsum(np.asarray(wl.query_lens, dtype=np.int64))])
    qrow = qstart[req] + j
    return req, j, L, ks, qrow


def prefill_chunk_logits(wl, rec, sample_rows=None):
    """Dict chunk_row -> float64 logits [L] for a chunk (or a sample of its
    rows)."""
    req, j, L, ks, qrow = prefill_chunk_row_info(wl, rec)
    idx = range(len(req)) if sample_rows is None else sample_rows
    key_cache = {}
    out = {}
    for r in idx:
        b = int(req[r])
        if b not in key_cache:
            key_cache = {b: cache.keys(wl, b, int(wl.seq_lens[b]) // getattr(wl, "compress_ratio", 1))}
        out[r] = score.logits(wl.q[qrow[r]], wl.w[qrow[r]], key_cache[b][: L[r]])
    return out
