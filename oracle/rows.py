"""Query rows and their causal key counts (oracle side).

Decode.  A batch of ``B`` requests is laid out on a padded grid of
``B * next_n`` rows; row ``(b, i)`` is the ``i``-th decode token of request
``b``.  Request ``b`` has ``decode_lens[b]`` real tokens (all ``next_n`` when
``decode_lens`` is absent), left-aligned in its grid row block, and
``seq_lens[b]`` keys in the cache, its own decode tokens included.

Reading adopted for the per-row key count (the pages disagree on the one
real row of a short request):

    L(b, i) = seq_lens[b] - decode_lens[b] + i + 1   for i < decode_lens[b]
    L(b, i) = 0                                      for padded rows

i.e. "position + 1" of that token.  The glm5next ``sparse_indexer`` page
(``_decode_topk_seq_lens``) gives every real row pos + 1 and every padded row
0 ("empty tail"); the DeepSeek-V3.2 indexer page gives the same numbers in
its flattened variable-length path (the worked example in
``_prepare_decode_tensors``) and, for full requests, the same
``L - next_n + j + 1`` in its native 2-D path.  The two agree whenever
decode_lens[b] == next_n.  Negative values (seq_len < decode_len) are out of
contract and clamp to 0.

Packed queries: when the caller's q/w rows are the packed decode tokens in
request order, grid row (b, i) reads packed token ``offset_b + i`` where
``offset_b`` is the exclusive prefix sum of decode_lens (the per-token
(request id, intra index) pairs of ``_build_decode_scatter_indices`` on the
glm5next page, inverted) -- not ``b * next_n + i``.

Prefill.  Request ``b`` of a chunk has ``query_lens[b]`` query tokens, the
last ones of its ``seq_lens[b]`` keys; its query token ``j`` sees
``seq_lens[b] - query_lens[b] + j + 1`` keys (``_build_prefill_chunk_metadata_kernel``
on the DeepSeek-V3.2 page, compress ratio 1), stored in the chunk's logits
columns starting at ``ks = sum(seq_lens[:b])`` (its ``cu_seqlen_ks``).

Compressed index cache (the DeepSeek-V4 variant of the DeepSeek-V3.2
indexer page: compress_ratio > 1, pages of 256 compressed tokens).  The
cache stores seq_len // ratio keys per request, and every per-token length
above is divided by the ratio and rounded down: the page divides the decode
per-token lengths by the ratio (``seq_lens //= compress_ratio``) and its
prefill chunk kernel gives token ``offset`` the length
``(start_pos + 1 + offset) // COMPRESS_RATIO`` with ``start_pos = seq_len -
query_len``, its columns starting at the compressed prefix sum.

Pins: tests/test_oracle_rows.py (the pages' worked example
seq [10,7,12,0] / decode [3,1,4,0] -> [8,9,10,7,9,10,11,12]; ``token_rows``;
brute-force enumeration of the packed mapping).
"""

from __future__ import annotations

import numpy as np


def decode_lengths(seq_lens, decode_lens, next_n: int, compress_ratio: int = 1) -> np.ndarray:
    """Per grid row key counts, shape [B * next_n], int64 (with a compressed
    index cache, the token's length divided by the ratio, rounded down)."""
    seq = np.asarray(seq_lens, dtype=np.int64)
    B = seq.shape[0]
    dl = np.full(B, next_n, dtype=np.int64) if decode_lens is None else np.asarray(decode_lens, dtype=np.int64)
    out = np.zeros(B * next_n, dtype=np.int64)
    for b in range(B):
        for i in range(next_n):
            if i < dl[b]:
                out[b * next_n + i] = max(0, int(seq[b] - dl[b] + i + 1)) // compress_ratio
    return out


def decode_query_rows(decode_lens, next_n: int, num_req: int, packed: bool) -> np.ndarray:
    """For every grid row, the index of its q/w row, or -1 for padded rows."""
    dl = np.full(num_req, next_n, dtype=np.int64) if decode_lens is None else np.asarray(decode_lens, dtype=np.int64)
    out = np.full(num_req * next_n, -1, dtype=np.int64)
    offset = 0
    for b in range(num_req):
        for i in range(next_n):
            if i < dl[b]:
                out[b * next_n + i] = (offset + i) if packed else (b * next_n + i)
        offset += int(dl[b])
    return out


def flattened_token_lengths(seq_lens, decode_lens) -> np.ndarray:
    """Per real decode token, in packed order, its key count pos + 1 (the
    flattened variable-length expansion of the DeepSeek-V3.2 page)."""
    seq = np.asarray(seq_lens, dtype=np.int64)
    dl = np.asarray(decode_lens, dtype=np.int64)
    out = []
    for b in range(seq.shape[0]):
        for i in range(int(dl[b])):
            out.append(int(seq[b] - dl[b] + i + 1))
    return np.asarray(out, dtype=np.int64)


def token_rows(seq_lens, q: int) -> np.ndarray:
    """``token_rows`` of the MiniMax-M3 mono runner page: a request of q query
    tokens becomes q rows, token j seeing seq_len - (q - 1 - j) keys."""
    seq = np.asarray(seq_lens, dtype=np.int64)
    return np.asarray([int(s) - (q - 1 - j) for s in seq for j in range(q)], dtype=np.int64)


def prefill_rows(seq_lens, query_lens, req_begin: int, req_end: int, q_begin: int, q_end: int,
                 compress_ratio: int = 1):
    """Rows of one prefill chunk.

    The chunk covers requests [req_begin, req_end) and, of their concatenated
    query tokens, the slice [q_begin, q_end).  Returns, per output row in
    order, (request index, query index j within that request, key count L,
    logits column base ks) as int64 arrays.  With a compressed index cache
    (ratio r) the key count is (seq_len - query_len + j + 1) // r and ks sums
    the earlier requests' compressed lengths seq_len // r.
    """
    seq = np.asarray(seq_lens, dtype=np.int64)
    ql = np.asarray(query_lens, dtype=np.int64)
    reqs, js, Ls, kss = [], [], [], []
    tok = 0
    ks = 0
    for b in range(req_begin, req_end):
        for j in range(int(ql[b])):
            if q_begin <= tok < q_end:
                reqs.append(b)
                js.append(j)
                Ls.append(max(0, int(seq[b] - ql[b] + j + 1)) // compress_ratio)
                kss.append(ks)
            tok += 1
        ks += int(seq[b]) // compress_ratio
    return (np.asarray(reqs, dtype=np.int64), np.asarray(js, dtype=np.int64),
            np.asarray(Ls, dtype=np.int64), np.asarray(kss, dtype=np.int64))
