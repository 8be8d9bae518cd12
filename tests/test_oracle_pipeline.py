"""Pins for the whole-batch oracle (oracle/pipeline.py), CPU only.

The decode grid and the prefill chunk are worked by hand in
tests/golden/pipeline_decode_grid.json and pipeline_prefill_chunk.json (each
with its derivation): which q/w row a grid or chunk row reads, its key count,
its logits column base, its logits and its top-k.  The tests below also
plant the two mistakes a composition of correct parts could still make
(reading the grid row instead of the packed token; ignoring the chunk's query
slice) in a copy of the oracle and check that the goldens catch them.
"""

from types import SimpleNamespace

import numpy as np
import pytest

from oracle import pipeline, rows, topk
from tests.conftest import load_golden
from workloads.gen import _bf16_bits


def _cache_from_keys(g):
    """Pool [num_pages, 64 * row_bytes] poisoned with 0xFF, request b's keys
    at slots 0.. of page block_table[b][0]."""
    D = g["head_dim"]
    rb = D + 4
    pool = np.full((g["num_pages"], g["page_size"] * rb), 0xFF, dtype=np.uint8)
    for b, keys in enumerate(g["keys"]):
        page = g["block_table"][b][0]
        for t, (c0, c1, s) in enumerate(keys):
            row = np.zeros(rb, dtype=np.uint8)
            row[0], row[1] = c0, c1
            row[D:] = np.array([s], dtype="<f4").view(np.uint8)
            pool[page, t * rb : (t + 1) * rb] = row
    return pool, g["page_size"] * rb


def _q_bits(qrows, H, D):
    q = np.zeros((len(qrows), H, D), dtype=np.float32)
    for r, heads in enumerate(qrows):
        for h, v in enumerate(heads):
            q[r, h, : len(v)] = v
    return _bf16_bits(q)


def _decode_wl():
    g = load_golden("pipeline_decode_grid.json")
    pool, pb = _cache_from_keys(g)
    wl = SimpleNamespace(
        kind="decode", fmt="fp8", heads=g["heads"], head_dim=g["head_dim"], topk=g["topk"],
        page_size=g["page_size"], page_bytes=pb, cache=pool,
        block_table=np.asarray(g["block_table"], dtype=np.int32),
        seq_lens=np.asarray(g["seq_lens"], dtype=np.int32),
        decode_lens=np.asarray(g["decode_lens"], dtype=np.int32), next_n=g["next_n"], q_packed=True,
        q=_q_bits(g["packed_q"], g["heads"], g["head_dim"]),
        w=np.asarray(g["packed_w"], dtype=np.float32), compress_ratio=1)
    wl.num_req = len(g["seq_lens"])
    return g, wl


def _prefill_wl():
    g = load_golden("pipeline_prefill_chunk.json")
    pool, pb = _cache_from_keys(g)
    wl = SimpleNamespace(
        kind="prefill", fmt="fp8", heads=g["heads"], head_dim=g["head_dim"], topk=g["topk"],
        page_size=g["page_size"], page_bytes=pb, cache=pool,
        block_table=np.asarray(g["block_table"], dtype=np.int32),
        seq_lens=np.asarray(g["seq_lens"], dtype=np.int32),
        query_lens=np.asarray(g["query_lens"], dtype=np.int32),
        q=_q_bits(g["q"], g["heads"], g["head_dim"]), w=np.asarray(g["w"], dtype=np.float32),
        compress_ratio=1)
    return g, wl


def test_decode_grid_rows_and_query_rows():
    g, wl = _decode_wl()
    L, qrow = pipeline.decode_row_info(wl)
    assert L.tolist() == g["grid_lengths"]
    assert qrow.tolist() == g["grid_query_rows"]


def test_decode_grid_logits_and_topk():
    g, wl = _decode_wl()
    lg = pipeline.decode_logits(wl)
    assert sorted(lg) == list(range(len(g["grid_lengths"])))
    for r, exp in g["logits"].items():
        assert lg[int(r)].tolist() == exp, f"row {r}"
    out = pipeline.decode_topk(wl, lg)
    assert out.tolist() == g["topk_rows"]
    # one request at a time gives the same rows
    part = pipeline.decode_logits(wl, requests=[2])
    assert sorted(part) == [4, 5] and part[4].tolist() == g["logits"]["4"]


def test_decode_grid_catches_grid_row_queries():
    """Planted mistake: q/w read at the grid row b * next_n + i instead of
    the packed token.  The golden must reject it."""
    g, wl = _decode_wl()
    grid = rows.decode_query_rows(wl.decode_lens, wl.next_n, wl.num_req, packed=False)
    q = np.zeros((len(grid),) + wl.q.shape[1:], dtype=wl.q.dtype)
    w = np.zeros((len(grid), wl.heads), dtype=np.float32)
    n = min(len(grid), wl.q.shape[0])
    q[:n], w[:n] = wl.q[:n], wl.w[:n]          # packed rows seen as grid rows
    wrong = SimpleNamespace(**{**vars(wl), "q": q, "w": w, "q_packed": False})
    lg = pipeline.decode_logits(wrong)
    assert lg[4].tolist() != g["logits"]["4"]


def test_prefill_chunk_rows():
    g, wl = _prefill_wl()
    req, j, L, ks, qrow = pipeline.prefill_chunk_row_info(wl, g["chunk"])
    exp = g["rows"]
    assert req.tolist() == exp["req"]
    assert j.tolist() == exp["j"]
    assert L.tolist() == exp["L"]
    assert ks.tolist() == exp["ks"]
    assert qrow.tolist() == exp["qrow"]


def test_prefill_chunk_logits_and_topk():
    g, wl = _prefill_wl()
    lg = pipeline.prefill_chunk_logits(wl, g["chunk"])
    assert [lg[r].tolist() for r in range(3)] == g["logits"]
    _, _, L, _, _ = pipeline.prefill_chunk_row_info(wl, g["chunk"])
    got = [topk.topk_row(lg[r], int(L[r]), g["topk"]).tolist() for r in range(3)]
    assert got == g["topk_rows"]
    # a sample of rows gives the same values
    part = pipeline.prefill_chunk_logits(wl, g["chunk"], sample_rows=[2, 0])
    assert part[2].tolist() == g["logits"][2] and part[0].tolist() == g["logits"][0]


def test_prefill_chunk_catches_ignored_slice():
    """Planted mistake: the chunk's query slice start ignored (rows counted
    from the first token of the chunk)."""
    g, wl = _prefill_wl()
    rec = dict(g["chunk"], q_begin=0, q_end=3)
    req, j, L, ks, qrow = pipeline.prefill_chunk_row_info(wl, rec)
    assert j.tolist() != g["rows"]["j"] and qrow.tolist() != g["rows"]["qrow"]


def test_token_rows_by_hand():
    """token_rows of the MiniMax-M3 mono runner page, applied by hand: a
    request of q query tokens becomes q rows, token j seeing
    seq_len - (q - 1 - j) keys; q == 1 passes the lengths through."""
    assert rows.token_rows([5, 100], 3).tolist() == [3, 4, 5, 98, 99, 100]
    assert rows.token_rows([7, 1, 64], 1).tolist() == [7, 1, 64]
    assert rows.token_rows([9], 2).tolist() == [8, 9]
    # a full next_n = 3 grid is the same rows (every request has decode_len 3)
    assert rows.decode_lengths([5, 100], None, 3).tolist() == [3, 4, 5, 98, 99, 100]


@pytest.mark.parametrize("ratio", [2, 4])
def test_prefill_chunk_rows_compressed(ratio):
    """Compressed cache: the golden chunk's lengths and column bases divided
    by the ratio, rounded down (the chunk kernel's (start_pos + 1 + offset)
    // COMPRESS_RATIO, columns at the compressed prefix sum)."""
    g, wl = _prefill_wl()
    wl.compress_ratio = ratio
    _, _, L, ks, _ = pipeline.prefill_chunk_row_info(wl, g["chunk"])
    assert L.tolist() == [x // ratio for x in g["rows"]["L"]]
    assert ks.tolist() == [0, 0, 5 // ratio]


def test_decode_grid_pool_topk():
    """The pool selection of the hand-worked grid, pools of 2 keys, one
    place, no kept pools:
      (0,0) L 3 [1.5, 1, 0.5]: one complete pool -> pool 0, tail key 2
      (0,1) L 4 [0.5, -1, 0.5, 0.5]: maxima 0.5, 0.5 tie -> pool 0
      (1,0) L 3: one complete pool -> pool 0, tail key 2
      (1,1) padded -> nothing
      (2,0) L 4 [1, 2, 4, 3]: maxima 2, 4 -> pool 1
      (2,1) L 5 [1, -2, 0, 3, -1]: maxima 1, 3 -> pool 1, tail key 4"""
    g, wl = _decode_wl()
    toks, pools = pipeline.decode_pool_topk(wl, 2, 1, 0, 0)
    assert pools[:, 0].tolist() == [0, 0, 0, -1, 1, 1]
    assert toks.tolist() == [[0, 1, 2, -1], [0, 1, -1, -1], [0, 1, 2, -1], [-1, -1, -1, -1],
                             [2, 3, -1, -1], [2, 3, 4, -1]]
